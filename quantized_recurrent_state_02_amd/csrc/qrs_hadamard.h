// qrs_hadamard.h -- device helpers of the first revision's low tier (DAMP
// arXiv HTML, section 3.2 Eq.(3); Appendix A.1 and Table 3
// "INT8+Hadamard"; Appendix A.5 Eq.(17)): each 32-value group of an INT8-tier
// row is taken through the normalized block-32 Hadamard transform and stored
// as asymmetric UINT8 codes with an FP16 scale and zero point.  Internal to
// the library.
//
// Thread mapping (the decode and codec kernels, and the prefill kernel's
// chunk-end pass): a group's 32 values sit on a lane pair, 16 on the even
// lane (positions 0..15) and 16 on the odd lane (16..31).  Sylvester's
// H_32 = H_2 (x) H_16, so each lane applies H_16 to its 16 values in
// registers and the pair finishes with one butterfly across the lanes, after
// which each lane holds its own 16 output positions.  The prefill kernel's
// read of the stored state uses a second mapping, a group on the 16 lanes of
// a DPP row with two values per lane (hadamard32_row).
//
// Precision: every butterfly runs in FP64 on FP32 inputs, so the sums are
// exact whenever the group's nonzero magnitudes span less than 2^24 (29 + 24
// bits fit in 53), and then equal the sums of the matrix definition in any
// order; the result is multiplied by RN64(2^-2.5) and rounded once to FP32.
// Metadata per group: one 32-bit word, FP16 scale in bits 0..15 and FP16
// zero point in bits 16..31 (4 bytes, the size of the INT8 tier's FP32
// scale, so the unit keeps its 20,224 bytes and offsets).
#pragma once

#include "qrs_internal.h"

namespace qrs {

// RN64(2^-2.5), the correctly rounded 1/sqrt(32).
constexpr double kInvSqrt32 = 0x1.6a09e667f3bcdp-3;

// An FP64 value moved across lanes by one DPP control (both halves).
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v) {
    const uint64_t b = __builtin_bit_cast(uint64_t, v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)b, CTRL, 0xF, 0xF, true);
    const uint32_t hi =
        (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)(b >> 32), CTRL, 0xF, 0xF, true);
    return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

// FP64 value of the partner lane tid ^ 1 (DPP quad_perm [1,0,3,2]).
__device__ __forceinline__ double partner_f64(double v) { return dpp_f64<0xB1>(v); }

// In place: x (this lane's 16 values of a group) -> this lane's 16 outputs of
// the normalized block-32 transform.  odd = lane parity within the pair.
__device__ __forceinline__ void hadamard32_pair(float (&x)[16], bool odd) {
    double a[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) a[i] = (double)x[i];
#pragma unroll
    for (int h = 1; h < 16; h <<= 1)
#pragma unroll
        for (int i = 0; i < 16; i += 2 * h)
#pragma unroll
            for (int j = i; j < i + h; ++j) {
                const double u = a[j], v = a[j + h];
                a[j] = u + v;
                a[j + h] = u - v;
            }
    // even lane: u0 + u1 (outputs 0..15); odd lane: u0 - u1 (outputs 16..31),
    // both as p + sgn a with sgn = +-1: one fma, exact in the product, rounded
    // once like the add or subtract (a per-lane select cost two more
    // instructions per value)
    const double sgn = odd ? -1.0 : 1.0;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const double p = partner_f64(a[i]);
        const double y = __builtin_fma(a[i], sgn, p);
        x[i] = (float)(y * kInvSqrt32);
    }
}

// FP64 value of lane l16 ^ (1 << M) of the same 16-lane DPP row (both halves
// moved).  Bits 0, 1 and 3 are single DPP exchanges (quad_perm [1,0,3,2],
// [2,3,0,1], row_ror:8); bit 2 takes the rotation by 4 (from lane l16 - 4) on
// lanes with the bit set and by 12 (from lane l16 + 4) on the others.
template <int M>
__device__ __forceinline__ double row_partner_f64(double v, int l16) {
    if (M == 0) return dpp_f64<0xB1>(v);
    if (M == 1) return dpp_f64<0x4E>(v);
    if (M == 3) return dpp_f64<0x128>(v);
    const double a = dpp_f64<0x124>(v), b = dpp_f64<0x12C>(v);
    return (l16 & 4) ? a : b;
}

// The normalized block-32 transform for a group held by the 16 lanes of a
// DPP row with two values per lane (the prefill kernel's accumulator
// layout): x0 is group position l16, x1 position 16 + l16.  H_32 = H_2 (x)
// H_16: H_2 between the two registers, then H_16 over the lane bits, all in
// FP64; the result is multiplied by RN64(2^-2.5) and rounded once.
__device__ __forceinline__ void hadamard32_row(float &x0, float &x1, int l16) {
    double u = (double)x0 + (double)x1, w = (double)x0 - (double)x1;
#define QRS_BFLY(M)                                                        \
    {                                                                      \
        const double pu = row_partner_f64<M>(u, l16), pw = row_partner_f64<M>(w, l16); \
        const double sg = ((l16 >> (M)) & 1) ? -1.0 : 1.0;                 \
        u = __builtin_fma(u, sg, pu);                                      \
        w = __builtin_fma(w, sg, pw);                                      \
    }
    QRS_BFLY(0)
    QRS_BFLY(1)
    QRS_BFLY(2)
    QRS_BFLY(3)
#undef QRS_BFLY
    x0 = (float)(u * kInvSqrt32);
    x1 = (float)(w * kInvSqrt32);
}

__device__ __forceinline__ float pair_minf(float a) {
    const float p = __builtin_bit_cast(
        float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, a), 0xB1, 0xF, 0xF, true));
    return fminf(a, p);
}
__device__ __forceinline__ float pair_maxf(float a) {
    const float p = __builtin_bit_cast(
        float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, a), 0xB1, 0xF, 0xF, true));
    return fmaxf(a, p);
}

// Parameters of one group from its transformed values (Eq.(3), b = 8):
// s = RN32((max - min) / 255) stored as FP16 (nearest even); z =
// round(-min / s16) stored as FP16; both used as stored.  lo / hi: this
// lane's extremes, combined across the pair here.  A zero stored scale
// (constant group, or below the FP16 range) gives rinv = 0, hence z = 0 and
// every code 0.
struct U8Params {
    float sh;      // FP16 scale as FP32
    float zh;      // FP16 zero point as FP32
    double rinv;   // FP64 reciprocal of sh (0 when sh = 0)
    uint32_t meta; // s16 | z16 << 16
};

__device__ __forceinline__ U8Params u8_params(float lo, float hi) {
    lo = pair_minf(lo);
    hi = pair_maxf(hi);
    const float d = hi - lo;
    const float s = (float)((double)d * (1.0 / 255.0));  // RN32(d / 255), as in group_scale
    const uint32_t s16 = f32_to_f16_bits(s);
    U8Params p;
    p.sh = f16_bits_to_f32(s16);
    p.rinv = scale_reciprocal(p.sh);
    const float z = rintf(quant_quotient(-lo, p.rinv));
    const uint32_t z16 = p.sh == 0.0f ? 0u : f32_to_f16_bits(z);
    p.zh = f16_bits_to_f32(z16);
    p.meta = s16 | (z16 << 16);
    return p;
}

// Code of one transformed value: round(y / s16) + z16, saturated to [0, 255],
// returned as an FP32 integer value.
__device__ __forceinline__ float u8_code(float y, const U8Params &p) {
    const float c = rintf(quant_quotient(y, p.rinv)) + p.zh;
    return __builtin_amdgcn_fmed3f(c, 0.0f, 255.0f);
}

// Four codes (FP32 integers in [0, 255]) packed little-endian.
__device__ __forceinline__ uint32_t pack4_u8(float c0, float c1, float c2, float c3) {
    return pack4_codes(c0, c1, c2, c3);
}

// Reconstruction in the transformed domain: RN32(s16 * (code - z16)).
__device__ __forceinline__ float u8_dequant(uint32_t w, int byte, float sh, float zh) {
    const float code = (float)((w >> (8 * byte)) & 0xffu);
    return sh * (code - zh);
}

}  // namespace qrs
