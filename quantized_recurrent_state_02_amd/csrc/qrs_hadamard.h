// qrs_hadamard.h -- device helpers of the first revision's low tier (DAMP
// arXiv HTML, section 3.2 Eq.(3); Appendix A.1 and Table 3
// "INT8+Hadamard"; Appendix A.5 Eq.(17)): each 32-value group of an INT8-tier
// row is taken through the normalized block-32 Hadamard transform and stored
// as asymmetric UINT8 codes with an FP16 scale and zero point.  Internal to
// the library.
//
// Thread mapping (the decode / codec kernels): a group's 32 values sit on a
// lane pair, 16 on the even lane (positions 0..15) and 16 on the odd lane
// (16..31).  Sylvester's H_32 = H_2 (x) H_16, so each lane applies H_16 to its
// 16 values in registers and the pair finishes with one butterfly across the
// lanes, after which each lane holds its own 16 output positions.
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

// FP64 value of the partner lane tid ^ 1 (DPP quad_perm [1,0,3,2] on both halves).
__device__ __forceinline__ double partner_f64(double v) {
    const uint64_t b = __builtin_bit_cast(uint64_t, v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)b, 0xB1, 0xF, 0xF, true);
    const uint32_t hi =
        (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)(b >> 32), 0xB1, 0xF, 0xF, true);
    return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

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
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const double p = partner_f64(a[i]);
        // even lane: u0 + u1 (outputs 0..15); odd lane: u0 - u1 (outputs 16..31)
        const double y = odd ? p - a[i] : a[i] + p;
        x[i] = (float)(y * kInvSqrt32);
    }
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
