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

// ---- the inverse transform of a stored group from its codes ----
//
// A stored group reconstructs as y_i = RN32(s16 (q_i - z16)) (Eq.(3)) and
// transforms back as RN32(RN64(2^-2.5) * sum_j H[i][j] y_j) with the sums in
// FP64.  When 0 < s16 <= 65504 and -7936 <= z16 <= 8191, every |q_i - z16| is
// below 2^13, so with the 11 significant bits of s16 each y_i is an exact
// FP32 product s16 m_i, every partial sum is s16 times an integer below 2^18
// (exact in FP64, in any order), and the sum is s16 (H q)_i - 32 z16 s16
// [i = 0] (only the first row of H has a nonzero sum).  H q, with |(H q)_i|
// <= 32 * 255, is computed on packed 16-bit integers; for i != 0, t =
// s16 (H q)_i is again an exact FP32 product, and RN32(RN64(c t)) for c =
// RN64(2^-2.5) equals fma(t, c_hi, RN32(t c_lo)) with c_hi = RN32(c), c_lo =
// RN32(c - c_hi) for every FP32 t whose products stay normal (an exhaustive
// check over all 2^23 significands; the test suite repeats it); the output
// with the z16 term takes the FP64 path.  Same bits as hadamard32_pair on
// the reconstruction, in about 8 instead of 13 VALU instructions per value.
// A zero scale takes the FP64 path (there a negative integer sum would give
// -0 for the +0 of the definition).

// A stored group (FP16 s16, z16 as FP32) inside the exact range above.
__device__ __forceinline__ bool u8_group_exact(float sh, float zh) {
    return sh > 0.0f && sh <= 65504.0f && zh >= -7936.0f && zh <= 8191.0f;
}

typedef short s16x2 __attribute__((ext_vector_type(2)));

// RN64(2^-2.5) as an unevaluated FP32 sum.
constexpr float kInvSqrt32Hi = 0x1.6a09e6p-3f;
constexpr float kInvSqrt32Lo = 0x1.9fcef4p-29f;

// x (this lane's 16 outputs, positions 16 odd .. + 15 of the group) from the
// lane's 16 codes (bytes of lw, position c in byte c & 3 of lw[c >> 2]) and
// the group's s16, z16, for a group with u8_group_exact(sh, zh).  Register
// P[j] holds positions j (low half) and j + 8 (high half).
__device__ __forceinline__ void hadamard32_pair_codes(const uint32_t (&lw)[4], float sh, float zh,
                                                      bool odd, float (&x)[16]) {
    s16x2 P[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)  // bytes j and j + 8, zero-extended to 16 bits
        P[j] = __builtin_bit_cast(
            s16x2, __builtin_amdgcn_perm(lw[(j >> 2) + 2], lw[j >> 2],
                                         0x0C040C00u + (uint32_t)(j & 3) * 0x00010001u));
    // H_16 in the lane: position bits 0..2 across registers, bit 3 across halves
#pragma unroll
    for (int h = 1; h < 8; h <<= 1)
#pragma unroll
        for (int j = 0; j < 8; ++j)
            if ((j & h) == 0) {
                const s16x2 u = P[j], v = P[j + h];
                P[j] = u + v;
                P[j + h] = u - v;
            }
    const s16x2 pm = {1, -1};
#pragma unroll
    for (int j = 0; j < 8; ++j) P[j] = P[j].xx + P[j].yy * pm;
    // H_2 across the lane pair: even lane u0 + u1, odd lane u0 - u1.  The
    // sign is opaque to the compiler, so the product stays one packed
    // multiply-add instead of a negate, a select and an add.
    uint32_t sgw = odd ? 0xffffffffu : 0x00010001u;
    asm volatile("" : "+v"(sgw));
    const s16x2 sg = __builtin_bit_cast(s16x2, sgw);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const s16x2 p = __builtin_bit_cast(
            s16x2, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, P[j]), 0xB1, 0xF, 0xF, true));
        P[j] = P[j] * sg + p;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        if (j > 0) {
            const float t = sh * (float)(int)P[j].x;
            x[j] = __builtin_fmaf(t, kInvSqrt32Hi, t * kInvSqrt32Lo);
        }
        const float t2 = sh * (float)(int)P[j].y;
        x[j + 8] = __builtin_fmaf(t2, kInvSqrt32Hi, t2 * kInvSqrt32Lo);
    }
    // position 0 of the group (even lane) carries -32 z16
    const int m0 = (int)P[0].x - (odd ? 0 : 32 * (int)zh);
    x[0] = (float)(((double)sh * (double)m0) * kInvSqrt32);
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
    // converted on every lane, then selected (no branch around it)
    uint32_t z16 = f32_to_f16_bits(z);
    asm volatile("" : "+v"(z16));
    z16 = p.sh == 0.0f ? 0u : z16;
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

// The codes of four transformed values, packed little-endian: u8_code's
// round(y / s16) + z16, saturated by v_cvt_pk_u8_f32, which converts to an
// unsigned byte with saturation to [0, 255] (NaN to 0; its input here is an
// integer, so its rounding never applies) and writes the byte in place: one
// instruction in place of the clamp and the packing step.
__device__ __forceinline__ uint32_t u8_pack4(float y0, float y1, float y2, float y3,
                                             const U8Params &p) {
    uint32_t d = __builtin_amdgcn_cvt_pk_u8_f32(rintf(quant_quotient(y0, p.rinv)) + p.zh, 0u, 0u);
    d = __builtin_amdgcn_cvt_pk_u8_f32(rintf(quant_quotient(y1, p.rinv)) + p.zh, 1u, d);
    d = __builtin_amdgcn_cvt_pk_u8_f32(rintf(quant_quotient(y2, p.rinv)) + p.zh, 2u, d);
    return __builtin_amdgcn_cvt_pk_u8_f32(rintf(quant_quotient(y3, p.rinv)) + p.zh, 3u, d);
}

// Reconstruction in the transformed domain: RN32(s16 * (code - z16)).
__device__ __forceinline__ float u8_dequant(uint32_t w, int byte, float sh, float zh) {
    const float code = (float)((w >> (8 * byte)) & 0xffu);
    return sh * (code - zh);
}

}  // namespace qrs
