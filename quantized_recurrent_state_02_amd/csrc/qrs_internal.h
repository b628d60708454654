// qrs_internal.h -- shapes, packed layout and device-side codec helpers of
// libqrs (gfx950).  Internal to the library.
//
// Thread mapping shared by the per-unit kernels: one 128-thread workgroup
// (two wave64s) owns one (slot, head) unit of 128x128 values.
//   cb = tid & 7   column block: columns [16 cb, 16 cb + 16)
//   rg = tid >> 3  row group 0..15: stored rows rg + 16 r, r = 0..7
// Row r = 0 of every thread is an FP16 row (stored rows 0..15), rows r >= 1
// are INT8 rows, so the FP16/INT8 split is uniform across all lanes.  The
// 32-value scale group of a thread is g = cb >> 1; its partner lane
// (tid ^ 1) holds the other 16 values of the group.  A wave's load of one
// INT8 row-slot covers 8 consecutive rows = 1 KiB contiguous.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qrs {

constexpr int DK = 128;
constexpr int DV = 128;
constexpr int KHI = 16;
constexpr int KLO = DK - KHI;
constexpr int GRP = 32;
constexpr int NGRP = DV / GRP;

constexpr int HI_OFF = 0;
constexpr int LO_OFF = KHI * DV * 2;                 // 4096
constexpr int SC_OFF = LO_OFF + KLO * DV;            // 18432
constexpr int UNIT_BYTES = SC_OFF + KLO * NGRP * 4;  // 20224
constexpr int F32_UNIT_BYTES = DK * DV * 4;          // 65536
static_assert(UNIT_BYTES == 20224, "packed unit size");
static_assert(UNIT_BYTES % 256 == 0, "units stay 256-byte aligned");

constexpr int THREADS = 128;
constexpr int ROWS_PER_THREAD = 8;   // rg + 16 r
constexpr int COLS_PER_THREAD = 16;  // 16 cb .. 16 cb + 15

// Plain host-side description of a pool, passed by value to kernels.
struct PoolView {
    uint8_t *base;          // unit 0
    const int32_t *perm;    // [H][128]
    const float *smooth;    // [H][128]
    int num_slots;
    int num_heads;
};

__device__ __forceinline__ float f16_bits_to_f32(uint32_t h) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

// IEEE binary16 round-to-nearest-even (v_cvt_f16_f32 in the default mode) of
// an FP32 value.  The empty asm pins x as a rounded FP32 register value:
// without it the compiler folds a preceding FP32 fma into v_fma_mix*_f16,
// which rounds the exact product-sum straight to FP16 (one rounding instead
// of FP32 then FP16) and so changes some results.
__device__ __forceinline__ uint32_t f32_to_f16_bits(float x) {
    asm volatile("" : "+v"(x));
    return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)x);
}

// max(a, a of the partner lane tid ^ 1) for a >= 0 (a group maximum of
// absolute values): non-negative IEEE floats order like their bit patterns,
// so one v_max_u32 with a DPP quad_perm [1,0,3,2] source does it.  The
// s_nop gives the two wait states a DPP read needs after a VALU write of its
// source register.
__device__ __forceinline__ float pair_max(float a) {
    uint32_t d;
    asm("s_nop 1\n\tv_max_u32_dpp %0, %1, %1 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf "
        "bound_ctrl:1"
        : "=v"(d)
        : "v"(__builtin_bit_cast(uint32_t, a)));
    return __builtin_bit_cast(float, d);
}

// v from the lane that the DPP control CTRL names (all controls used here
// name lanes inside the same 16-lane row, so every source lane exists).
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
    return __builtin_bit_cast(
        float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xf, 0xf, false));
}

// Sum over the 16 lanes of each DPP row (lanes 16 r .. 16 r + 15), in every
// lane of the row: quad_perm [1,0,3,2] and [2,3,0,1], then the half-row and
// row mirrors.  Each step adds a lane and its partner in both orders, so by
// commutativity all lanes of a row hold the same bits.
__device__ __forceinline__ float row16_sum(float x) {
    x += dpp_f<0xb1>(x);
    x += dpp_f<0x4e>(x);
    x += dpp_f<0x141>(x);
    x += dpp_f<0x140>(x);
    return x;
}

// The same reduction for a maximum.
__device__ __forceinline__ float row16_max(float x) {
    x = fmaxf(x, dpp_f<0xb1>(x));
    x = fmaxf(x, dpp_f<0x4e>(x));
    x = fmaxf(x, dpp_f<0x141>(x));
    x = fmaxf(x, dpp_f<0x140>(x));
    return x;
}

// Sum over the 64 lanes of a wave, the same value in every lane: the row
// sums, then the four rows' sums read through scalar registers.  (A
// butterfly of shuffles takes six LDS-unit permutes, each with the latency
// of an LDS access.)
__device__ __forceinline__ float wave_allsum(float x) {
    x = row16_sum(x);
    const int xi = __builtin_bit_cast(int, x);
    const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(xi, 0));
    const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(xi, 16));
    const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(xi, 32));
    const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(xi, 48));
    return (r0 + r1) + (r2 + r3);
}

// Scale of a group: RN32(amax / 127).  Evaluated as RN32(RN64(amax * RN64(1/127))):
// the FP64 product is within 2^-52 relative of amax/127, while a quotient of
// two FP32 numbers is never within 2^-49 relative of an FP32 rounding
// midpoint, so the final FP32 rounding equals that of the exact quotient.
__device__ __forceinline__ float group_scale(float amax) {
    return (float)((double)amax * (1.0 / 127.0));
}

// Reciprocal of a scale in FP64, accurate to a few FP64 ulps (hardware
// estimate plus two Newton steps); 0 for a zero scale.
__device__ __forceinline__ double scale_reciprocal(float s) {
    double sd = (double)s;
    double r = __builtin_amdgcn_rcp(sd);
    double e = __builtin_fma(-sd, r, 1.0);
    r = __builtin_fma(r, e, r);
    e = __builtin_fma(-sd, r, 1.0);
    r = __builtin_fma(r, e, r);
    return s == 0.0f ? 0.0 : r;
}

// scale_reciprocal for the packing quantizer (quant4): a zero scale is first
// raised to 2^-1000 (one integer max on the high word of the FP64 value, in
// place of a compare and two selects), so its reciprocal is 2^1000.  A group
// with s = 0 then still gets code 0 everywhere: zero values give 0, and the
// nonzero values of a group whose amax / 127 underflowed to zero give an
// infinite quotient, whose packed low byte is 0.  Nonzero scales are at least
// 2^-149 and pass unchanged.
__device__ __forceinline__ double pack_reciprocal(float s) {
    const uint64_t bits = __builtin_bit_cast(uint64_t, (double)s);
    const uint32_t floor_hi = 0x01700000u;  // high word of 2^-1000
    uint32_t hi;
    asm("v_max_u32 %0, %1, %2" : "=v"(hi) : "v"((uint32_t)(bits >> 32)), "v"(floor_hi));
    const double sd = __builtin_bit_cast(double, ((uint64_t)hi << 32) | (uint32_t)bits);
    double r = __builtin_amdgcn_rcp(sd);
    double e = __builtin_fma(-sd, r, 1.0);
    r = __builtin_fma(r, e, r);
    e = __builtin_fma(-sd, r, 1.0);
    r = __builtin_fma(r, e, r);
    return r;
}

// RN32(x / s) for a group with reciprocal rinv.  The FP64 product is within
// 2^-52 relative of the exact quotient (|rinv - 1/s| is far below that), and a
// quotient of two FP32 numbers is never within 2^-49 relative of an FP32
// rounding midpoint, so rounding the product to FP32 gives the correctly
// rounded quotient (the same argument as in group_scale).
__device__ __forceinline__ float quant_quotient(float x, double rinv) {
    return (float)((double)x * rinv);
}

// Codes of four quotients y0..y3 (|y| <= 127 + 2^-16), packed little-endian
// (byte i <- code of y_i, two's complement).  Adding 1.5 * 2^23 rounds y to
// an integer, half to even, and leaves that integer in the low mantissa bits;
// the SDWA form writes the low byte of each sum straight into byte i of the
// packed word (dst_sel BYTE_i: result bits [7:0] -> destination bits
// [8i+7:8i]; the first write zeroes the other bytes, the rest preserve them).
__device__ __forceinline__ uint32_t pack4_codes(float y0, float y1, float y2, float y3) {
    const float magic = 12582912.0f;
    uint32_t d;
    asm(
        "v_add_f32_sdwa %0, %1, %2 dst_sel:BYTE_0 dst_unused:UNUSED_PAD src0_sel:DWORD "
        "src1_sel:DWORD"
        : "=v"(d)
        : "v"(y0), "v"(magic));
    asm(
        "v_add_f32_sdwa %0, %1, %2 dst_sel:BYTE_1 dst_unused:UNUSED_PRESERVE src0_sel:DWORD "
        "src1_sel:DWORD"
        : "+v"(d)
        : "v"(y1), "v"(magic));
    asm(
        "v_add_f32_sdwa %0, %1, %2 dst_sel:BYTE_2 dst_unused:UNUSED_PRESERVE src0_sel:DWORD "
        "src1_sel:DWORD"
        : "+v"(d)
        : "v"(y2), "v"(magic));
    asm(
        "v_add_f32_sdwa %0, %1, %2 dst_sel:BYTE_3 dst_unused:UNUSED_PRESERVE src0_sel:DWORD "
        "src1_sel:DWORD"
        : "+v"(d)
        : "v"(y3), "v"(magic));
    return d;
}

// Packed codes of four values sharing the reciprocal scale rinv.
__device__ __forceinline__ uint32_t quant4(float x0, float x1, float x2, float x3, double rinv) {
    return pack4_codes(quant_quotient(x0, rinv), quant_quotient(x1, rinv),
                       quant_quotient(x2, rinv), quant_quotient(x3, rinv));
}

// Two FP32 values to packed IEEE binary16 (lo -> bits [15:0], hi -> bits
// [31:16]), each rounded to nearest even: the same results as f32_to_f16_bits.
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
    uint32_t d;
    asm("v_cvt_pk_f16_f32 %0, %1, %2" : "=v"(d) : "v"(lo), "v"(hi));
    return d;
}

// a * f32(binary16 in the low / high half of w) with one rounding, as a
// mixed-precision fma whose addend is -0 (x + (-0) = x for every x, the sign
// of zero included), so the result equals the FP32 product a * f32(h).
__device__ __forceinline__ float mul_f16lo(float a, uint32_t w) {
    float d;
    asm("v_fma_mix_f32 %0, %1, %2, %3 op_sel_hi:[0,1,0]" : "=v"(d) : "v"(a), "v"(w), "v"(-0.0f));
    return d;
}
__device__ __forceinline__ float mul_f16hi(float a, uint32_t w) {
    float d;
    asm("v_fma_mix_f32 %0, %1, %2, %3 op_sel:[0,1,0] op_sel_hi:[0,1,0]"
        : "=v"(d)
        : "v"(a), "v"(w), "v"(-0.0f));
    return d;
}

__device__ __forceinline__ float sext_byte_to_f32(uint32_t w, int b) {
    return (float)(int32_t)(int8_t)(w >> (8 * b));
}

// ---- raw buffer access -------------------------------------------------
// A buffer resource holds a uniform base address and a byte range in
// SGPRs; each lane supplies only a 32-bit offset, and accesses outside
// [0, bytes) read zero and write nothing.  kStream marks data touched once
// per step (the state, q/k/v/g, o) as non-temporal.
struct alignas(16) U4 {
    uint32_t x, y, z, w;
};
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kRsrcWord3 = 0x00020000;  // gfx9 raw buffer, 32-bit data format
constexpr int kStream = 2;              // nt cache policy

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, bytes,
                                             kRsrcWord3);
}
__device__ __forceinline__ U4 buf_load16(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, kStream);
    return U4{v.x, v.y, v.z, v.w};
}
__device__ __forceinline__ void buf_store16(__amdgpu_buffer_rsrc_t r, U4 d, int voff, int soff) {
    const u32x4 v = {d.x, d.y, d.z, d.w};
    __builtin_amdgcn_raw_buffer_store_b128(v, r, voff, soff, kStream);
}
__device__ __forceinline__ void buf_store16_cached(__amdgpu_buffer_rsrc_t r, U4 d, int voff,
                                                   int soff) {
    const u32x4 v = {d.x, d.y, d.z, d.w};
    __builtin_amdgcn_raw_buffer_store_b128(v, r, voff, soff, 0);
}
__device__ __forceinline__ float buf_loadf(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, kStream));
}
__device__ __forceinline__ void buf_storef(__amdgpu_buffer_rsrc_t r, float d, int voff, int soff) {
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, d), r, voff, soff,
                                          kStream);
}

// ---- operand I/O in FP32 or bf16 (IO = 0 / 1) ---------------------------
// bf16 operands widen exactly to FP32; bf16 outputs are rounded to nearest
// even from the FP32 result (a NaN stays a quiet NaN).
template <int IO>
__device__ __forceinline__ float ld_gather(const void *base, size_t ob, int i) {
    if (IO == 0) return buf_loadf(make_rsrc(static_cast<const float *>(base) + ob, DK * 4), i * 4, 0);
    const uint16_t bits = __builtin_amdgcn_raw_buffer_load_b16(
        make_rsrc(static_cast<const uint16_t *>(base) + ob, DK * 2), i * 2, 0, kStream);
    return __builtin_bit_cast(float, (uint32_t)bits << 16);
}
template <int IO>
__device__ __forceinline__ float ld_stream(const void *base, size_t idx) {
    if (IO == 0) return __builtin_nontemporal_load(static_cast<const float *>(base) + idx);
    const uint16_t bits = __builtin_nontemporal_load(static_cast<const uint16_t *>(base) + idx);
    return __builtin_bit_cast(float, (uint32_t)bits << 16);
}
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float x) {
    const uint32_t u = __builtin_bit_cast(uint32_t, x);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
    return (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}
template <int IO>
__device__ __forceinline__ void st_stream(void *base, size_t idx, float v) {
    if (IO == 0)
        __builtin_nontemporal_store(v, static_cast<float *>(base) + idx);
    else
        __builtin_nontemporal_store(f32_to_bf16_rne(v), static_cast<uint16_t *>(base) + idx);
}

}  // namespace qrs
