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

// IEEE binary16 round-to-nearest-even (v_cvt_f16_f32 in the default mode).
__device__ __forceinline__ uint32_t f32_to_f16_bits(float x) {
    return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)x);
}

// Value of the partner lane tid ^ 1 (DPP quad_perm [1,0,3,2]).
__device__ __forceinline__ float partner_xor1(float x) {
    return __builtin_bit_cast(
        float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0xB1, 0xF, 0xF, true));
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

// Code of x in a group with reciprocal rinv: RN_int(RN32(x / s)), returned
// in the low byte (two's complement) of the result.  RN32(x * rinv) in FP64
// equals RN32(x / s) for the same reason as in group_scale (|rinv - 1/s| is
// far below the 2^-49 margin); adding 1.5 * 2^23 then rounds the FP32
// quotient to an integer, half to even, and leaves that integer in the low
// mantissa bits.  |x / s| <= 127 + 2^-16 keeps the result in [-127, 127].
__device__ __forceinline__ uint32_t quant_code_bits(float x, double rinv) {
    float qf = (float)((double)x * rinv);
    float y = qf + 12582912.0f;
    return __builtin_bit_cast(uint32_t, y);
}

// Pack the low bytes of four code words into one dword (byte i <- c_i).
__device__ __forceinline__ uint32_t pack4_low_bytes(uint32_t c0, uint32_t c1, uint32_t c2,
                                                    uint32_t c3) {
    uint32_t lo = __builtin_amdgcn_perm(c1, c0, 0x0c0c0400u);
    uint32_t hi = __builtin_amdgcn_perm(c3, c2, 0x04000c0cu);
    return lo | hi;
}

__device__ __forceinline__ float sext_byte_to_f32(uint32_t w, int b) {
    return (float)(int32_t)(int8_t)(w >> (8 * b));
}

}  // namespace qrs
