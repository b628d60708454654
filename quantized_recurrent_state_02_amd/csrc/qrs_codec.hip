// qrs_codec.hip -- standalone store (encode) and dequant (decode) of whole
// states, for set-up, export/import and checks.
//
// Encoding of one unit in stored coordinates (DAMP v2 reading notes,
// section 2.2, Eqs.(5)-(6); packed layout of the arXiv HTML, Appendix A.5,
// Eq.(17)): rows 0..15 FP16 round-to-nearest-even; rows 16..127 per 32-value
// group s = RN(max|x| / 127), code = RN_int(RN(x / s)).  Model-space input is
// first mapped to stored coordinates, T[i][j] = S[perm[i]][j] / c[j]
// (v2 notes, section 2.7).  Same thread mapping as the decode kernels.
// CODEC 1 is the first revision's low tier instead (block-32 Hadamard,
// asymmetric UINT8 codes, FP16 scale and zero point: HTML section 3.2
// Eq.(3), Appendix A.1), see qrs_hadamard.h.
#include "qrs_hadamard.h"

namespace qrs {

namespace {
struct alignas(16) V4 {
    uint32_t x, y, z, w;
};
}  // namespace

// Load this thread's 8 x 16 block of state in stored coordinates.
__device__ __forceinline__ void load_input_block(const float *Su, const int32_t *perm_h,
                                                 const float *c_h, int space, int rg, int cb,
                                                 float (&x)[ROWS_PER_THREAD][COLS_PER_THREAD]) {
#pragma unroll
    for (int r = 0; r < ROWS_PER_THREAD; ++r) {
        const int row = rg + 16 * r;
        const int src = space == 0 ? perm_h[row] : row;
        const float4 *p = reinterpret_cast<const float4 *>(Su + (size_t)src * DV + cb * 16);
#pragma unroll
        for (int c4 = 0; c4 < 4; ++c4) {
            const float4 t = p[c4];
            x[r][4 * c4] = t.x;
            x[r][4 * c4 + 1] = t.y;
            x[r][4 * c4 + 2] = t.z;
            x[r][4 * c4 + 3] = t.w;
        }
        if (space == 0) {
#pragma unroll
            for (int c = 0; c < COLS_PER_THREAD; ++c) x[r][c] = x[r][c] / c_h[cb * 16 + c];
        }
    }
}

template <int CODEC>
__global__ __launch_bounds__(THREADS) void store_packed_kernel(PoolView pool,
                                                               const int32_t *__restrict__ slots,
                                                               const float *__restrict__ S,
                                                               int space) {
    const int tid = threadIdx.x;
    const int uu = blockIdx.x;
    const int H = pool.num_heads;
    const int b = uu / H;
    const int h = uu - b * H;
    const int slot = slots[b];
    if (slot < 0 || slot >= pool.num_slots) return;
    const int cb = tid & 7;
    const int rg = tid >> 3;
    uint8_t *unit = pool.base + ((size_t)slot * H + h) * UNIT_BYTES;
    float x[ROWS_PER_THREAD][COLS_PER_THREAD];
    load_input_block(S + (size_t)uu * DK * DV, pool.perm + h * DK, pool.smooth + h * DV, space,
                     rg, cb, x);
    {
        uint32_t hw[8];
#pragma unroll
        for (int c = 0; c < 8; ++c)
            hw[c] = pack_f16x2(x[0][2 * c], x[0][2 * c + 1]);
        V4 *hp = reinterpret_cast<V4 *>(unit + HI_OFF + rg * (DV * 2) + cb * 32);
        hp[0] = V4{hw[0], hw[1], hw[2], hw[3]};
        hp[1] = V4{hw[4], hw[5], hw[6], hw[7]};
    }
#pragma unroll
    for (int r = 1; r < ROWS_PER_THREAD; ++r) {
        const int lrow = rg + 16 * (r - 1);
        V4 cw;
        uint32_t meta;
        if (CODEC == 0) {
            float amax = 0.f;
#pragma unroll
            for (int c = 0; c < COLS_PER_THREAD; ++c) amax = fmaxf(amax, fabsf(x[r][c]));
            amax = pair_max(amax);
            const float s = group_scale(amax);
            const double rinv = pack_reciprocal(s);
            cw.x = quant4(x[r][0], x[r][1], x[r][2], x[r][3], rinv);
            cw.y = quant4(x[r][4], x[r][5], x[r][6], x[r][7], rinv);
            cw.z = quant4(x[r][8], x[r][9], x[r][10], x[r][11], rinv);
            cw.w = quant4(x[r][12], x[r][13], x[r][14], x[r][15], rinv);
            meta = __builtin_bit_cast(uint32_t, s);
        } else {
            hadamard32_pair(x[r], (cb & 1) != 0);
            float lo = x[r][0], hi = x[r][0];
#pragma unroll
            for (int c = 1; c < COLS_PER_THREAD; ++c) {
                lo = fminf(lo, x[r][c]);
                hi = fmaxf(hi, x[r][c]);
            }
            const U8Params pr = u8_params(lo, hi);
            cw.x = u8_pack4(x[r][0], x[r][1], x[r][2], x[r][3], pr);
            cw.y = u8_pack4(x[r][4], x[r][5], x[r][6], x[r][7], pr);
            cw.z = u8_pack4(x[r][8], x[r][9], x[r][10], x[r][11], pr);
            cw.w = u8_pack4(x[r][12], x[r][13], x[r][14], x[r][15], pr);
            meta = pr.meta;
        }
        *reinterpret_cast<V4 *>(unit + LO_OFF + lrow * DV + cb * 16) = cw;
        if ((cb & 1) == 0)
            *reinterpret_cast<uint32_t *>(unit + SC_OFF + (lrow * NGRP + (cb >> 1)) * 4) = meta;
    }
}

template <int CODEC>
__global__ __launch_bounds__(THREADS) void dequant_packed_kernel(PoolView pool,
                                                                 const int32_t *__restrict__ slots,
                                                                 float *__restrict__ S, int space) {
    const int tid = threadIdx.x;
    const int uu = blockIdx.x;
    const int H = pool.num_heads;
    const int b = uu / H;
    const int h = uu - b * H;
    const int slot = slots[b];
    const int cb = tid & 7;
    const int rg = tid >> 3;
    float *Su = S + (size_t)uu * DK * DV;
    const bool valid = slot >= 0 && slot < pool.num_slots;
    const uint8_t *unit = pool.base + ((size_t)(valid ? slot : 0) * H + h) * UNIT_BYTES;
#pragma unroll
    for (int r = 0; r < ROWS_PER_THREAD; ++r) {
        const int row = rg + 16 * r;
        float x[COLS_PER_THREAD];
        if (!valid) {
#pragma unroll
            for (int c = 0; c < COLS_PER_THREAD; ++c) x[c] = __builtin_nanf("");
        } else if (r == 0) {
            const V4 *hp = reinterpret_cast<const V4 *>(unit + HI_OFF + rg * (DV * 2) + cb * 32);
            const V4 a = hp[0], bb = hp[1];
            const uint32_t hw[8] = {a.x, a.y, a.z, a.w, bb.x, bb.y, bb.z, bb.w};
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                x[2 * c] = f16_bits_to_f32(hw[c] & 0xffffu);
                x[2 * c + 1] = f16_bits_to_f32(hw[c] >> 16);
            }
        } else {
            const int lrow = row - KHI;
            const V4 lw = *reinterpret_cast<const V4 *>(unit + LO_OFF + lrow * DV + cb * 16);
            const uint32_t meta =
                *reinterpret_cast<const uint32_t *>(unit + SC_OFF + (lrow * NGRP + (cb >> 1)) * 4);
            const uint32_t w4[4] = {lw.x, lw.y, lw.z, lw.w};
            if (CODEC == 0) {
                const float s = __builtin_bit_cast(float, meta);
#pragma unroll
                for (int c = 0; c < 16; ++c) x[c] = s * sext_byte_to_f32(w4[c >> 2], c & 3);
            } else {
                const float sh = f16_bits_to_f32(meta & 0xffffu), zh = f16_bits_to_f32(meta >> 16);
#pragma unroll
                for (int c = 0; c < 16; ++c) x[c] = u8_dequant(w4[c >> 2], c & 3, sh, zh);
                hadamard32_pair(x, (cb & 1) != 0);
            }
        }
        int dst = row;
        if (space == 0 && valid) {
            dst = pool.perm[h * DK + row];
#pragma unroll
            for (int c = 0; c < COLS_PER_THREAD; ++c) x[c] = x[c] * pool.smooth[h * DV + cb * 16 + c];
        }
        float4 *p = reinterpret_cast<float4 *>(Su + (size_t)dst * DV + cb * 16);
#pragma unroll
        for (int c4 = 0; c4 < 4; ++c4)
            p[c4] = make_float4(x[4 * c4], x[4 * c4 + 1], x[4 * c4 + 2], x[4 * c4 + 3]);
    }
}

// FP32 pools: the state is stored as is (stored coordinates).
__global__ __launch_bounds__(THREADS) void store_f32_kernel(PoolView pool,
                                                            const int32_t *__restrict__ slots,
                                                            const float *__restrict__ S,
                                                            int space) {
    const int tid = threadIdx.x;
    const int uu = blockIdx.x;
    const int H = pool.num_heads;
    const int b = uu / H;
    const int h = uu - b * H;
    const int slot = slots[b];
    if (slot < 0 || slot >= pool.num_slots) return;
    const int cb = tid & 7;
    const int rg = tid >> 3;
    float *unit = reinterpret_cast<float *>(pool.base + ((size_t)slot * H + h) * F32_UNIT_BYTES);
    float x[ROWS_PER_THREAD][COLS_PER_THREAD];
    load_input_block(S + (size_t)uu * DK * DV, pool.perm + h * DK, pool.smooth + h * DV, space,
                     rg, cb, x);
#pragma unroll
    for (int r = 0; r < ROWS_PER_THREAD; ++r) {
        float4 *p = reinterpret_cast<float4 *>(unit + (rg + 16 * r) * DV + cb * 16);
#pragma unroll
        for (int c4 = 0; c4 < 4; ++c4)
            p[c4] = make_float4(x[r][4 * c4], x[r][4 * c4 + 1], x[r][4 * c4 + 2], x[r][4 * c4 + 3]);
    }
}

__global__ __launch_bounds__(THREADS) void dequant_f32_kernel(PoolView pool,
                                                              const int32_t *__restrict__ slots,
                                                              float *__restrict__ S, int space) {
    const int tid = threadIdx.x;
    const int uu = blockIdx.x;
    const int H = pool.num_heads;
    const int b = uu / H;
    const int h = uu - b * H;
    const int slot = slots[b];
    const int cb = tid & 7;
    const int rg = tid >> 3;
    float *Su = S + (size_t)uu * DK * DV;
    const bool valid = slot >= 0 && slot < pool.num_slots;
    const float *unit = reinterpret_cast<const float *>(
        pool.base + ((size_t)(valid ? slot : 0) * H + h) * F32_UNIT_BYTES);
#pragma unroll
    for (int r = 0; r < ROWS_PER_THREAD; ++r) {
        const int row = rg + 16 * r;
        float x[COLS_PER_THREAD];
        const float4 *p = reinterpret_cast<const float4 *>(unit + row * DV + cb * 16);
#pragma unroll
        for (int c4 = 0; c4 < 4; ++c4) {
            const float4 t = p[c4];
            x[4 * c4] = valid ? t.x : __builtin_nanf("");
            x[4 * c4 + 1] = valid ? t.y : __builtin_nanf("");
            x[4 * c4 + 2] = valid ? t.z : __builtin_nanf("");
            x[4 * c4 + 3] = valid ? t.w : __builtin_nanf("");
        }
        int dst = row;
        if (space == 0 && valid) {
            dst = pool.perm[h * DK + row];
#pragma unroll
            for (int c = 0; c < COLS_PER_THREAD; ++c) x[c] = x[c] * pool.smooth[h * DV + cb * 16 + c];
        }
        float4 *q = reinterpret_cast<float4 *>(Su + (size_t)dst * DV + cb * 16);
#pragma unroll
        for (int c4 = 0; c4 < 4; ++c4)
            q[c4] = make_float4(x[4 * c4], x[4 * c4 + 1], x[4 * c4 + 2], x[4 * c4 + 3]);
    }
}

hipError_t launch_store(int fmt, const PoolView &pool, const int32_t *slots, int n, const float *S,
                        int space, hipStream_t stream) {
    dim3 grid((unsigned)(n * pool.num_heads)), block(THREADS);
    if (fmt == 1)
        hipLaunchKernelGGL(store_packed_kernel<0>, grid, block, 0, stream, pool, slots, S, space);
    else if (fmt == 2)
        hipLaunchKernelGGL(store_packed_kernel<1>, grid, block, 0, stream, pool, slots, S, space);
    else
        hipLaunchKernelGGL(store_f32_kernel, grid, block, 0, stream, pool, slots, S, space);
    return hipGetLastError();
}

hipError_t launch_dequant(int fmt, const PoolView &pool, const int32_t *slots, int n, float *S,
                          int space, hipStream_t stream) {
    dim3 grid((unsigned)(n * pool.num_heads)), block(THREADS);
    if (fmt == 1)
        hipLaunchKernelGGL(dequant_packed_kernel<0>, grid, block, 0, stream, pool, slots, S, space);
    else if (fmt == 2)
        hipLaunchKernelGGL(dequant_packed_kernel<1>, grid, block, 0, stream, pool, slots, S, space);
    else
        hipLaunchKernelGGL(dequant_f32_kernel, grid, block, 0, stream, pool, slots, S, space);
    return hipGetLastError();
}

}  // namespace qrs
