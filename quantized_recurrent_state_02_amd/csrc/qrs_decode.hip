// qrs_decode.hip -- fused compressed-state decode step for GDN and KDA on gfx950.
//
// One workgroup of 128 threads owns one (slot, head) unit and performs, in one
// pass over HBM (DAMP arXiv HTML, Appendix A.5 "Fused decode executor"; v2
// reading notes, section 2.2):
//   load the 20,224-byte packed unit (16 FP16 rows, 112 INT8 rows, FP32 scales)
//   -> dequantize and decay in VGPRs (Tbar = Lambda That)
//   -> w = Tbar^T k', z = Tbar^T q' (column reductions through LDS)
//   -> delta = v' - w, readout o = c (.) (z + (q'.k') beta delta)
//   -> rank-1 write T = Tbar + k' (beta delta)^T            (HTML section 3.1, Eq.(1))
//   -> per-32-value absmax, s = amax/127, codes RN(x/s)      (v2 notes, Eqs.(5)-(6))
//   -> store the unit back in place.
// The state never leaves registers between the load and the store.  Operands
// arrive in model key order and are gathered through the per-head
// permutation; v is divided by the smoothing scales c and the readout is
// multiplied by them (v2 notes, section 2.7).
//
// The readout uses z + (q'.k') beta delta = T^T q' (the post-update FP32
// state of this step, before requantization), so both column reductions run
// in the same pass before the update.
#include "qrs_internal.h"

namespace qrs {

namespace {

struct alignas(16) U4 {
    uint32_t x, y, z, w;
};

__device__ __forceinline__ U4 ld16(const uint8_t *p) {
    return *reinterpret_cast<const U4 *>(p);
}
__device__ __forceinline__ void st16(uint8_t *p, U4 v) {
    *reinterpret_cast<U4 *>(p) = v;
}

// Sum over the 64 lanes of a wave (every lane gets the total).
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, 64);
    return x;
}

}  // namespace

// KIND 0: GDN (gate = alpha [n][H]); KIND 1: KDA (gate = g [n][H][128]).
template <int KIND>
__global__ __launch_bounds__(THREADS) void decode_i8f16_kernel(
    PoolView pool, const int32_t *__restrict__ slots, const float *__restrict__ q,
    const float *__restrict__ k, const float *__restrict__ v, const float *__restrict__ gate,
    const float *__restrict__ beta, float *__restrict__ o) {
    __shared__ float s_k[DK];
    __shared__ float s_q[DK];
    __shared__ float s_dec[DK];
    __shared__ float s_bd[DV];
    __shared__ float s_qk[2];
    __shared__ float4 red_w[16][DV / 4];
    __shared__ float4 red_z[16][DV / 4];

    const int tid = threadIdx.x;
    const int uu = blockIdx.x;  // b * H + h
    const int H = pool.num_heads;
    const int b = uu / H;
    const int h = uu - b * H;
    const int slot = slots[b];
    if (slot < 0 || slot >= pool.num_slots) {
        o[(size_t)uu * DV + tid] = __builtin_nanf("");
        return;
    }
    const int cb = tid & 7;
    const int rg = tid >> 3;
    uint8_t *unit = pool.base + ((size_t)slot * H + h) * UNIT_BYTES;

    // ---- issue the state loads first (the long-latency part) ----
    U4 hi_raw[2];
    U4 lo_raw[ROWS_PER_THREAD - 1];
    float sc_old[ROWS_PER_THREAD - 1];
    {
        const uint8_t *hp = unit + HI_OFF + rg * (DV * 2) + cb * 32;
        hi_raw[0] = ld16(hp);
        hi_raw[1] = ld16(hp + 16);
#pragma unroll
        for (int r = 1; r < ROWS_PER_THREAD; ++r) {
            const int lrow = rg + 16 * (r - 1);  // INT8 row index 0..111
            lo_raw[r - 1] = ld16(unit + LO_OFF + lrow * DV + cb * 16);
            sc_old[r - 1] =
                *reinterpret_cast<const float *>(unit + SC_OFF + (lrow * NGRP + (cb >> 1)) * 4);
        }
    }

    // ---- operands: thread t gathers stored row t and owns value column t ----
    const size_t ob = (size_t)uu * DK;
    const int src = pool.perm[h * DK + tid];
    const float kt = k[ob + src];
    const float qt = q[ob + src];
    float dec_t;
    if (KIND == 0)
        dec_t = gate[uu];
    else
        dec_t = expf(gate[ob + src]);
    const float c_t = pool.smooth[h * DV + tid];
    const float vp_t = v[ob + tid] / c_t;  // v' = D_c^{-1} v
    const float beta_u = beta[uu];
    s_k[tid] = kt;
    s_q[tid] = qt;
    if (KIND == 1) s_dec[tid] = dec_t;
    {
        const float p = wave_sum(qt * kt);
        if ((tid & 63) == 0) s_qk[tid >> 6] = p;
    }
    __syncthreads();

    float kr[ROWS_PER_THREAD], qr[ROWS_PER_THREAD], dr[ROWS_PER_THREAD];
#pragma unroll
    for (int r = 0; r < ROWS_PER_THREAD; ++r) {
        kr[r] = s_k[rg + 16 * r];
        qr[r] = s_q[rg + 16 * r];
        dr[r] = KIND == 0 ? dec_t : s_dec[rg + 16 * r];
    }

    // ---- dequantize + decay (Tbar = Lambda That) ----
    float x[ROWS_PER_THREAD][COLS_PER_THREAD];
    {
        const uint32_t hw[8] = {hi_raw[0].x, hi_raw[0].y, hi_raw[0].z, hi_raw[0].w,
                                hi_raw[1].x, hi_raw[1].y, hi_raw[1].z, hi_raw[1].w};
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            x[0][2 * c] = dr[0] * f16_bits_to_f32(hw[c] & 0xffffu);
            x[0][2 * c + 1] = dr[0] * f16_bits_to_f32(hw[c] >> 16);
        }
    }
#pragma unroll
    for (int r = 1; r < ROWS_PER_THREAD; ++r) {
        const float a = dr[r] * sc_old[r - 1];
        const uint32_t lw[4] = {lo_raw[r - 1].x, lo_raw[r - 1].y, lo_raw[r - 1].z,
                                lo_raw[r - 1].w};
#pragma unroll
        for (int c = 0; c < 16; ++c) x[r][c] = a * sext_byte_to_f32(lw[c >> 2], c & 3);
    }

    // ---- partial column reductions over this thread's 8 rows ----
    {
        float pw[COLS_PER_THREAD], pz[COLS_PER_THREAD];
#pragma unroll
        for (int c = 0; c < COLS_PER_THREAD; ++c) {
            float aw = kr[0] * x[0][c];
            float az = qr[0] * x[0][c];
#pragma unroll
            for (int r = 1; r < ROWS_PER_THREAD; ++r) {
                aw = __builtin_fmaf(kr[r], x[r][c], aw);
                az = __builtin_fmaf(qr[r], x[r][c], az);
            }
            pw[c] = aw;
            pz[c] = az;
        }
#pragma unroll
        for (int c4 = 0; c4 < 4; ++c4) {
            red_w[rg][cb * 4 + c4] =
                make_float4(pw[4 * c4], pw[4 * c4 + 1], pw[4 * c4 + 2], pw[4 * c4 + 3]);
            red_z[rg][cb * 4 + c4] =
                make_float4(pz[4 * c4], pz[4 * c4 + 1], pz[4 * c4 + 2], pz[4 * c4 + 3]);
        }
    }
    __syncthreads();

    // ---- thread t finishes column t: delta, readout ----
    {
        const float *rw = reinterpret_cast<const float *>(red_w);
        const float *rz = reinterpret_cast<const float *>(red_z);
        float w = 0.f, z = 0.f;
#pragma unroll
        for (int g = 0; g < 16; ++g) {
            w += rw[g * DV + tid];
            z += rz[g * DV + tid];
        }
        const float delta = vp_t - w;
        const float bd = beta_u * delta;
        const float qk = s_qk[0] + s_qk[1];
        o[(size_t)uu * DV + tid] = c_t * __builtin_fmaf(qk, bd, z);
        s_bd[tid] = bd;
    }
    __syncthreads();

    float bdc[COLS_PER_THREAD];
#pragma unroll
    for (int c = 0; c < COLS_PER_THREAD; ++c) bdc[c] = s_bd[cb * 16 + c];

    // ---- rank-1 write, requantize, store ----
    // FP16 row (r = 0)
    {
#pragma unroll
        for (int c = 0; c < COLS_PER_THREAD; ++c) x[0][c] = __builtin_fmaf(kr[0], bdc[c], x[0][c]);
        uint32_t hw[8];
#pragma unroll
        for (int c = 0; c < 8; ++c)
            hw[c] = f32_to_f16_bits(x[0][2 * c]) | (f32_to_f16_bits(x[0][2 * c + 1]) << 16);
        uint8_t *hp = unit + HI_OFF + rg * (DV * 2) + cb * 32;
        st16(hp, U4{hw[0], hw[1], hw[2], hw[3]});
        st16(hp + 16, U4{hw[4], hw[5], hw[6], hw[7]});
    }
    // INT8 rows
#pragma unroll
    for (int r = 1; r < ROWS_PER_THREAD; ++r) {
        float amax = 0.f;
#pragma unroll
        for (int c = 0; c < COLS_PER_THREAD; ++c) {
            x[r][c] = __builtin_fmaf(kr[r], bdc[c], x[r][c]);
            amax = fmaxf(amax, fabsf(x[r][c]));
        }
        amax = fmaxf(amax, partner_xor1(amax));
        const float s = group_scale(amax);
        const double rinv = scale_reciprocal(s);
        uint32_t cw[4];
#pragma unroll
        for (int c4 = 0; c4 < 4; ++c4)
            cw[c4] = pack4_low_bytes(quant_code_bits(x[r][4 * c4], rinv),
                                     quant_code_bits(x[r][4 * c4 + 1], rinv),
                                     quant_code_bits(x[r][4 * c4 + 2], rinv),
                                     quant_code_bits(x[r][4 * c4 + 3], rinv));
        const int lrow = rg + 16 * (r - 1);
        st16(unit + LO_OFF + lrow * DV + cb * 16, U4{cw[0], cw[1], cw[2], cw[3]});
        if ((cb & 1) == 0)
            *reinterpret_cast<float *>(unit + SC_OFF + (lrow * NGRP + (cb >> 1)) * 4) = s;
    }
}

// Launchers (host).
hipError_t launch_decode_i8f16(int kind, const PoolView &pool, const int32_t *slots, int n,
                               const float *q, const float *k, const float *v, const float *gate,
                               const float *beta, float *o, hipStream_t stream) {
    dim3 grid((unsigned)(n * pool.num_heads)), block(THREADS);
    if (kind == 0)
        hipLaunchKernelGGL(decode_i8f16_kernel<0>, grid, block, 0, stream, pool, slots, q, k, v,
                           gate, beta, o);
    else
        hipLaunchKernelGGL(decode_i8f16_kernel<1>, grid, block, 0, stream, pool, slots, q, k, v,
                           gate, beta, o);
    return hipGetLastError();
}

}  // namespace qrs
