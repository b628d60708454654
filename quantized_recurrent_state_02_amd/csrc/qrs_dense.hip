// qrs_dense.hip -- decode step on an uncompressed FP32 state (compression
// disabled): the deployment default the compressed format is compared with
// (DAMP arXiv HTML, section 6.1 "Inference": FP32 recurrent-state storage as
// the baseline).  Same delta-rule update and readout as the fused kernel
// (HTML section 3.1, Eq.(1)), same thread mapping and stored coordinates;
// each unit is 65,536 bytes of FP32 read and written once.
#include "qrs_internal.h"

namespace qrs {

namespace {
__device__ __forceinline__ float wave_sum_f(float x) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, 64);
    return x;
}
}  // namespace

template <int KIND>
__global__ __launch_bounds__(THREADS) void decode_f32_kernel(
    PoolView pool, const int32_t *__restrict__ slots, int h0, int hc, const float *__restrict__ q,
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
    const int H = pool.num_heads;
    const int b = blockIdx.x / hc;  // heads [h0, h0 + hc) of each slot
    const int h = h0 + (blockIdx.x - b * hc);
    const int uu = b * H + h;
    const int slot = slots[b];
    if (slot < 0 || slot >= pool.num_slots) {
        o[(size_t)uu * DV + tid] = __builtin_nanf("");
        return;
    }
    const int cb = tid & 7;
    const int rg = tid >> 3;
    float *unit = reinterpret_cast<float *>(pool.base + ((size_t)slot * H + h) * F32_UNIT_BYTES);

    float x[ROWS_PER_THREAD][COLS_PER_THREAD];
#pragma unroll
    for (int r = 0; r < ROWS_PER_THREAD; ++r) {
        const float4 *p = reinterpret_cast<const float4 *>(unit + (rg + 16 * r) * DV + cb * 16);
#pragma unroll
        for (int c4 = 0; c4 < 4; ++c4) {
            const float4 t = p[c4];
            x[r][4 * c4] = t.x;
            x[r][4 * c4 + 1] = t.y;
            x[r][4 * c4 + 2] = t.z;
            x[r][4 * c4 + 3] = t.w;
        }
    }

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
    const float vp_t = v[ob + tid] / c_t;
    const float beta_u = beta[uu];
    s_k[tid] = kt;
    s_q[tid] = qt;
    if (KIND == 1) s_dec[tid] = dec_t;
    {
        const float p = wave_sum_f(qt * kt);
        if ((tid & 63) == 0) s_qk[tid >> 6] = p;
    }
    __syncthreads();

    float kr[ROWS_PER_THREAD];
#pragma unroll
    for (int r = 0; r < ROWS_PER_THREAD; ++r) {
        kr[r] = s_k[rg + 16 * r];
        const float d = KIND == 0 ? dec_t : s_dec[rg + 16 * r];
#pragma unroll
        for (int c = 0; c < COLS_PER_THREAD; ++c) x[r][c] *= d;
    }
    {
        float pw[COLS_PER_THREAD], pz[COLS_PER_THREAD];
#pragma unroll
        for (int c = 0; c < COLS_PER_THREAD; ++c) {
            float aw = kr[0] * x[0][c];
            float az = s_q[rg] * x[0][c];
#pragma unroll
            for (int r = 1; r < ROWS_PER_THREAD; ++r) {
                aw = __builtin_fmaf(kr[r], x[r][c], aw);
                az = __builtin_fmaf(s_q[rg + 16 * r], x[r][c], az);
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
    {
        const float *rw = reinterpret_cast<const float *>(red_w);
        const float *rz = reinterpret_cast<const float *>(red_z);
        float w = 0.f, z = 0.f;
#pragma unroll
        for (int g = 0; g < 16; ++g) {
            w += rw[g * DV + tid];
            z += rz[g * DV + tid];
        }
        const float bd = beta_u * (vp_t - w);
        const float qk = s_qk[0] + s_qk[1];
        o[(size_t)uu * DV + tid] = c_t * __builtin_fmaf(qk, bd, z);
        s_bd[tid] = bd;
    }
    __syncthreads();
    float bdc[COLS_PER_THREAD];
#pragma unroll
    for (int c = 0; c < COLS_PER_THREAD; ++c) bdc[c] = s_bd[cb * 16 + c];
#pragma unroll
    for (int r = 0; r < ROWS_PER_THREAD; ++r) {
        float4 *p = reinterpret_cast<float4 *>(unit + (rg + 16 * r) * DV + cb * 16);
#pragma unroll
        for (int c4 = 0; c4 < 4; ++c4) {
            float4 t;
            t.x = __builtin_fmaf(kr[r], bdc[4 * c4], x[r][4 * c4]);
            t.y = __builtin_fmaf(kr[r], bdc[4 * c4 + 1], x[r][4 * c4 + 1]);
            t.z = __builtin_fmaf(kr[r], bdc[4 * c4 + 2], x[r][4 * c4 + 2]);
            t.w = __builtin_fmaf(kr[r], bdc[4 * c4 + 3], x[r][4 * c4 + 3]);
            p[c4] = t;
        }
    }
}

hipError_t launch_decode_f32(int kind, const PoolView &pool, const int32_t *slots, int n, int h0,
                             int hc, const float *q, const float *k, const float *v,
                             const float *gate, const float *beta, float *o, hipStream_t stream) {
    dim3 grid((unsigned)(n * hc)), block(THREADS);
    if (kind == 0)
        hipLaunchKernelGGL(decode_f32_kernel<0>, grid, block, 0, stream, pool, slots, h0, hc, q, k,
                           v, gate, beta, o);
    else
        hipLaunchKernelGGL(decode_f32_kernel<1>, grid, block, 0, stream, pool, slots, h0, hc, q, k,
                           v, gate, beta, o);
    return hipGetLastError();
}

}  // namespace qrs
