// qrs_dense.hip -- decode step on an uncompressed FP32 state (compression
// disabled): the deployment default the compressed format is compared with
// (DAMP arXiv HTML, section 6.1 "Inference": FP32 recurrent-state storage as
// the baseline).  Same delta-rule update and readout as the fused kernel
// (HTML section 3.1, Eq.(1)), the same rows per thread (its columns are
// interleaved, below) and the same stored coordinates; each unit is 65,536
// bytes of FP32 read and written once.
#include <atomic>

#include "qrs_internal.h"

namespace qrs {

// Thread t (cb = t & 7, rg = t >> 3) owns rows rg + 16 r (r = 0..7) and the
// 16 columns 32 j + 4 cb + i (j, i = 0..3): each 16-byte access of a wave
// then covers 8 whole 128-byte row segments.  The unit is addressed through
// a buffer resource (one 32-bit offset per lane), which keeps the kernel at
// three waves per SIMD.  As in the compressed kernel, the first generation
// of a grid of more than two generations starts staggered, here by j x 4096
// cycles for the j-th workgroup on a CU (a unit is 3.2 times as many bytes):
// 196.4-196.7 against 197.9-198.2 us at 8,192 units, 2 x 4096 within noise of
// that, 2048 between (two passes each, alternating in one run).
template <int KIND>
__global__ __launch_bounds__(THREADS) __attribute__((amdgpu_waves_per_eu(3, 3))) void
decode_f32_kernel(PoolView pool, const int32_t *__restrict__ slots, int h0, int hc, int first_gen,
                  int n_cus, const float *__restrict__ q, const float *__restrict__ k,
                  const float *__restrict__ v, const float *__restrict__ gate,
                  const float *__restrict__ beta, float *__restrict__ o) {
    __shared__ float s_k[DK];
    __shared__ float s_q[DK];
    __shared__ float s_dec[DK];
    __shared__ float s_bd[DV];
    __shared__ float s_vp[DV];
    __shared__ float s_kraw[DK];
    __shared__ float s_qraw[DK];
    __shared__ float s_graw[DK];
    __shared__ float s_qk[2];
    __shared__ float4 red_w[16][DV / 4];
    __shared__ float4 red_z[16][DV / 4];

    if ((int)blockIdx.x < first_gen) {
        const int j = (int)blockIdx.x / n_cus;
        for (int i = 0; i < j; ++i) __builtin_amdgcn_s_sleep(64);
    }
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
    const __amdgpu_buffer_rsrc_t st =
        make_rsrc(pool.base + ((size_t)slot * H + h) * F32_UNIT_BYTES, F32_UNIT_BYTES);
    const int off = rg * (DV * 4) + cb * 16;  // + 128 j bytes, + 8192 r (row rg + 16 r)

    // operand loads in model order (no load waits on another), then the state
    const size_t ob = (size_t)uu * DK;
    const int src = pool.perm[h * DK + tid];
    const float k_m = __builtin_nontemporal_load(k + ob + tid);
    const float q_m = __builtin_nontemporal_load(q + ob + tid);
    float g_m = 0.f;
    if (KIND == 1) g_m = __builtin_nontemporal_load(gate + ob + tid);
    const float c_t = pool.smooth[h * DV + tid];
    const float v_m = __builtin_nontemporal_load(v + ob + tid);
    __builtin_amdgcn_sched_barrier(0);
    float x[ROWS_PER_THREAD][COLS_PER_THREAD];
#pragma unroll
    for (int r = 0; r < ROWS_PER_THREAD; ++r) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const U4 t = buf_load16(st, off + 128 * j, 8192 * r);
            x[r][4 * j] = __builtin_bit_cast(float, t.x);
            x[r][4 * j + 1] = __builtin_bit_cast(float, t.y);
            x[r][4 * j + 2] = __builtin_bit_cast(float, t.z);
            x[r][4 * j + 3] = __builtin_bit_cast(float, t.w);
        }
    }
    __builtin_amdgcn_sched_barrier(0);

    // gather through pi in LDS: thread t takes stored row t
    const float beta_u = beta[uu];
    s_kraw[tid] = k_m;
    s_qraw[tid] = q_m;
    if (KIND == 1) s_graw[tid] = g_m;
    s_vp[tid] = v_m / c_t;
    __syncthreads();
    const float kt = s_kraw[src];
    const float qt = s_qraw[src];
    s_k[tid] = kt;
    s_q[tid] = qt;
    float dec_t;
    if (KIND == 0) {
        dec_t = gate[uu];
    } else {
        dec_t = expf(s_graw[src]);
        s_dec[tid] = dec_t;
    }
    {
        const float p = wave_allsum(qt * kt);
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
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        float pw[4], pz[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int c = 4 * j + i;
            float aw = kr[0] * x[0][c];
            float az = s_q[rg] * x[0][c];
#pragma unroll
            for (int r = 1; r < ROWS_PER_THREAD; ++r) {
                aw = __builtin_fmaf(kr[r], x[r][c], aw);
                az = __builtin_fmaf(s_q[rg + 16 * r], x[r][c], az);
            }
            pw[i] = aw;
            pz[i] = az;
        }
        red_w[rg][8 * j + cb] = make_float4(pw[0], pw[1], pw[2], pw[3]);
        red_z[rg][8 * j + cb] = make_float4(pz[0], pz[1], pz[2], pz[3]);
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
        const float bd = beta_u * (s_vp[tid] - w);
        const float qk = s_qk[0] + s_qk[1];
        __builtin_nontemporal_store(c_t * __builtin_fmaf(qk, bd, z), o + (size_t)uu * DV + tid);
        s_bd[tid] = bd;
    }
    __syncthreads();
    float bdc[COLS_PER_THREAD];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const float4 t = reinterpret_cast<const float4 *>(s_bd)[8 * j + cb];
        bdc[4 * j] = t.x;
        bdc[4 * j + 1] = t.y;
        bdc[4 * j + 2] = t.z;
        bdc[4 * j + 3] = t.w;
    }
#pragma unroll
    for (int r = 0; r < ROWS_PER_THREAD; ++r) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            U4 t;
            t.x = __builtin_bit_cast(uint32_t, __builtin_fmaf(kr[r], bdc[4 * j], x[r][4 * j]));
            t.y = __builtin_bit_cast(uint32_t,
                                     __builtin_fmaf(kr[r], bdc[4 * j + 1], x[r][4 * j + 1]));
            t.z = __builtin_bit_cast(uint32_t,
                                     __builtin_fmaf(kr[r], bdc[4 * j + 2], x[r][4 * j + 2]));
            t.w = __builtin_bit_cast(uint32_t,
                                     __builtin_fmaf(kr[r], bdc[4 * j + 3], x[r][4 * j + 3]));
            buf_store16(st, t, off + 128 * j, 8192 * r);
        }
    }
}

// Workgroups resident at launch (occupancy x CUs), queried once per device;
// both kinds have the same resources.  Concurrent first calls may both query,
// which is harmless (they store the same values).
static void f32_residency(int *per_cu, int *cus) {
    static std::atomic<int> s_per[16], s_cus[16];
    *per_cu = 0;
    *cus = 1;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 16) return;
    int p = s_per[dev].load(std::memory_order_acquire);
    int c = s_cus[dev].load(std::memory_order_relaxed);
    if (p == 0) {
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&p, decode_f32_kernel<0>, THREADS, 0) !=
                hipSuccess ||
            hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            c <= 0 || p <= 0)
            return;
        s_cus[dev].store(c, std::memory_order_relaxed);
        s_per[dev].store(p, std::memory_order_release);
    }
    *per_cu = p;
    *cus = c;
}

hipError_t launch_decode_f32(int kind, const PoolView &pool, const int32_t *slots, int n, int h0,
                             int hc, const float *q, const float *k, const float *v,
                             const float *gate, const float *beta, float *o, hipStream_t stream) {
    int per_cu = 0, cus = 1;
    f32_residency(&per_cu, &cus);
    const int units = n * hc, resident = per_cu * cus;
    const int first_gen = units > 2 * resident ? resident : 0;
    dim3 grid((unsigned)units), block(THREADS);
    if (kind == 0)
        hipLaunchKernelGGL(decode_f32_kernel<0>, grid, block, 0, stream, pool, slots, h0, hc,
                           first_gen, cus, q, k, v, gate, beta, o);
    else
        hipLaunchKernelGGL(decode_f32_kernel<1>, grid, block, 0, stream, pool, slots, h0, hc,
                           first_gen, cus, q, k, v, gate, beta, o);
    return hipGetLastError();
}

}  // namespace qrs
