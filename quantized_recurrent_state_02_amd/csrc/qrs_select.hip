// qrs_select.hip -- statistics for the offline choice of the FP16 key channels
// (DAMP arXiv HTML, section 4 "Accumulated-error risk" and "Budgeted
// selection", Appendix A.2 Eqs.(13)-(15); v2 reading notes, section 2.5).
//
//   channel_error_kernel      e[s][h][u]: squared error of key channel u of
//                             calibration state s under the INT8 storage
//                             mapping, in model coordinates (Eq.(14) integrand)
//   persistence_window_kernel W[s][h][u] = 1 + sum_{j=1..H} prod_{r<=j} a_{t+r,u}^2
//                             over the sample's own trajectory (v2 notes)
//   persistence_geo_kernel    P[h][u] = 1 / max(1 - a_eff^2, tau),
//                             a_eff = exp(sum_s w_s log a_s)  (Eq.(15))
//   channel_scores_kernel     C[h][u] = sum_s w_s e_s W_s, or (sum_s w_s e_s) P
//
// The error kernel reads each 64 KiB calibration state once with 16-byte
// loads (HBM-bound); the others are small.  Sums over samples run in sample
// order inside one thread, so every result is deterministic.  Multiply-add
// contraction is off in this file: each product and sum is rounded on its
// own, in the order written.
#include "qrs_internal.h"

#pragma clang fp contract(off)

namespace qrs {

namespace {

constexpr int SEL_THREADS = 128;
static_assert(SEL_THREADS == DK, "the error kernel's last step gives thread t row t");

// max(m, m of the lane that the DPP control CTRL names, inside the lane's
// 16-lane row), for m the bits of a non-negative float (such floats order
// like their bit patterns): one DPP-modified v_max_u32.
template <int CTRL>
__device__ __forceinline__ uint32_t lane_max_step(uint32_t m) {
    const uint32_t o = (uint32_t)__builtin_amdgcn_mov_dpp((int)m, CTRL, 0xf, 0xf, true);
    return m > o ? m : o;
}

// v from the lane that the DPP control CTRL names (inside the lane's 16-lane
// row), for an FP64 value: its two halves moved separately.
template <int CTRL>
__device__ __forceinline__ double dpp_d(double v) {
    const uint64_t b = __builtin_bit_cast(uint64_t, v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)b, CTRL, 0xf, 0xf, true);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)(b >> 32), CTRL, 0xf, 0xf, true);
    return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

// One workgroup per (sample, head).  Thread t works on row 4 p + (t >> 5) in
// pass p (32 passes) and holds columns 4 (t & 31) .. +3; the eight threads of
// one 32-value group are consecutive lanes, so the group maximum takes three
// DPP steps (the partner in the pair, in the quad, in the eight lanes).  A
// row's squared errors are summed over each 16-lane half of its 32 threads
// with DPP (each step adds a lane and its partner in both orders, so the 16
// lanes hold the same bits) and the two half sums go to LDS; at the end
// thread t adds row t's two.
__global__ __launch_bounds__(SEL_THREADS) void channel_error_kernel(
    const float *__restrict__ S, const float *__restrict__ smooth, int num_heads,
    double *__restrict__ e) {
    const int tid = threadIdx.x;
    const size_t sh = blockIdx.x;
    const int h = (int)(sh % (size_t)num_heads);
    __shared__ double part[2][DK];   // the two half-row sums of each row
    const int rr = tid >> 5;
    const int l = tid & 31;
    const __amdgpu_buffer_rsrc_t sr = make_rsrc(S + sh * (size_t)(DK * DV), DK * DV * 4);
    float4 c4 = make_float4(1.f, 1.f, 1.f, 1.f);
    if (smooth) c4 = *reinterpret_cast<const float4 *>(smooth + (size_t)h * DV + 4 * l);
    const float cv[4] = {c4.x, c4.y, c4.z, c4.w};
    // S / c as RN32(S * rc) with an FP64 reciprocal: the correctly rounded
    // quotient, by the argument of quant_quotient (c > 0)
    double rc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) rc[j] = scale_reciprocal(cv[j]);
    // 16 rows per thread in flight: all loads of a batch are issued first
    constexpr int BATCH = 16;
    for (int p0 = 0; p0 < DK / 4; p0 += BATCH) {
        U4 raw[BATCH];
#pragma unroll
        for (int i = 0; i < BATCH; ++i)
            raw[i] = buf_load16(sr, ((4 * (p0 + i) + rr) * DV + 4 * l) * 4, 0);
#pragma unroll
        for (int i = 0; i < BATCH; ++i) {
            const int u = 4 * (p0 + i) + rr;
            const float sv[4] = {__builtin_bit_cast(float, raw[i].x), __builtin_bit_cast(float, raw[i].y),
                                 __builtin_bit_cast(float, raw[i].z), __builtin_bit_cast(float, raw[i].w)};
            float x[4];
            float amax = 0.f;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                x[j] = quant_quotient(sv[j], rc[j]);  // stored value coordinates
                amax = fmaxf(amax, fabsf(x[j]));
            }
            uint32_t mb = __builtin_bit_cast(uint32_t, amax);
            mb = lane_max_step<0xb1>(mb);    // quad_perm [1,0,3,2]
            mb = lane_max_step<0x4e>(mb);    // quad_perm [2,3,0,1]
            mb = lane_max_step<0x141>(mb);   // row_half_mirror
            amax = __builtin_bit_cast(float, mb);
            const float s = group_scale(amax);
            const double rinv = scale_reciprocal(s);
            double acc = 0.0;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float code = fminf(fmaxf(rintf(quant_quotient(x[j], rinv)), -127.f), 127.f);
                const float back = (s * code) * cv[j];
                const double d = (double)back - (double)sv[j];
                acc += d * d;
            }
            acc += dpp_d<0xb1>(acc);    // quad_perm [1,0,3,2]
            acc += dpp_d<0x4e>(acc);    // quad_perm [2,3,0,1]
            acc += dpp_d<0x141>(acc);   // row_half_mirror
            acc += dpp_d<0x140>(acc);   // row_mirror
            if ((l & 15) == 0) part[l >> 4][u] = acc;
        }
    }
    __syncthreads();
    e[sh * DK + tid] = part[0][tid] + part[1][tid];
}

__device__ __forceinline__ bool sample_ok(int seq, int t, int n_seq, int T) {
    return seq >= 0 && seq < n_seq && t >= 0 && t < T;
}

// One workgroup per block of PW_SAMPLES consecutive samples of the list and
// one head, thread u = key channel.  Consecutive samples of one sequence
// (a run) read overlapping stretches of its decays: the run's stretch is
// staged through LDS PW_STEPS steps at a time, read from memory once, and
// each sample of the run advances its own product and sum over its steps in
// step order, so every result is the one-sample loop's.  A list in any
// other order is still correct (runs of one sample).  PW_SPLIT threads per
// channel take every PW_SPLIT-th sample, so that many chains run at once.
constexpr int PW_SAMPLES = 16;
constexpr int PW_STEPS = 64;
constexpr int PW_SPLIT = 4;   // threads per channel, each taking every PW_SPLIT-th sample
constexpr int PW_THREADS = PW_SPLIT * DK;
__global__ __launch_bounds__(PW_THREADS) void persistence_window_kernel(
    const float *__restrict__ a, int n_seq, int T, int num_heads, int n,
    const int32_t *__restrict__ sample_seq, const int32_t *__restrict__ sample_t, int horizon,
    double *__restrict__ W) {
    __shared__ float stage[PW_STEPS][DK];
    const int u = threadIdx.x & (DK - 1);
    const int part = threadIdx.x / DK;
    const int h = blockIdx.y;
    const int s0 = blockIdx.x * PW_SAMPLES;
    const int cnt = min(PW_SAMPLES, n - s0);
    int seq[PW_SAMPLES], t[PW_SAMPLES], last[PW_SAMPLES];
    double p[PW_SAMPLES], acc[PW_SAMPLES];
#pragma unroll
    for (int i = 0; i < PW_SAMPLES; ++i) {
        seq[i] = -1;
        t[i] = 0;
        last[i] = 0;
        if (i < cnt) {
            seq[i] = sample_seq[s0 + i];
            t[i] = sample_t[s0 + i];
            if (!sample_ok(seq[i], t[i], n_seq, T)) seq[i] = -1;   // out of range: NaN
            else last[i] = min(horizon, T - 1 - t[i]);
        }
        p[i] = 1.0;
        acc[i] = seq[i] >= 0 ? 1.0 : __builtin_nan("");
    }
    for (int i0 = 0; i0 < cnt;) {
        int i1 = i0 + 1;
        if (seq[i0] >= 0)
            while (i1 < cnt && seq[i1] == seq[i0]) ++i1;
        if (seq[i0] >= 0) {
            // the run's steps: from the earliest sample's next step to the
            // latest window end
            int lo = 0x7fffffff, hi = -1;
#pragma unroll
            for (int i = 0; i < PW_SAMPLES; ++i)
                if (i >= i0 && i < i1) {
                    lo = min(lo, t[i] + 1);
                    hi = max(hi, t[i] + last[i]);
                }
            const float *as = a + ((size_t)seq[i0] * T * num_heads + h) * DK + u;  // step 0
            const size_t step = (size_t)num_heads * DK;
            for (int c0 = lo; c0 <= hi; c0 += PW_STEPS) {
                const int nst = min(PW_STEPS, hi - c0 + 1);
                float v[PW_STEPS / PW_SPLIT];
                // the threads of a channel load alternate steps; past the
                // stretch the index repeats its last step, so every load is
                // in range and none sits behind a branch
#pragma unroll
                for (int j = 0; j < PW_STEPS / PW_SPLIT; ++j)
                    v[j] = as[(size_t)(c0 + min(PW_SPLIT * j + part, nst - 1)) * step];
                __syncthreads();   // the previous chunk has been read
#pragma unroll
                for (int j = 0; j < PW_STEPS / PW_SPLIT; ++j) stage[PW_SPLIT * j + part][u] = v[j];
                __syncthreads();
#pragma unroll
                for (int i = 0; i < PW_SAMPLES; ++i)
                    if (i >= i0 && i < i1 && i % PW_SPLIT == part) {
                        const int from = max(c0, t[i] + 1), to = min(c0 + nst - 1, t[i] + last[i]);
                        double pi = p[i], ai = acc[i];
                        int r = from;
                        // eight steps' decays read before the chain takes them
                        for (; r + 8 <= to + 1; r += 8) {
                            float av[8];
#pragma unroll
                            for (int k = 0; k < 8; ++k) av[k] = stage[r - c0 + k][u];
#pragma unroll
                            for (int k = 0; k < 8; ++k) {
                                const double aj = (double)av[k];
                                pi = pi * (aj * aj);
                                ai = ai + pi;
                            }
                        }
                        for (; r <= to; ++r) {
                            const double aj = (double)stage[r - c0][u];
                            pi = pi * (aj * aj);
                            ai = ai + pi;
                        }
                        p[i] = pi;
                        acc[i] = ai;
                    }
            }
        }
        i0 = i1;
    }
#pragma unroll
    for (int i = 0; i < PW_SAMPLES; ++i)
        if (i < cnt && i % PW_SPLIT == part) W[((size_t)(s0 + i) * num_heads + h) * DK + u] = acc[i];
}

// The geometric persistence and the scores: one workgroup per head and block
// of SUM_CH key channels (DK / SUM_CH workgroups per head), SUM_PARTS
// threads per channel.  In each pass the workgroup forms the terms of
// SUM_BATCH samples (thread part p takes samples p, p + SUM_PARTS, ...) into
// one of two LDS buffers, and the channel's first thread adds them to its sum
// in sample order while the others form the next pass's terms in the other
// buffer, so each sum is that of the one-thread loop over the samples.
constexpr int SUM_CH = 16;
constexpr int SUM_PARTS = 64;
constexpr int SUM_THREADS = SUM_CH * SUM_PARTS;
constexpr int SUM_BATCH = 128;
constexpr int SUM_PER = SUM_BATCH / SUM_PARTS;   // terms per thread and pass
static_assert(DK % SUM_CH == 0 && SUM_BATCH % SUM_PARTS == 0, "summation tiling");

__global__ __launch_bounds__(SUM_THREADS) void persistence_geo_kernel(
    const float *__restrict__ a, int n_seq, int T, int num_heads, int n,
    const int32_t *__restrict__ sample_seq, const int32_t *__restrict__ sample_t,
    const double *__restrict__ weight, double tau, double *__restrict__ P) {
    __shared__ double term[2][SUM_BATCH][SUM_CH];
    __shared__ int kind[2][SUM_BATCH];   // 0: skipped (zero weight), 1: used, 2: out of range
    const int ul = threadIdx.x & (SUM_CH - 1);
    const int part = threadIdx.x / SUM_CH;
    const int h = blockIdx.x / (DK / SUM_CH);
    const int u = (blockIdx.x % (DK / SUM_CH)) * SUM_CH + ul;
    double L = 0.0;
    bool bad = false;
    for (int s0 = 0, pass = 0; s0 < n; s0 += SUM_BATCH, pass ^= 1) {
        const int cnt = min(SUM_BATCH, n - s0);
#pragma unroll
        for (int j = 0; j < SUM_PER; ++j) {
            const int i = part + SUM_PARTS * j;
            int kd = 0;
            double v = 0.0;
            if (i < cnt) {
                const int s = s0 + i;
                const double w = weight[s];
                const int seq = sample_seq[s], t = sample_t[s];
                if (w != 0.0) {
                    kd = sample_ok(seq, t, n_seq, T) ? 1 : 2;
                    if (kd == 1)
                        v = w * log((double)a[(((size_t)seq * T + t) * num_heads + h) * DK + u]);
                }
            }
            term[pass][i][ul] = v;
            if (ul == 0) kind[pass][i] = kd;
        }
        // this pass's terms are in; the pass before last has been summed
        // (its buffer is the one written above)
        __syncthreads();
        if (part == 0) {
            for (int i0 = 0; i0 < cnt; i0 += 8) {
                double tv[8];
                int kv[8];
#pragma unroll
                for (int q = 0; q < 8; ++q) {
                    tv[q] = term[pass][min(i0 + q, SUM_BATCH - 1)][ul];
                    kv[q] = i0 + q < cnt ? kind[pass][min(i0 + q, SUM_BATCH - 1)] : 0;
                }
#pragma unroll
                for (int q = 0; q < 8; ++q) {
                    if (kv[q] == 2 && !bad) {
                        L = __builtin_nan("");
                        bad = true;
                    }
                    if (kv[q] == 1 && !bad) L = L + tv[q];
                }
            }
        }
    }
    if (part != 0) return;
    const double ae = exp(L);
    const double gap = 1.0 - ae * ae;
    // fmax would drop a NaN gap (an out-of-range sample); keep it
    P[(size_t)h * DK + u] = gap != gap ? gap : 1.0 / fmax(gap, tau);
}

// Scores: term w_s e_s (times W_s for the window persistence), summed in
// sample order, times P for the geometric one.  The summation tiling above.
__global__ __launch_bounds__(SUM_THREADS) void channel_scores_kernel(
    int n, int num_heads, const double *__restrict__ e, const double *__restrict__ W,
    const double *__restrict__ P, const double *__restrict__ weight, double *__restrict__ C) {
    __shared__ double term[2][SUM_BATCH][SUM_CH];
    const int ul = threadIdx.x & (SUM_CH - 1);
    const int part = threadIdx.x / SUM_CH;
    const int h = blockIdx.x / (DK / SUM_CH);
    const int u = (blockIdx.x % (DK / SUM_CH)) * SUM_CH + ul;
    double acc = 0.0;
    for (int s0 = 0, pass = 0; s0 < n; s0 += SUM_BATCH, pass ^= 1) {
        const int cnt = min(SUM_BATCH, n - s0);
        double ev[SUM_PER], wv[SUM_PER], wt[SUM_PER];
        // past the last sample the index repeats it: no load behind a branch
#pragma unroll
        for (int j = 0; j < SUM_PER; ++j) {
            const int sm = s0 + min(part + SUM_PARTS * j, cnt - 1);
            const size_t idx = ((size_t)sm * num_heads + h) * DK + u;
            ev[j] = e[idx];
            wv[j] = W ? W[idx] : 1.0;
            wt[j] = weight[sm];
        }
#pragma unroll
        for (int j = 0; j < SUM_PER; ++j) {
            double t = wt[j] * ev[j];
            if (W) t = t * wv[j];
            term[pass][part + SUM_PARTS * j][ul] = t;
        }
        // this pass's terms are in; the pass before last has been summed
        // (its buffer is the one written above)
        __syncthreads();
        if (part == 0) {
            for (int i0 = 0; i0 < cnt; i0 += 8) {
                double tv[8];
#pragma unroll
                for (int q = 0; q < 8; ++q) tv[q] = term[pass][min(i0 + q, SUM_BATCH - 1)][ul];
#pragma unroll
                for (int q = 0; q < 8; ++q)
                    if (i0 + q < cnt) acc = acc + tv[q];
            }
        }
    }
    if (part != 0) return;
    if (P) acc = acc * P[(size_t)h * DK + u];
    C[(size_t)h * DK + u] = acc;
}

}  // namespace

hipError_t launch_channel_error(int n, int num_heads, const float *S, const float *smooth,
                                double *e, hipStream_t stream) {
    hipLaunchKernelGGL(channel_error_kernel, dim3((unsigned)(n * num_heads)), dim3(SEL_THREADS),
                       0, stream, S, smooth, num_heads, e);
    return hipGetLastError();
}

hipError_t launch_persistence_window(int n_seq, int T, int num_heads, const float *a, int n,
                                     const int32_t *sample_seq, const int32_t *sample_t,
                                     int horizon, double *W, hipStream_t stream) {
    hipLaunchKernelGGL(persistence_window_kernel,
                       dim3((unsigned)((n + PW_SAMPLES - 1) / PW_SAMPLES), (unsigned)num_heads),
                       dim3(PW_THREADS), 0, stream, a, n_seq, T, num_heads, n, sample_seq,
                       sample_t, horizon, W);
    return hipGetLastError();
}

hipError_t launch_persistence_geometric(int n_seq, int T, int num_heads, const float *a, int n,
                                        const int32_t *sample_seq, const int32_t *sample_t,
                                        const double *weight, double tau, double *P,
                                        hipStream_t stream) {
    hipLaunchKernelGGL(persistence_geo_kernel, dim3((unsigned)(num_heads * (DK / SUM_CH))),
                       dim3(SUM_THREADS), 0,
                       stream, a, n_seq, T, num_heads, n, sample_seq, sample_t, weight, tau, P);
    return hipGetLastError();
}

hipError_t launch_channel_scores(int n, int num_heads, const double *e, const double *W,
                                 const double *P, const double *weight, double *C,
                                 hipStream_t stream) {
    hipLaunchKernelGGL(channel_scores_kernel, dim3((unsigned)(num_heads * (DK / SUM_CH))),
                       dim3(SUM_THREADS), 0,
                       stream, n, num_heads, e, W, P, weight, C);
    return hipGetLastError();
}

}  // namespace qrs
