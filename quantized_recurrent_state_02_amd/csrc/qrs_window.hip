// qrs_window.hip -- per-window quantization on the packed pool ("LeapQuant:
// Efficient Linear Attention with Accurate Recurrent State Quantization",
// section 3.2 and Figure 2): the stored state of a slot stays fixed for a
// window of tokens, each token's update is kept in a small buffer (k and v in
// FP16, beta and the gate in FP32), outputs come from the fixed state and the
// buffered updates, and the token that completes the window writes the
// requantized state.
//
// One 128-thread workgroup per (slot, head), the decode kernels' mapping
// (thread = 8 rows x 16 columns of the FP32 state).  With S_0 the dequantized
// window-start state (stored coordinates) and tokens 1..j of the window,
//   S_j^T q = S_0^T x_0 + sum_t v'_t beta_t (k'_t . x_t),
//   x_j = q',  x_{t-1} = Lambda_t (x_t - beta_t k'_t (k'_t . x_t)),
// which follows from S_t = (I - beta k k^T) Lambda S_{t-1} + beta k v^T
// (HTML of DAMP, section 3.1, Eq.(2)); so a step inside the window costs one
// matrix-vector product over the stored state plus O(j d) vector work, and
// writes only its 528-byte (GDN) / 1,040-byte (KDA) record.  The step that
// completes the window replays the window's updates on the state in
// registers (the recurrence of the decode kernels, token by token), reads
// out, and requantizes into the pool.
//
// Record of token t of slot s, head h, at buffer + ((s H + h) window + t) R:
//   [0, 256) k FP16 [128], [256, 512) v FP16 [128] (model order);
//   GDN (R = 528): [512] beta, [516] alpha (FP32);
//   KDA (R = 784): [512, 768) the decay factors exp(g) FP16 [128], [768] beta.
// The record is the token's update in FP16 (LeapQuant's FP16 update buffer):
// k, v and, for KDA, exp(g) taken in FP64 and rounded once to FP16 (ties to
// even), evaluated when the token is recorded; beta and GDN's alpha stay FP32.
#include "qrs_internal.h"
#include "qrs_window.h"

namespace qrs {

constexpr int WIN_MAX = 32;


namespace {

typedef float v4f __attribute__((ext_vector_type(4)));

// A KDA decay factor as recorded: exp(g) in FP64, rounded once to FP16 (ties
// to even).  The FP64 value is first rounded to FP32 with round-to-odd (the
// nearest-even FP32 value, moved one step toward zero and made odd when it is
// inexact and above), then FP32 -> FP16 rounds to nearest even; with 13 more
// bits in FP32 than in FP16 the two steps equal one correct rounding.
// Returns the FP16 bits.
__device__ __forceinline__ uint32_t decay_f16_bits(float g) {
    const double e = exp((double)g);  // in [0, 1] for g <= 0
    const float t = (float)e;
    uint32_t u = __builtin_bit_cast(uint32_t, t);
    if ((double)t != e) {
        if ((double)t > e) u -= 1u;  // e >= 0, so t > e >= 0 and u >= 1
        u |= 1u;
    }
    return f32_to_f16_bits(__builtin_bit_cast(float, u));
}

// Fields of a record staged in LDS (the record layout, byte offsets).
__device__ __forceinline__ float lds_f16(const uint8_t *base, int byte_off) {
    return f16_bits_to_f32(*reinterpret_cast<const uint16_t *>(base + byte_off));
}
__device__ __forceinline__ float lds_f32(const uint8_t *base, int byte_off) {
    return *reinterpret_cast<const float *>(base + byte_off);
}

// Calls of at most this many requests whose slots sit at different
// positions of their windows run the requests at their window's last token
// first.  Workgroups start in grid order, and a window-end token replays the
// window and lives several times longer than the others: those started last
// would set the end of the launch.  Longer calls keep the batch order.
constexpr int ORDER_MAX = 1024;

// The batch's positions as lane l holds them for ends_first_request:
// positions 16 l .. 16 l + 15 (reads past the batch return zero).  Issued
// before the unit's other loads, so that waiting for them waits for nothing
// else.
struct BatchPositions {
    int v[16];
};
__device__ __forceinline__ BatchPositions load_positions(const int32_t *__restrict__ pos, int n) {
    const int lane = __lane_id();
    const __amdgpu_buffer_rsrc_t pr = make_rsrc(pos, min(n, ORDER_MAX) * 4);
    BatchPositions bp;
#pragma unroll
    for (int j = 0; j < 16; ++j)
        bp.v[j] = (int)__builtin_amdgcn_raw_buffer_load_b32(pr, (16 * lane + j) * 4, 0, 0);
    return bp;
}

// The request that request rank r runs: the stable partition of the batch
// into the requests at position `end` first and the rest after them, each
// part in batch order (positions out of range count with the rest).  Lane l
// holds positions 16 l .. 16 l + 15 (those past the batch are masked off);
// the lanes' counts are prefix-summed from their five bit planes (a count is
// at most 16) with one ballot and one lane count each; the lane whose range
// holds the wanted request finds it among its 16 by halving.  Every wave
// computes it from the same loads, so the result is wave-uniform.
// 1 <= n <= ORDER_MAX.
__device__ __forceinline__ int ends_first_request(const BatchPositions &bp, int n, int end, int r) {
    const int lane = __lane_id();
    const int nv = min(16, max(0, n - 16 * lane));   // this lane's positions in the batch
    const uint32_t valid = (1u << nv) - 1u;
    uint32_t m = 0;   // bit j: position 16 lane + j is at its window's end
#pragma unroll
    for (int j = 0; j < 16; ++j) m |= (bp.v[j] == end ? 1u : 0u) << j;
    m &= valid;
    const int ce = __builtin_popcount(m);
    int pre = 0, total = 0;   // ends before this lane's range, and in the batch
#pragma unroll
    for (int bit = 0; bit < 5; ++bit) {
        const uint64_t bm = __ballot((ce >> bit) & 1);
        pre += (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bm >> 32),
                                              __builtin_amdgcn_mbcnt_lo((uint32_t)bm, 0u))
               << bit;
        total += __popcll(bm) << bit;
    }
    const bool want_end = r < total;
    const uint32_t mk = want_end ? m : (~m & valid);
    const int cnt = want_end ? ce : nv - ce;
    const int before = want_end ? pre : min(16 * lane, n) - pre;
    const int t = (want_end ? r : r - total) - before;   // wanted request's index in this lane's part
    const bool own = t >= 0 && t < cnt;
    // the t-th set bit of mk
    uint32_t mm = mk;
    int k = t, at = 0;
#pragma unroll
    for (int w = 8; w >= 1; w >>= 1) {
        const int c = __builtin_popcount(mm & ((1u << w) - 1u));
        const bool up = k >= c;
        k -= up ? c : 0;
        mm = up ? mm >> w : mm;
        at += up ? w : 0;
    }
    const uint64_t ob = __ballot(own);
    int b = r;
    if (ob != 0ull)
        b = __builtin_amdgcn_readlane(16 * lane + at, (int)__builtin_ctzll(ob));
    return min(b, n - 1);
}

}  // namespace

template <int KIND>
// Held to 168 VGPRs: three waves per SIMD against two at the 218 it took
// unconstrained, 6% faster per token in phase.  The last replayed token
// forms its w and z partial sums in two passes and the store offsets are
// re-derived after the replay, which leaves a few dwords of spills outside
// the per-token work.  One 8 KB partial-sum buffer (not two) keeps the LDS of
// a 16-token GDN window at 19 KB, so six workgroups fit per CU (five for KDA):
// 4% faster per token in phase than with two buffers.
__global__ __launch_bounds__(THREADS) __attribute__((amdgpu_waves_per_eu(3, 3))) void window_kernel(
    PoolView pool, uint8_t *__restrict__ buf, int window, const int32_t *__restrict__ slots,
    const int32_t *__restrict__ pos, int n, const float *__restrict__ q, const float *__restrict__ k,
    const float *__restrict__ v, const float *__restrict__ gate, const float *__restrict__ beta,
    float *__restrict__ o) {
    constexpr int R = window_record_bytes(KIND);
    constexpr int BOFF = KIND == 0 ? 512 : 768;  // beta's byte offset in a record
    // 16-byte pieces of the earlier records that one thread stages (at most
    // WIN_MAX - 1 records precede a token)
    constexpr int NCH = ((WIN_MAX - 1) * (R / 16) + THREADS - 1) / THREADS;
    __shared__ float s_kc[DK];     // current token's k (FP16-rounded), model order
    __shared__ float s_q[DK];      // q, model order
    __shared__ float s_lam[DK];    // KDA: exp(g) of the current token, model order
    __shared__ int s_perm[DK];
    __shared__ float s_x0[DK];     // back-propagated query, stored order
    __shared__ float s_coef[WIN_MAX];
    __shared__ float s_bd[DV];
    __shared__ float s_qk[2];
    __shared__ float4 red[16][DV / 4];  // column partial sums (w or z)
    extern __shared__ __align__(16) uint8_t s_rec[];  // this window's earlier records, (window - 1) * R bytes

    const int tid = threadIdx.x;
    const int H = pool.num_heads;
    const int rank = blockIdx.x / H;
    const int h = blockIdx.x - rank * H;
    // the request of the batch-order position is read with the three
    // probes below and read again only where the partition moves the
    // request; the partition's position loads are the first vector loads, so
    // waiting for them waits for nothing else
    int slot = slots[rank];
    int p = pos[rank];
    int b = rank;
    // the partition only for a batch whose first, middle and last requests
    // are not all at one position (a call with every slot in the same phase
    // keeps the batch order without the scan); every workgroup decides from
    // the same three entries, so all of them take the same order
    const int p_first = pos[0], p_mid = pos[n >> 1], p_last = pos[n - 1];
    if (n <= ORDER_MAX && (p_first != p_mid || p_first != p_last)) {
        b = ends_first_request(load_positions(pos, n), n, window - 1, rank);
        if (b != rank) {
            slot = slots[b];
            p = pos[b];
        }
    }
    const size_t ob = ((size_t)b * H + h) * DK;
    const float k_in = k[ob + tid];
    const float v_in = v[ob + tid];
    const float q_in = q[ob + tid];
    const float beta_c = beta[b * H + h];
    const float alpha_c = KIND == 0 ? gate[b * H + h] : 0.f;
    const float g_c = KIND == 1 ? gate[ob + tid] : 0.f;
    const int uu = b * H + h;   // the unit's output index
    if (slot < 0 || slot >= pool.num_slots || p < 0 || p >= window) {
        o[(size_t)uu * DV + tid] = __builtin_nanf("");
        return;
    }
    const bool boundary = p == window - 1;
    const int cb = tid & 7;
    const int rg = tid >> 3;
    const __amdgpu_buffer_rsrc_t st =
        make_rsrc(pool.base + ((size_t)slot * H + h) * UNIT_BYTES, UNIT_BYTES);
    uint8_t *const recs = buf + ((size_t)slot * H + h) * (size_t)window * R;
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(recs, window * R);
    const __amdgpu_buffer_rsrc_t rr = make_rsrc(recs, p * R);  // the p earlier records only
    const int off_hi = HI_OFF + rg * (DV * 2) + cb * 32;
    const int off_lo = rg * DV + cb * 16;
    const int off_sc = (rg * NGRP + (cb >> 1)) * 4;

    // ---- loads, in the order their results are needed.  All of a thread's
    //      record pieces are issued before any is used (reads past the p
    //      earlier records return zero and touch no memory); the
    //      window-start state is issued last and stays in flight while wave 0
    //      back-propagates the query ----
    U4 part[NCH];
#pragma unroll
    for (int i = 0; i < NCH; ++i) part[i] = buf_load16(rr, 16 * (tid + THREADS * i), 0);
    const float c_t = pool.smooth[h * DV + tid];
    const int perm_t = pool.perm[h * DK + tid];
    // this token's decay of key channel tid as recorded (FP16), KDA
    const uint32_t lam16 = KIND == 1 ? decay_f16_bits(g_c) : 0u;
    const float lam_c = f16_bits_to_f32(lam16);
    U4 hi_raw[2];
    U4 lo_raw[ROWS_PER_THREAD - 1];
    float sc_old[ROWS_PER_THREAD - 1];
    hi_raw[0] = buf_load16(st, off_hi, 0);
    hi_raw[1] = buf_load16(st, off_hi + 16, 0);
#pragma unroll
    for (int r = 1; r < ROWS_PER_THREAD; ++r) {
        lo_raw[r - 1] = buf_load16(st, off_lo, LO_OFF + 2048 * (r - 1));
        sc_old[r - 1] = buf_loadf(st, off_sc + 256 * (r - 1), SC_OFF);
    }
    const int nrec = p * (R / 16);
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
        const int e = tid + THREADS * i;
        if (e < nrec) *reinterpret_cast<U4 *>(s_rec + 16 * e) = part[i];
    }

    // ---- the current token: FP16 k and v, recorded unless it ends the window ----
    const uint32_t k16 = f32_to_f16_bits(k_in);
    const uint32_t v16 = f32_to_f16_bits(v_in);
    if (!boundary) {
        __builtin_amdgcn_raw_buffer_store_b16((uint16_t)k16, rb, p * R + 2 * tid, 0, 0);
        __builtin_amdgcn_raw_buffer_store_b16((uint16_t)v16, rb, p * R + 256 + 2 * tid, 0, 0);
        if (KIND == 1)
            __builtin_amdgcn_raw_buffer_store_b16((uint16_t)lam16, rb, p * R + 512 + 2 * tid, 0, 0);
        if (tid == 0) {
            buf_storef(rb, beta_c, p * R + BOFF, 0);
            if (KIND == 0) buf_storef(rb, alpha_c, p * R + 516, 0);
        }
    }
    s_kc[tid] = f16_bits_to_f32(k16);
    s_q[tid] = q_in;
    s_perm[tid] = perm_t;
    if (KIND == 1) s_lam[tid] = lam_c;
    __syncthreads();

    if (!boundary) {
        // ---- wave 0: back-propagate the query through tokens p, p-1, ..., 0;
        //      the next token's fields are read from LDS ahead of each sum ----
        if (tid < 64) {
            const int i0 = tid, i1 = tid + 64;  // stored rows of this lane
            const int m0 = s_perm[i0], m1 = s_perm[i1];
            float x0 = s_q[m0], x1 = s_q[m1];
            float ka = s_kc[m0], kb = s_kc[m1], bt = beta_c;
            float la = KIND == 0 ? alpha_c : s_lam[m0];
            float lb = KIND == 0 ? alpha_c : s_lam[m1];
            for (int t = p; t >= 0; --t) {
                // token t - 1 (record 0 again at t = 0, where it goes unused)
                const uint8_t *rec = s_rec + (t > 0 ? t - 1 : 0) * R;
                const float nka = lds_f16(rec, 2 * m0), nkb = lds_f16(rec, 2 * m1);
                const float nbt = lds_f32(rec, BOFF);
                const float nla = KIND == 0 ? lds_f32(rec, 516) : lds_f16(rec, 512 + 2 * m0);
                const float nlb = KIND == 0 ? nla : lds_f16(rec, 512 + 2 * m1);
                const float coef = bt * wave_allsum(__builtin_fmaf(ka, x0, kb * x1));
                if (tid == 0) s_coef[t] = coef;
                x0 = la * (x0 - coef * ka);
                x1 = lb * (x1 - coef * kb);
                ka = nka;
                kb = nkb;
                bt = nbt;
                la = nla;
                lb = nlb;
            }
            s_x0[i0] = x0;
            s_x0[i1] = x1;
        }
        __syncthreads();
        // ---- z = S_0^T x_0 straight from the packed rows: FP16 rows as
        //      x_0 * f32(h), INT8 rows as (x_0 s) * code ----
        float xr0 = s_x0[rg];
        float xs[ROWS_PER_THREAD - 1];
#pragma unroll
        for (int r = 1; r < ROWS_PER_THREAD; ++r) xs[r - 1] = s_x0[rg + 16 * r] * sc_old[r - 1];
        const uint32_t hw[8] = {hi_raw[0].x, hi_raw[0].y, hi_raw[0].z, hi_raw[0].w,
                                hi_raw[1].x, hi_raw[1].y, hi_raw[1].z, hi_raw[1].w};
#pragma unroll
        for (int c4 = 0; c4 < 4; ++c4) {
            float pz[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int c = 4 * c4 + j;
                float az = (c & 1) ? mul_f16hi(xr0, hw[c >> 1]) : mul_f16lo(xr0, hw[c >> 1]);
#pragma unroll
                for (int r = 1; r < ROWS_PER_THREAD; ++r) {
                    const uint32_t lw[4] = {lo_raw[r - 1].x, lo_raw[r - 1].y, lo_raw[r - 1].z,
                                            lo_raw[r - 1].w};
                    az = __builtin_fmaf(xs[r - 1], sext_byte_to_f32(lw[c >> 2], c & 3), az);
                }
                pz[j] = az;
            }
            red[rg][cb * 4 + c4] = make_float4(pz[0], pz[1], pz[2], pz[3]);
        }
        __syncthreads();
        const float *rz = reinterpret_cast<const float *>(red);
        float z = 0.f;
#pragma unroll
        for (int g = 0; g < 16; ++g) z += rz[g * DV + tid];
        // the buffered writes: o = c z + sum_t coef_t v_t, since v'_t = v_t / c
        float acc = s_coef[p] * f16_bits_to_f32(v16);
        for (int t = 0; t < p; ++t)
            acc = __builtin_fmaf(s_coef[t], lds_f16(s_rec + t * R, 256 + 2 * tid), acc);
        __builtin_nontemporal_store(__builtin_fmaf(c_t, z, acc), o + (size_t)uu * DV + tid);
        return;
    }

    // ---- dequantize (no decay: decays come with each token) ----
    const float vc = f16_bits_to_f32(v16) / c_t;  // v' of the current token, column tid
    // The state as accumulators of v_mfma_f32_4x4x1f32 (16 blocks of 4 lanes;
    // lane l's element i is A of lane 4 (l / 4) + i times B of lane l): the 4
    // lanes of a block share the row group rg and hold columns 16 cb + c for
    // cb = 4 j .. 4 j + 3, so block accumulator X[h][c] of a lane is its own
    // rows 4 h .. 4 h + 3 at its own column 16 cb + c.  The rank-1 write of a
    // token is then one 4x4x1 product per accumulator, with A = k at row
    // rg + 16 (4 h + (cb & 3)) and B = beta delta at the lane's column.
    v4f X[2][COLS_PER_THREAD];
#define XV(r, c) X[(r) >> 2][c][(r) & 3]
    {
        const uint32_t hw[8] = {hi_raw[0].x, hi_raw[0].y, hi_raw[0].z, hi_raw[0].w,
                                hi_raw[1].x, hi_raw[1].y, hi_raw[1].z, hi_raw[1].w};
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            XV(0, 2 * c) = f16_bits_to_f32(hw[c] & 0xffffu);
            XV(0, 2 * c + 1) = f16_bits_to_f32(hw[c] >> 16);
        }
    }
#pragma unroll
    for (int r = 1; r < ROWS_PER_THREAD; ++r) {
        const uint32_t lw[4] = {lo_raw[r - 1].x, lo_raw[r - 1].y, lo_raw[r - 1].z,
                                lo_raw[r - 1].w};
#pragma unroll
        for (int c = 0; c < 16; ++c) XV(r, c) = sc_old[r - 1] * sext_byte_to_f32(lw[c >> 2], c & 3);
    }

    // ---- the window's last token: replay tokens 0..p on the state ----
    {
        const float pqk = wave_allsum(s_q[tid] * f16_bits_to_f32(k16));
        if ((tid & 63) == 0) s_qk[tid >> 6] = pqk;
    }
    // GDN: every row decays by the same alpha, so the state is kept as gam X
    // with gam the product of the window's alphas so far: a token's decay is
    // one multiply instead of one per value; w = sum (k gam) X and the write
    // adds (k / gam) (beta delta).  When gam falls below 2^-60 (a zero alpha
    // included), and at the window's last token, it is folded back into X, so
    // the state leaves the loop unscaled (a separate pass over it after the
    // loop made the compiler spill).  KDA decays its rows in place.
    float gam = 1.f;
    for (int t = 0; t <= p; ++t) {
        float kr[ROWS_PER_THREAD], dr[ROWS_PER_THREAD], ka[2], bt, vp;
        // The model channels of this lane's two rank-1 write operands, read
        // each token from an opaque copy of the thread id: held across the
        // replay they were spilled and reloaded with a full memory wait.
        int tid2 = tid;
        asm volatile("" : "+v"(tid2));
        const int ma[2] = {s_perm[(tid2 >> 3) + 16 * (tid2 & 3)],
                           s_perm[(tid2 >> 3) + 16 * (4 + (tid2 & 3))]};
        if (t < p) {
            const uint8_t *rec = s_rec + t * R;
            vp = lds_f16(rec, 256 + 2 * tid) / c_t;
            bt = lds_f32(rec, BOFF);
            const float at = KIND == 0 ? lds_f32(rec, 516) : 0.f;
#pragma unroll
            for (int r = 0; r < ROWS_PER_THREAD; ++r) {
                const int m = s_perm[rg + 16 * r];
                kr[r] = lds_f16(rec, 2 * m);
                dr[r] = KIND == 0 ? at : lds_f16(rec, 512 + 2 * m);
            }
            ka[0] = lds_f16(rec, 2 * ma[0]);
            ka[1] = lds_f16(rec, 2 * ma[1]);
        } else {
            vp = vc;
            bt = beta_c;
#pragma unroll
            for (int r = 0; r < ROWS_PER_THREAD; ++r) {
                const int m = s_perm[rg + 16 * r];
                kr[r] = s_kc[m];
                dr[r] = KIND == 0 ? alpha_c : s_lam[m];
            }
            ka[0] = s_kc[ma[0]];
            ka[1] = s_kc[ma[1]];
        }
        if (KIND == 0) {
            gam *= dr[0];
            if (gam < 0x1p-60f || t == p) {  // the same for every thread
#pragma unroll
                for (int hh = 0; hh < 2; ++hh)
#pragma unroll
                    for (int c = 0; c < COLS_PER_THREAD; ++c) X[hh][c] *= gam;
                gam = 1.f;
            }
            const float ginv = __builtin_amdgcn_rcpf(gam);
#pragma unroll
            for (int r = 0; r < ROWS_PER_THREAD; ++r) kr[r] *= gam;
            ka[0] *= ginv;
            ka[1] *= ginv;
        } else {
#pragma unroll
            for (int r = 0; r < ROWS_PER_THREAD; ++r)
#pragma unroll
                for (int c = 0; c < COLS_PER_THREAD; ++c) XV(r, c) = dr[r] * XV(r, c);
        }
        // w partials; at the window's last token the z partials follow in the
        // same buffer once every thread has read the w sums (one more barrier
        // on that token only, one 8 KB buffer instead of two)
#pragma unroll
        for (int c4 = 0; c4 < 4; ++c4) {
            float pw[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int c = 4 * c4 + j;
                float aw = kr[0] * XV(0, c);
#pragma unroll
                for (int r = 1; r < ROWS_PER_THREAD; ++r) aw = __builtin_fmaf(kr[r], XV(r, c), aw);
                pw[j] = aw;
            }
            red[rg][cb * 4 + c4] = make_float4(pw[0], pw[1], pw[2], pw[3]);
        }
        __syncthreads();
        float bd;
        {
            const float *rw = reinterpret_cast<const float *>(red);
            float w = 0.f;
#pragma unroll
            for (int g = 0; g < 16; ++g) w += rw[g * DV + tid];
            bd = bt * (vp - w);
            s_bd[tid] = bd;
        }
        __syncthreads();
        if (t == p) {
            float qr[ROWS_PER_THREAD];
#pragma unroll
            for (int r = 0; r < ROWS_PER_THREAD; ++r)
                qr[r] = s_q[s_perm[rg + 16 * r]] * (KIND == 0 ? gam : 1.f);
#pragma unroll
            for (int c4 = 0; c4 < 4; ++c4) {
                float pz[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int c = 4 * c4 + j;
                    float az = qr[0] * XV(0, c);
#pragma unroll
                    for (int r = 1; r < ROWS_PER_THREAD; ++r)
                        az = __builtin_fmaf(qr[r], XV(r, c), az);
                    pz[j] = az;
                }
                red[rg][cb * 4 + c4] = make_float4(pz[0], pz[1], pz[2], pz[3]);
            }
            __syncthreads();
            const float *rz = reinterpret_cast<const float *>(red);
            float zz = 0.f;
#pragma unroll
            for (int g = 0; g < 16; ++g) zz += rz[g * DV + tid];
            const float qk = s_qk[0] + s_qk[1];
            __builtin_nontemporal_store(c_t * __builtin_fmaf(qk, bd, zz), o + (size_t)uu * DV + tid);
        }
        float bdc[COLS_PER_THREAD];
#pragma unroll
        for (int c = 0; c < COLS_PER_THREAD; ++c) bdc[c] = s_bd[cb * 16 + c];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
            for (int c = 0; c < COLS_PER_THREAD; ++c)
                X[hh][c] = __builtin_amdgcn_mfma_f32_4x4x1f32(ka[hh], bdc[c], X[hh][c], 0, 0, 0);
    }
    // ---- requantize the window-end state into the pool (offsets re-derived
    //      from an opaque copy of the thread id rather than held across the
    //      replay) ----
    int tid2 = threadIdx.x;
    asm volatile("" : "+v"(tid2));
    const int cb2 = tid2 & 7;
    const int rg2 = tid2 >> 3;
    const int off_hi2 = HI_OFF + rg2 * (DV * 2) + cb2 * 32;
    const int off_lo2 = rg2 * DV + cb2 * 16;
    const int off_sc2 = (rg2 * NGRP + (cb2 >> 1)) * 4;
    {
        uint32_t hw[8];
#pragma unroll
        for (int c = 0; c < 8; ++c) hw[c] = pack_f16x2(XV(0, 2 * c), XV(0, 2 * c + 1));
        buf_store16_cached(st, U4{hw[0], hw[1], hw[2], hw[3]}, off_hi2, 0);
        buf_store16_cached(st, U4{hw[4], hw[5], hw[6], hw[7]}, off_hi2 + 16, 0);
    }
#pragma unroll
    for (int r = 1; r < ROWS_PER_THREAD; ++r) {
        float xr[COLS_PER_THREAD];
        float amax = 0.f;
#pragma unroll
        for (int c = 0; c < COLS_PER_THREAD; ++c) {
            xr[c] = XV(r, c);
            amax = fmaxf(amax, fabsf(xr[c]));
        }
        amax = pair_max(amax);
        const float s = group_scale(amax);
        const double rinv = pack_reciprocal(s);
        U4 cw;
        cw.x = quant4(xr[0], xr[1], xr[2], xr[3], rinv);
        cw.y = quant4(xr[4], xr[5], xr[6], xr[7], rinv);
        cw.z = quant4(xr[8], xr[9], xr[10], xr[11], rinv);
        cw.w = quant4(xr[12], xr[13], xr[14], xr[15], rinv);
        buf_store16(st, cw, off_lo2, LO_OFF + 2048 * (r - 1));
        if ((cb2 & 1) == 0) buf_storef(st, s, off_sc2 + 256 * (r - 1), SC_OFF);
    }
#undef XV
}

hipError_t launch_window(int kind, const PoolView &pool, uint8_t *buf, int window,
                         const int32_t *slots, const int32_t *pos, int n, const float *q,
                         const float *k, const float *v, const float *gate, const float *beta,
                         float *o, hipStream_t stream) {
    dim3 grid((unsigned)(n * pool.num_heads)), block(THREADS);
    // at most window - 1 earlier records are staged (the current token's is not)
    const size_t lds = (size_t)(window - 1) * window_record_bytes(kind);
    if (kind == 0)
        hipLaunchKernelGGL(window_kernel<0>, grid, block, lds, stream, pool, buf, window, slots,
                           pos, n, q, k, v, gate, beta, o);
    else
        hipLaunchKernelGGL(window_kernel<1>, grid, block, lds, stream, pool, buf, window, slots,
                           pos, n, q, k, v, gate, beta, o);
    return hipGetLastError();
}

}  // namespace qrs
