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
// multiplied by them (v2 notes, section 2.7).  The readout uses
// z + (q'.k') beta delta = T^T q' (the FP32 state of this step before
// requantization), so both column reductions run in one pass before the
// update.
//
// Cost model (gfx950): every byte of the unit is read once and written once
// with 128-bit buffer accesses (non-temporal, except the FP16-row stores, see
// below).  The VALU work is about 10.5 instructions per state value: convert,
// scale, two reduction FMAs, the update FMA, half an absmax, a
// four-instruction exact quantizer whose last step also packs the code byte,
// and per-row / per-unit overheads.  Six workgroups fit per CU (168 VGPRs,
// three waves per SIMD); the grid is one workgroup per unit, so the hardware
// refills CUs as units finish.  On MI355X the step time follows the VALU
// count (a kernel with a cheaper, inexact quantizer ran 7% faster) and the
// residency (three waves per SIMD against two: 3-4%), while changes to the
// memory side alone did not move it: workgroups that prefetch a second unit,
// one wave per column half over a layout with contiguous column halves, and
// single 16-byte scale accesses all measured the same or slower.
#include <atomic>

#include "qrs_decode_half.h"
#include "qrs_hadamard.h"

namespace qrs {

// KIND 0: GDN (gate = alpha [n][H]); KIND 1: KDA (gate = g [n][H][128]).
// CODEC 0: the INT8 tier (symmetric codes, FP32 scale); CODEC 1: the first
// revision's tier (block-32 Hadamard, asymmetric UINT8, FP16 scale and zero
// point; qrs_hadamard.h), read and written at the same offsets.
// IO 0: q, k, v, o in FP32; IO 1: in bf16 (gates and beta stay FP32).
// Workgroup i < nwhole handles unit i (slot b = i / hc, head h0 + i % hc);
// operands and outputs are indexed [n][H] as for the full head range.  The
// INT8 tier may end its grid with half-unit workgroups (i >= nwhole, two per
// unit, qrs_decode_half.h) for units nwhole .. units - 1: they live about
// half as long, so the launch drains sooner (the launcher below).
template <int CODEC>
struct DecodeOccupancy {
    static constexpr int waves = CODEC == 0 ? 3 : 2;
};

// LDS of a whole-unit workgroup (the kernel's own arrays, lent to the body).
struct DecodeLds {
    float *s_k, *s_q, *s_dec;          // [DK]
    float *s_bd, *s_vp;                // [DV]
    float *s_kraw, *s_qraw, *s_graw;   // [DK]
    float *s_qk;                       // [2]
    float4 (*red_w)[DV / 4];           // [16][DV / 4]
    float4 (*red_z)[DV / 4];
};

// Staggered start of the first generation (the workgroups resident at
// launch; first_gen = 0 when the grid is too small to benefit): the j-th
// workgroup placed on each CU waits j x 2048 cycles (~0.85 us), so the first
// workgroups get their state sooner and compute while the others load,
// instead of all loading and then all computing at once.  pos is the
// workgroup's launch position.
__device__ __forceinline__ void stagger_start(int pos, int first_gen, int n_cus) {
    if (pos < first_gen) {
        const int j = pos / n_cus;
        for (int i = 0; i < j; ++i) __builtin_amdgcn_s_sleep(32);
    }
}

// One workgroup's share of a decode call: workgroup bid < nwhole owns unit
// bid, a later one half of a unit of the half-unit tail.
template <int KIND, int CODEC, int IO>
__device__ __forceinline__ void decode_unit(
    PoolView pool, const int32_t *__restrict__ slots, int bid, int first_gen, int n_cus, int h0,
    int hc, int nwhole, int units, const void *__restrict__ q, const void *__restrict__ k,
    const void *__restrict__ v, const float *__restrict__ gate, const float *__restrict__ beta,
    void *__restrict__ o, const DecodeLds &L) {
    float *const s_k = L.s_k, *const s_q = L.s_q, *const s_dec = L.s_dec;
    float *const s_bd = L.s_bd, *const s_vp = L.s_vp;
    float *const s_kraw = L.s_kraw, *const s_qraw = L.s_qraw, *const s_graw = L.s_graw;
    float *const s_qk = L.s_qk;
    float4 (*const red_w)[DV / 4] = L.red_w;
    float4 (*const red_z)[DV / 4] = L.red_z;

    if (CODEC == 0 && bid >= nwhole) {
        const HalfLds HL{s_k,    s_q,    s_dec, s_bd,         s_vp,        s_kraw,
                         s_qraw, s_graw, s_qk,  &red_w[0][0], &red_z[0][0]};
        decode_half_unit<KIND, IO>(pool, slots, units, h0, hc, bid - nwhole, nwhole, q, k, v, gate,
                                   beta, o, HL);
        return;
    }
    stagger_start(bid, first_gen, n_cus);
    // Raised wave priority until the state loads are issued: a workgroup
    // that starts while the SIMD's other waves run long VALU stretches gets
    // its loads out first (KDA 0.2 us per step faster, GDN within noise; the
    // same change slowed the FP32-state and per-window kernels).
    __builtin_amdgcn_s_setprio(3);
    const int tid = threadIdx.x;
    const int H = pool.num_heads;
    const unsigned ubid = (unsigned)bid;
    const int b = ubid / hc;
    const int h = h0 + (ubid - b * hc);
    const int uu = b * H + h;
    const int slot = slots[b];
    if (slot < 0 || slot >= pool.num_slots) {
        st_stream<IO>(o, (size_t)uu * DV + tid, __builtin_nanf(""));
        return;
    }
    const int cb = tid & 7;
    const int rg = tid >> 3;
    const __amdgpu_buffer_rsrc_t st =
        make_rsrc(pool.base + ((size_t)slot * H + h) * UNIT_BYTES, UNIT_BYTES);
    // Byte offsets of this thread's pieces: FP16 row rg (32 B at off_hi); INT8
    // row rg + 16 (r - 1) (16 B at off_lo + LO_OFF + 2048 (r - 1)) and its
    // scale (off_sc + SC_OFF + 256 (r - 1)).
    const int off_hi = HI_OFF + rg * (DV * 2) + cb * 32;
    const int off_lo = rg * DV + cb * 16;
    const int off_sc = (rg * NGRP + (cb >> 1)) * 4;

    // ---- operand loads: thread t loads element t of k, q (KDA: g) and v in
    //      model order, pi[h][t] and c[h][t].  None depends on another, so
    //      they and the state loads behind them leave at once; the gather
    //      through pi runs in LDS afterwards.  (A gather from global memory
    //      needs pi first, and with one in-order load counter that wait would
    //      hold back the state loads by a full memory round trip.) ----
    const size_t ob = (size_t)uu * DK;
    const int src = pool.perm[h * DK + tid];
    const float k_m = ld_stream<IO>(k, ob + tid);
    const float q_m = ld_stream<IO>(q, ob + tid);
    float g_m = 0.f;
    if (KIND == 1) g_m = __builtin_nontemporal_load(gate + ob + tid);
    const float c_t = pool.smooth[h * DV + tid];
    const float v_m = ld_stream<IO>(v, ob + tid);
    __builtin_amdgcn_sched_barrier(0);

    // ---- state loads (the long-latency part) ----
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
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_setprio(0);

    // ---- gather through pi: thread t takes stored row t ----
    const float beta_u = beta[uu];
    s_kraw[tid] = k_m;
    s_qraw[tid] = q_m;
    if (KIND == 1) s_graw[tid] = g_m;
    s_vp[tid] = v_m / c_t;  // v' = D_c^{-1} v, read back by this thread after the reductions
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
            x[0][2 * c] = mul_f16lo(dr[0], hw[c]);
            x[0][2 * c + 1] = mul_f16hi(dr[0], hw[c]);
        }
    }
    // first revision's tier: the integer inverse transform when every group
    // of the wave is in its exact range (a wave-uniform choice), else FP64
    bool v1_int = false;
    if (CODEC == 1) {
        bool ok = true;
#pragma unroll
        for (int r = 1; r < ROWS_PER_THREAD; ++r) {
            const uint32_t m = __builtin_bit_cast(uint32_t, sc_old[r - 1]);
            ok &= u8_group_exact(f16_bits_to_f32(m & 0xffffu), f16_bits_to_f32(m >> 16));
        }
        v1_int = __builtin_amdgcn_ballot_w64(!ok) == 0;
    }
    // The row loop is written out once per path, so that the wave-uniform
    // choice is one branch and each path one basic block (a choice inside
    // the loop cut the rows apart: v1 tier 120.3 -> 117.7 us per step).
    auto row_codes = [&](int r, uint32_t (&lw)[4]) {
        lw[0] = lo_raw[r - 1].x;
        lw[1] = lo_raw[r - 1].y;
        lw[2] = lo_raw[r - 1].z;
        lw[3] = lo_raw[r - 1].w;
    };
    if (CODEC == 0) {
#pragma unroll
        for (int r = 1; r < ROWS_PER_THREAD; ++r) {
            uint32_t lw[4];
            row_codes(r, lw);
            const float a = dr[r] * sc_old[r - 1];
#pragma unroll
            for (int c = 0; c < 16; ++c) x[r][c] = a * sext_byte_to_f32(lw[c >> 2], c & 3);
        }
    } else if (v1_int) {
#pragma unroll
        for (int r = 1; r < ROWS_PER_THREAD; ++r) {
            uint32_t lw[4];
            row_codes(r, lw);
            const uint32_t m = __builtin_bit_cast(uint32_t, sc_old[r - 1]);
            const float sh = f16_bits_to_f32(m & 0xffffu), zh = f16_bits_to_f32(m >> 16);
            hadamard32_pair_codes(lw, sh, zh, (cb & 1) != 0, x[r]);
#pragma unroll
            for (int c = 0; c < 16; ++c) x[r][c] = dr[r] * x[r][c];
        }
    } else {
#pragma unroll
        for (int r = 1; r < ROWS_PER_THREAD; ++r) {
            uint32_t lw[4];
            row_codes(r, lw);
            // reconstruct in the transformed domain, transform back, then decay
            const uint32_t m = __builtin_bit_cast(uint32_t, sc_old[r - 1]);
            const float sh = f16_bits_to_f32(m & 0xffffu), zh = f16_bits_to_f32(m >> 16);
#pragma unroll
            for (int c = 0; c < 16; ++c) x[r][c] = u8_dequant(lw[c >> 2], c & 3, sh, zh);
            hadamard32_pair(x[r], (cb & 1) != 0);
#pragma unroll
            for (int c = 0; c < 16; ++c) x[r][c] = dr[r] * x[r][c];
        }
    }

    // ---- partial column reductions over this thread's 8 rows, written to
    //      LDS four columns at a time ----
#pragma unroll
    for (int c4 = 0; c4 < 4; ++c4) {
        float pw[4], pz[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int c = 4 * c4 + j;
            float aw = kr[0] * x[0][c];
            float az = qr[0] * x[0][c];
#pragma unroll
            for (int r = 1; r < ROWS_PER_THREAD; ++r) {
                aw = __builtin_fmaf(kr[r], x[r][c], aw);
                az = __builtin_fmaf(qr[r], x[r][c], az);
            }
            pw[j] = aw;
            pz[j] = az;
        }
        red_w[rg][cb * 4 + c4] = make_float4(pw[0], pw[1], pw[2], pw[3]);
        red_z[rg][cb * 4 + c4] = make_float4(pz[0], pz[1], pz[2], pz[3]);
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
        const float delta = s_vp[tid] - w;
        const float bd = beta_u * delta;
        const float qk = s_qk[0] + s_qk[1];
        st_stream<IO>(o, (size_t)uu * DV + tid, c_t * __builtin_fmaf(qk, bd, z));
        s_bd[tid] = bd;
    }
    __syncthreads();

    // Re-derive this thread's offsets from an opaque copy of the thread id:
    // a few integer instructions, where keeping them live across the
    // reductions made the compiler spill at the 168-VGPR limit.
    int tid2 = tid;
    asm volatile("" : "+v"(tid2));
    const int cb2 = tid2 & 7;
    const int rg2 = tid2 >> 3;
    const int off_hi2 = HI_OFF + rg2 * (DV * 2) + cb2 * 32;
    const int off_lo2 = rg2 * DV + cb2 * 16;
    // The group's scale (or v1 metadata) is written by the even lane of the
    // pair; the odd lane's offset lies past the unit's buffer range, so its
    // store is dropped, with no branch around each row's store.
    const int off_sc2 = (cb2 & 1) == 0 ? (rg2 * NGRP + (cb2 >> 1)) * 4 : kDropOffset;
    float bdc[COLS_PER_THREAD];
#pragma unroll
    for (int c = 0; c < COLS_PER_THREAD; ++c) bdc[c] = s_bd[cb2 * 16 + c];

    // ---- rank-1 write, requantize, store: FP16 row (r = 0) ----
    {
        uint32_t hw[8];
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            const float e0 = __builtin_fmaf(kr[0], bdc[2 * c], x[0][2 * c]);
            const float e1 = __builtin_fmaf(kr[0], bdc[2 * c + 1], x[0][2 * c + 1]);
            hw[c] = pack_f16x2(e0, e1);
        }
        // Each store instruction covers only every other 16 B of the FP16
        // rows, so these two use the default cache policy and meet in L2;
        // as non-temporal stores the half-filled lines each reached HBM as
        // separate writes (+12% write traffic).
        buf_store16_cached(st, U4{hw[0], hw[1], hw[2], hw[3]}, off_hi2, 0);
        buf_store16_cached(st, U4{hw[4], hw[5], hw[6], hw[7]}, off_hi2 + 16, 0);
    }
    // ---- INT8 rows ----
#pragma unroll
    for (int r = 1; r < ROWS_PER_THREAD; ++r) {
        U4 cw;
        float meta;
        if (CODEC == 0) {
            float amax = 0.f;
#pragma unroll
            for (int c = 0; c < COLS_PER_THREAD; ++c) {
                x[r][c] = __builtin_fmaf(kr[r], bdc[c], x[r][c]);
                amax = fmaxf(amax, fabsf(x[r][c]));
            }
            amax = pair_max(amax);
            const float s = group_scale(amax);
            const double rinv = pack_reciprocal(s);
            cw.x = quant4(x[r][0], x[r][1], x[r][2], x[r][3], rinv);
            cw.y = quant4(x[r][4], x[r][5], x[r][6], x[r][7], rinv);
            cw.z = quant4(x[r][8], x[r][9], x[r][10], x[r][11], rinv);
            cw.w = quant4(x[r][12], x[r][13], x[r][14], x[r][15], rinv);
            meta = s;
        } else {
#pragma unroll
            for (int c = 0; c < COLS_PER_THREAD; ++c)
                x[r][c] = __builtin_fmaf(kr[r], bdc[c], x[r][c]);
            hadamard32_pair(x[r], (cb2 & 1) != 0);
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
            meta = __builtin_bit_cast(float, pr.meta);
        }
        buf_store16(st, cw, off_lo2, LO_OFF + 2048 * (r - 1));
        buf_storef(st, meta, off_sc2 + 256 * (r - 1), SC_OFF);
    }
}

// The INT8 tier is held to 168 VGPRs, three waves per SIMD (six units per
// CU); at 180 VGPRs it ran two waves per SIMD and was 3-4% slower.  The
// first revision's tier needs about 200 VGPRs for its transforms and stays
// at two waves per SIMD.
template <int KIND, int CODEC, int IO>
__global__ __launch_bounds__(THREADS) __attribute__((
    amdgpu_waves_per_eu(DecodeOccupancy<CODEC>::waves, DecodeOccupancy<CODEC>::waves))) void
decode_packed_kernel(PoolView pool, const int32_t *__restrict__ slots, int first_gen, int n_cus,
                     int h0, int hc, int nwhole, int units, const void *__restrict__ q,
                     const void *__restrict__ k, const void *__restrict__ v,
                     const float *__restrict__ gate, const float *__restrict__ beta,
                     void *__restrict__ o) {
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
    const DecodeLds L{s_k, s_q, s_dec, s_bd, s_vp, s_kraw, s_qraw, s_graw, s_qk, red_w, red_z};
    decode_unit<KIND, CODEC, IO>(pool, slots, (int)blockIdx.x, first_gen, n_cus, h0, hc, nwhole,
                                 units, q, k, v, gate, beta, o, L);
}


// XCD-aware order for a run of n whole units, g to a slot.  Workgroups go to
// the 8 XCDs round-robin by launch position, and each XCD has its own L2 and
// address-translation caches.  Position 8j + x (on XCD x, up to a constant
// shift) takes head j mod g of slot (j / g) * 8 + x, so each XCD works through
// whole slots, every eighth one, and touches an eighth of the slots in flight
// instead of all of them.  Positions past the last full round of 8 slots keep
// their own unit.  A bijection on [0, n).
__device__ __forceinline__ int slot_per_xcd(int pos, int n, int g) {
    const int full = ((n / g) & ~7) * g;
    if (pos >= full) return pos;
    const int x = pos & 7, j = pos >> 3;
    return ((j / g) * 8 + x) * g + j % g;
}

// One launch for a GDN call and a KDA call on disjoint slots of one INT8-tier
// pool, all heads, FP32 operands: the two request groups of a model with GDN
// and KDA layers, or of a pool shared by such models.  Workgroups [0, ug) run
// the GDN units, the rest the KDA units (with their half-unit tail at the end
// of the grid), so the pair pays the launch ramp and drain once.  The whole
// units of each group run in slot_per_xcd order: with the scattered slots of
// a shared pool this took 2.6% off a 248 us step (16,384 units per group,
// random slots of a 2.65 GB pool) and 1.5% with sorted slots, while on the
// contiguous slots of a single call the same order cost 0.7-1.4%, which is
// why decode_packed_kernel keeps head-major order.  Each unit's arithmetic is
// that of decode_packed_kernel, so the results are those of the two calls.
__global__ __launch_bounds__(THREADS) __attribute__((amdgpu_waves_per_eu(3, 3))) void
decode_pair_kernel(PoolView pool, int first_gen, int n_cus, int ug, int uk, int nwhole_k,
                   const int32_t *__restrict__ slots_g, const float *__restrict__ q_g,
                   const float *__restrict__ k_g, const float *__restrict__ v_g,
                   const float *__restrict__ alpha, const float *__restrict__ beta_g,
                   float *__restrict__ o_g, const int32_t *__restrict__ slots_k,
                   const float *__restrict__ q_k, const float *__restrict__ k_k,
                   const float *__restrict__ v_k, const float *__restrict__ g,
                   const float *__restrict__ beta_k, float *__restrict__ o_k) {
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
    const DecodeLds L{s_k, s_q, s_dec, s_bd, s_vp, s_kraw, s_qraw, s_graw, s_qk, red_w, red_z};
    const int H = pool.num_heads;
    const int i = (int)blockIdx.x;
    stagger_start(i, first_gen, n_cus);
    if (i < ug)
        decode_unit<0, 0, 0>(pool, slots_g, slot_per_xcd(i, ug, H), 0, n_cus, 0, H, ug, ug, q_g,
                             k_g, v_g, alpha, beta_g, o_g, L);
    else
        decode_unit<1, 0, 0>(pool, slots_k, slot_per_xcd(i - ug, nwhole_k, H), 0, n_cus, 0, H,
                             nwhole_k, uk, q_k, k_k, v_k, g, beta_k, o_k, L);
}

// Launcher (host): one workgroup per (slot, head) unit of heads [h0, h0 + hc).
// The number of workgroups resident at launch (occupancy x CUs) is queried
// once per device and kernel.
// The cache is per device; host threads launching concurrently may both
// query it first, which is harmless (they store the same values).
template <typename Kernel>
static void residency(Kernel kernel, std::atomic<int> (&s_per)[16], std::atomic<int> (&s_cus)[16],
                      int *per_cu, int *cus) {
    int dev = 0;
    *per_cu = 0;
    *cus = 1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 16) return;
    int p = s_per[dev].load(std::memory_order_acquire);
    int c = s_cus[dev].load(std::memory_order_relaxed);
    if (p == 0) {
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&p, kernel, THREADS, 0) != hipSuccess ||
            hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            c <= 0 || p <= 0)
            return;
        s_cus[dev].store(c, std::memory_order_relaxed);
        s_per[dev].store(p, std::memory_order_release);
    }
    *per_cu = p;
    *cus = c;
}
template <int K, int C, int I>
static void decode_residency(int *per_cu, int *cus) {
    static std::atomic<int> s_per[16], s_cus[16];
    residency(decode_packed_kernel<K, C, I>, s_per, s_cus, per_cu, cus);
}
// The stagger pays off only when the grid holds more than two generations of
// resident workgroups.  The half-unit tail (INT8 tier, half_tail set): when
// the grid holds at least 4/3 of a generation, its last resident / 8 units (a
// multiple of 8) run as value-column halves.  On MI355X (6 x 256 resident)
// this took 0.5-0.7 us off a 60.5 us step at batch 256 x 32 heads for GDN and
// KDA on two boxes (tails of 192, 256 and 384 units within noise of each
// other; 512 gained less, 1,536 lost 1.5 us), 1.4 us off 21.5 at batch 64 and
// off 27.7 at batch 96; at batch 56 (1,792 units) it cost 0.2 us and at
// exactly one generation (batch 48) 1.0 us.
#define QRS_DECODE_CASE(K, C, I)                                                                  \
    if (kind == K && codec == C && io == I) {                                                     \
        int per_cu = 0, cus = 1;                                                                  \
        decode_residency<K, C, I>(&per_cu, &cus);                                                 \
        const int units = n * hc, resident = per_cu * cus;                                        \
        const bool big = units > 2 * resident;                                                    \
        const int first_gen = big ? resident : 0;                                                 \
        const bool tailed =                                                                       \
            C == 0 && half_tail && 3 * (int64_t)units >= 4 * (int64_t)resident;                   \
        const int tail = tailed ? (resident / 8) & ~7 : 0;                                        \
        const int nwhole = units - tail;                                                          \
        dim3 grid((unsigned)(nwhole + 16 * ((tail + 7) / 8))), block(THREADS);                    \
        hipLaunchKernelGGL((decode_packed_kernel<K, C, I>), grid, block, 0, stream, pool, slots,  \
                           first_gen, cus, h0, hc, nwhole, units, q, k, v, gate, beta, o);        \
        return hipGetLastError();                                                                 \
    }
hipError_t launch_decode_packed(int kind, int codec, int io, const PoolView &pool,
                                const int32_t *slots, int n, int h0, int hc, const void *q,
                                const void *k, const void *v, const float *gate, const float *beta,
                                void *o, bool half_tail, hipStream_t stream) {
    QRS_DECODE_CASE(0, 0, 0)
    QRS_DECODE_CASE(1, 0, 0)
    QRS_DECODE_CASE(0, 1, 0)
    QRS_DECODE_CASE(1, 1, 0)
    QRS_DECODE_CASE(0, 0, 1)
    QRS_DECODE_CASE(1, 0, 1)
    QRS_DECODE_CASE(0, 1, 1)
    QRS_DECODE_CASE(1, 1, 1)
    return hipErrorInvalidValue;
}
#undef QRS_DECODE_CASE

// The pair launch: the stagger on the first generation, the half-unit tail on
// the KDA units at the end of the grid, with the same rules as a single call
// over ug + uk units.
hipError_t launch_decode_pair(const PoolView &pool, const int32_t *slots_g, int n_g,
                              const float *q_g, const float *k_g, const float *v_g,
                              const float *alpha, const float *beta_g, float *o_g,
                              const int32_t *slots_k, int n_k, const float *q_k, const float *k_k,
                              const float *v_k, const float *g, const float *beta_k, float *o_k,
                              bool half_tail, hipStream_t stream) {
    static std::atomic<int> s_per[16], s_cus[16];
    int per_cu = 0, cus = 1;
    residency(decode_pair_kernel, s_per, s_cus, &per_cu, &cus);
    const int H = pool.num_heads;
    const int ug = n_g * H, uk = n_k * H, resident = per_cu * cus;
    const bool big = ug + uk > 2 * resident;
    const int first_gen = big ? resident : 0;
    const bool tailed = half_tail && 3 * ((int64_t)ug + uk) >= 4 * (int64_t)resident;
    int tail = tailed ? (resident / 8) & ~7 : 0;
    if (tail > uk / 2) tail = 0;
    const int nwhole_k = uk - tail;
    dim3 grid((unsigned)(ug + nwhole_k + 16 * ((tail + 7) / 8))), block(THREADS);
    hipLaunchKernelGGL(decode_pair_kernel, grid, block, 0, stream, pool, first_gen, cus, ug, uk,
                       nwhole_k, slots_g, q_g, k_g, v_g, alpha, beta_g, o_g, slots_k, q_k, k_k,
                       v_k, g, beta_k, o_k);
    return hipGetLastError();
}

}  // namespace qrs
