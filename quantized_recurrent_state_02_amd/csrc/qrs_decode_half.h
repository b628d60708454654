// qrs_decode_half.h -- the fused compressed-state decode step (GDN and KDA,
// INT8 tier) for one 64-column half of the value axis of a (slot, head) unit,
// run by one workgroup: the body of decode_half_kernel (qrs_decode_half.hip,
// two workgroups per unit for grids too small to fill the GPU) and of the
// half-unit workgroups at the end of decode_packed_kernel's grid
// (qrs_decode.hip), which shorten the drain at the end of a large launch.
// Internal to the library.
//
// Every part of the update stays within a value column: the column sums
// w = Tbar^T k' and z = Tbar^T q', delta = v' - w, the readout, the rank-1
// write k' (beta delta)^T and the 32-value requantization groups (DAMP arXiv
// HTML, section 3.1 Eq.(1); v2 reading notes, section 2.2, Eqs.(5)-(6)).  So a
// half needs only the full k' and q' (and KDA's decays), its own 64 columns of
// v, c and the state, and no exchange with the other half.  The arithmetic
// is that of decode_packed_kernel (qrs_decode.hip) on half the columns: the
// same dequantization, column sums in the same per-thread-then-LDS order,
// update and exact quantizer, so the two kernels give the same bits.
//
// Why: a workgroup that owns a whole unit lives about 9 us on an otherwise
// empty GPU (its loads, then 1,347 VALU instructions per wave at one wave per
// SIMD); when the grid is a fraction of one generation of resident workgroups,
// that lifetime is the step time.  Halves double the workgroups and halve the
// work of each: on MI355X, 7.6 against 9.2 us per step at 512 units (batch 16
// x 32 heads), 9.6 against 10.3 at 768, equal at 1,024, and slower above (the
// whole-unit kernel issues 16-byte code loads, shares each group's scale
// between two lanes, and spends fewer instructions per value on the per-row
// scale), so the library picks this kernel below 1,024 units per call.
//
// Thread mapping (128 threads, two wave64s, half hf of unit u):
//   cb = tid & 7   column block: columns 64 hf + 8 cb .. + 7
//   rg = tid >> 3  row group 0..15: stored rows rg + 16 r, r = 0..7
// Row r = 0 is an FP16 row for every thread.  A 32-value scale group spans
// the 4 lanes tid & ~3 .. tid | 3 (one DPP quad).
#pragma once

#include "qrs_internal.h"

namespace qrs {

// A buffer offset past every resource range here: a store at it is dropped.
constexpr int kDropOffset = 0x40000000;

namespace half_unit {

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// 8-byte code pieces, non-temporal like the rest of the state traffic.  (A
// half reads and writes 64 of a row's 128 code bytes; with the default cache
// policy, so that the sibling half would meet each line in L2, the dirty lines
// were written back only at the kernel's end: 13.9 against 11.5 us per step
// at 1,024 units.)
__device__ __forceinline__ u32x2 buf_load8(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
    return __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, kStream);
}
__device__ __forceinline__ void buf_store8(__amdgpu_buffer_rsrc_t r, u32x2 d, int voff, int soff) {
    __builtin_amdgcn_raw_buffer_store_b64(d, r, voff, soff, kStream);
}

// max over the 4 lanes of a DPP quad for a >= 0 (non-negative floats order
// like their bit patterns): quad_perm [1,0,3,2], then [2,3,0,1].
__device__ __forceinline__ float quad_max(float a) {
    uint32_t d = __builtin_bit_cast(uint32_t, a);
    uint32_t e;
    asm("s_nop 1\n\tv_max_u32_dpp %0, %1, %1 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf "
        "bound_ctrl:1"
        : "=v"(e)
        : "v"(d));
    asm("s_nop 1\n\tv_max_u32_dpp %0, %1, %1 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf "
        "bound_ctrl:1"
        : "=v"(d)
        : "v"(e));
    return __builtin_bit_cast(float, d);
}

constexpr int HCOLS = DV / 2;   // columns per half
constexpr int HCPT = 8;         // columns per thread

}  // namespace half_unit

// LDS of a half-unit workgroup.  The whole-unit kernel lends its own arrays
// (each at least as large) to the halves at the end of its grid.
struct HalfLds {
    float *s_k, *s_q, *s_dec;          // [DK]
    float *s_bd, *s_vp;                // [HCOLS]
    float *s_kraw, *s_qraw, *s_graw;   // [DK]
    float *s_qk;                       // [2]
    float4 *red_w, *red_z;             // [16][HCOLS / 4]
};

// Half hf = (i >> 3) & 1 of unit ubase + (i >> 4) * 8 + (i & 7), for i the
// workgroup's index among the half-unit workgroups: the two halves of a unit
// are 8 workgroups apart, so with workgroups dealt round-robin to the 8 XCDs
// they run on the same XCD and read k, q and pi through one L2.
// KIND 0: GDN (gate = alpha [n][H]); KIND 1: KDA (gate = g [n][H][128]).
// IO 0: q, k, v, o in FP32; IO 1: in bf16 (gates and beta stay FP32).
template <int KIND, int IO>
__device__ __forceinline__ void decode_half_unit(
    PoolView pool, const int32_t *__restrict__ slots, int units, int h0, int hc, int i, int ubase,
    const void *__restrict__ q, const void *__restrict__ k, const void *__restrict__ v,
    const float *__restrict__ gate, const float *__restrict__ beta, void *__restrict__ o,
    const HalfLds &L) {
    using namespace half_unit;
    float *const s_k = L.s_k, *const s_q = L.s_q, *const s_dec = L.s_dec;
    float *const s_bd = L.s_bd, *const s_vp = L.s_vp;
    float *const s_kraw = L.s_kraw, *const s_qraw = L.s_qraw, *const s_graw = L.s_graw;
    float *const s_qk = L.s_qk;
    float4 (*red_w)[HCOLS / 4] = reinterpret_cast<float4 (*)[HCOLS / 4]>(L.red_w);
    float4 (*red_z)[HCOLS / 4] = reinterpret_cast<float4 (*)[HCOLS / 4]>(L.red_z);

    const int ui = ubase + (i >> 4) * 8 + (i & 7);  // unit index in the call
    const int hf = (i >> 3) & 1;                    // value-column half
    if (ui >= units) return;  // the grid is rounded up to whole groups of 16
    const int tid = threadIdx.x;
    const int H = pool.num_heads;
    const int b = ui / hc;
    const int h = h0 + (ui - b * hc);
    const int uu = b * H + h;
    const int col0 = HCOLS * hf;
    const int slot = slots[b];
    if (slot < 0 || slot >= pool.num_slots) {
        if (tid < HCOLS) st_stream<IO>(o, (size_t)uu * DV + col0 + tid, __builtin_nanf(""));
        return;
    }
    const int cb = tid & 7;
    const int rg = tid >> 3;
    const __amdgpu_buffer_rsrc_t st =
        make_rsrc(pool.base + ((size_t)slot * H + h) * UNIT_BYTES, UNIT_BYTES);
    // this thread's pieces: FP16 row rg (16 B), INT8 rows rg + 16 r (8 B each)
    // and their group scales (group 2 hf + (cb >> 2) of the row)
    const int off_hi = HI_OFF + rg * (DV * 2) + (col0 + HCPT * cb) * 2;
    const int off_lo = rg * DV + col0 + HCPT * cb;
    const int off_sc = (rg * NGRP + 2 * hf + (cb >> 2)) * 4;

    // ---- operand loads (model order; the gather through pi runs in LDS) ----
    const size_t ob = (size_t)uu * DK;
    const int src = pool.perm[h * DK + tid];
    const float k_m = ld_stream<IO>(k, ob + tid);
    const float q_m = ld_stream<IO>(q, ob + tid);
    float g_m = 0.f;
    if (KIND == 1) g_m = __builtin_nontemporal_load(gate + ob + tid);
    const int vc = tid & (HCOLS - 1);
    const float c_t = pool.smooth[h * DV + col0 + vc];
    const float v_m = ld_stream<IO>(v, ob + col0 + vc);
    __builtin_amdgcn_sched_barrier(0);

    // ---- state loads ----
    const U4 hi_raw = buf_load16(st, off_hi, 0);
    u32x2 lo_raw[ROWS_PER_THREAD - 1];
    float sc_old[ROWS_PER_THREAD - 1];
#pragma unroll
    for (int r = 1; r < ROWS_PER_THREAD; ++r) {
        lo_raw[r - 1] = buf_load8(st, off_lo, LO_OFF + 2048 * (r - 1));
        sc_old[r - 1] = buf_loadf(st, off_sc + 256 * (r - 1), SC_OFF);
    }
    __builtin_amdgcn_sched_barrier(0);
    // v is used by the first 64 threads only; this keeps its load where it
    // is, ahead of the state loads, instead of inside that branch behind them
    // (where its wait was a wait for every state load)
    float v_keep = v_m;
    asm volatile("" : "+v"(v_keep));

    // ---- gather through pi ----
    const float beta_u = beta[uu];
    s_kraw[tid] = k_m;
    s_qraw[tid] = q_m;
    if (KIND == 1) s_graw[tid] = g_m;
    if (tid < HCOLS) s_vp[tid] = v_keep / c_t;
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

    // ---- dequantize + decay ----
    float x[ROWS_PER_THREAD][HCPT];
    {
        const uint32_t hw[4] = {hi_raw.x, hi_raw.y, hi_raw.z, hi_raw.w};
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            x[0][2 * c] = mul_f16lo(dr[0], hw[c]);
            x[0][2 * c + 1] = mul_f16hi(dr[0], hw[c]);
        }
    }
#pragma unroll
    for (int r = 1; r < ROWS_PER_THREAD; ++r) {
        const uint32_t lw[2] = {lo_raw[r - 1].x, lo_raw[r - 1].y};
        const float a = dr[r] * sc_old[r - 1];
#pragma unroll
        for (int c = 0; c < HCPT; ++c) x[r][c] = a * sext_byte_to_f32(lw[c >> 2], c & 3);
    }

    // ---- partial column sums over this thread's 8 rows ----
#pragma unroll
    for (int c4 = 0; c4 < 2; ++c4) {
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
        red_w[rg][cb * 2 + c4] = make_float4(pw[0], pw[1], pw[2], pw[3]);
        red_z[rg][cb * 2 + c4] = make_float4(pz[0], pz[1], pz[2], pz[3]);
    }
    __syncthreads();

    // ---- wave 0 finishes the half's 64 columns: delta, readout ----
    if (tid < HCOLS) {
        const float *rw = reinterpret_cast<const float *>(red_w);
        const float *rz = reinterpret_cast<const float *>(red_z);
        float w = 0.f, z = 0.f;
#pragma unroll
        for (int g = 0; g < 16; ++g) {
            w += rw[g * HCOLS + tid];
            z += rz[g * HCOLS + tid];
        }
        const float delta = s_vp[tid] - w;
        const float bd = beta_u * delta;
        const float qk = s_qk[0] + s_qk[1];
        st_stream<IO>(o, (size_t)uu * DV + col0 + tid, c_t * __builtin_fmaf(qk, bd, z));
        s_bd[tid] = bd;
    }
    __syncthreads();

    int tid2 = tid;
    asm volatile("" : "+v"(tid2));
    const int cb2 = tid2 & 7;
    const int rg2 = tid2 >> 3;
    const int off_hi2 = HI_OFF + rg2 * (DV * 2) + (col0 + HCPT * cb2) * 2;
    const int off_lo2 = rg2 * DV + col0 + HCPT * cb2;
    const int off_sc2 = (cb2 & 3) == 0 ? (rg2 * NGRP + 2 * hf + (cb2 >> 2)) * 4 : kDropOffset;
    float bdc[HCPT];
#pragma unroll
    for (int c = 0; c < HCPT; ++c) bdc[c] = s_bd[cb2 * HCPT + c];

    // ---- rank-1 write, requantize, store: FP16 row (a half's 8 lanes of a
    //      row write one whole 128-byte line) ----
    {
        uint32_t hw[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const float e0 = __builtin_fmaf(kr[0], bdc[2 * c], x[0][2 * c]);
            const float e1 = __builtin_fmaf(kr[0], bdc[2 * c + 1], x[0][2 * c + 1]);
            hw[c] = pack_f16x2(e0, e1);
        }
        buf_store16(st, U4{hw[0], hw[1], hw[2], hw[3]}, off_hi2, 0);
    }
    // ---- INT8 rows ----
#pragma unroll
    for (int r = 1; r < ROWS_PER_THREAD; ++r) {
        float amax = 0.f;
#pragma unroll
        for (int c = 0; c < HCPT; ++c) {
            x[r][c] = __builtin_fmaf(kr[r], bdc[c], x[r][c]);
            amax = fmaxf(amax, fabsf(x[r][c]));
        }
        amax = quad_max(amax);
        const float s = group_scale(amax);
        const double rinv = pack_reciprocal(s);
        u32x2 cw;
        cw.x = quant4(x[r][0], x[r][1], x[r][2], x[r][3], rinv);
        cw.y = quant4(x[r][4], x[r][5], x[r][6], x[r][7], rinv);
        buf_store8(st, cw, off_lo2, LO_OFF + 2048 * (r - 1));
        buf_storef(st, s, off_sc2 + 256 * (r - 1), SC_OFF);
    }
}

}  // namespace qrs
