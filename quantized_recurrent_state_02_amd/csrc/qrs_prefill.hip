// qrs_prefill.hip -- chunked prefill that writes the compressed state, GDN gating.
//
// Prefill runs the FP32 recurrence inside each chunk and writes the chunk-final
// state into the same packed cache the decode kernel uses; the next chunk and
// later decode steps read that compressed state (DAMP arXiv HTML, Appendix A.5
// "Prefill path"; v2 reading notes, section 2.2).  The pages give no chunk
// algebra, so the one used here is derived from the delta form of the update
// (HTML section 3.1, Eq.(1)) in stored coordinates (v2 notes, section 2.7).
//
// Within a chunk of C tokens starting from state S0 (GDN: Lambda_t = alpha_t I),
// let g_t = alpha_1 ... alpha_t (g_0 = 1) and r(t, i) = g_t / g_i.  With
// delta_t = beta_t (v'_t - alpha_t S_{t-1}^T k'_t) the update is
// S_t = alpha_t S_{t-1} + k'_t delta_t^T, so
//     S_t     = g_t S0 + sum_{i<=t} r(t, i) k'_i delta_i^T
//     delta_t = beta_t (v'_t - g_t S0^T k'_t - sum_{i<t} r(t, i) (k'_i . k'_t) delta_i).
// In matrix form over the chunk (rows = tokens), with M[t][i] = r(t,i) k'_t.k'_i
// for i < t:
//     (I + B M) Delta = B (V - Gamma K S0)       (unit lower triangular)
//     O     = Gamma Q S0 + (L o Q K^T) Delta,     L[t][i] = r(t, i) for i <= t
//     S_C   = g_C S0 + K^T diag(r(C, t)) Delta.
// (The same Delta as U - W S0 with (I + B M) [W | U] = B [Gamma K | V]; the
// start state is known when the chunk begins, so the solve needs only the
// d_v right-hand-side columns of V - Gamma K S0.)
// Decay ratios are taken from FP64 prefix sums of log(alpha) (a chunk product
// of alphas underflows FP32); a zero alpha makes every ratio across it zero.
//
// Launch: one 256-thread workgroup (four wave64) per (sequence, head); chunks
// run in order.  Per chunk the waves share K, Q, V and the two 64x64 masked
// Gram tiles in LDS; wave w owns value columns [32w, 32w + 32) of S0, Y,
// Delta and O, which stay in registers in the accumulator layout of
// v_mfma_f32_16x16x4f32 (lane l holds column l & 15 of rows 4 (l >> 4) + r of
// each 16x16 tile).  That layout feeds the next contraction's B operand
// directly when the contraction index inside each 16-block is taken in the
// order 4 (l >> 4) + j at step j.  Every contraction runs on FP32 MFMA; the
// unit lower triangular solve goes block by block (16 tokens): the four
// diagonal blocks are inverted by forward substitution (one lane per column,
// all four blocks at once), then each wave applies the inverses and the
// updates of the later blocks to its columns on the matrix cores.  At
// each chunk end the state is requantized through an LDS copy of the packed
// unit, stored with 16-byte writes, and dequantized back into registers (the
// same values a reload of the stored unit gives).  A wave's 32 columns of a
// row are exactly one 32-value group, held by the 16 lanes of a DPP row (two
// values per lane), so a group's scale, or the block-32 transform and
// extremes of the INT8+Hadamard tier, never leave the wave.
#include <atomic>
#include <cstddef>

#include "qrs_hadamard.h"
#include "qrs_internal.h"

namespace qrs {

namespace {

typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int PT = 256;     // threads per workgroup
constexpr int CT = 64;      // tokens per tile (chunks <= 64 are zero-padded)
constexpr int LDK = 132;    // row stride (floats) of the [64][128] LDS tiles
constexpr int LDM = 68;     // row stride of the [64][64] Gram tile
constexpr int LDI = 20;     // row stride of the inverted diagonal blocks

struct PrefillSmem {
    float K[CT * LDK];   // k' (stored key order)
    float Q[CT * LDK];   // q'; at chunk end, the packed unit being written
    float VU[CT * LDK];  // v' = v / c, then U = T V in place
    float W[CT * LDK];   // A_qk = inclusive-lower decayed Q K^T ([64][LDM]) during a chunk
    float M[CT * LDM];   // strict-lower decayed K K^T
    double lg[CT];       // prefix sum of log(alpha) over the non-zero alphas
    int zi[CT];          // last token <= t with alpha = 0 (-1 if none)
    float gam[CT];       // g_t
    float rc[CT];        // r(C, t): decay from token t to the chunk end
    float bet[CT];
    int inv[DK];         // stored row of each model key channel (inverse of pi)
    float Dinv[CT * LDI];  // block d, row t, column j at (16 d + t) LDI + j: (I + B M)_dd^-1 B_d
};
static_assert(sizeof(PrefillSmem) <= 160 * 1024, "fits the 160 KB LDS of a gfx950 CU");
static_assert(CT * LDM <= CT * LDK, "A_qk fits in the W tile");
static_assert(offsetof(PrefillSmem, W) == offsetof(PrefillSmem, VU) + sizeof(float) * CT * LDK &&
                  KLO * LDK <= 2 * CT * LDK,
              "the chunk-end FP32 rows fit in VU and W");

__device__ __forceinline__ v4f mfma4(float a, float b, v4f c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ v4f lds4(const float *p) { return *reinterpret_cast<const v4f *>(p); }

// r(t, i) = prod_{j=i+1..t} alpha_j for i < t inside the tile.
__device__ __forceinline__ float ratio(const PrefillSmem &s, int t, int i) {
    if (s.zi[t] > i) return 0.f;
    return expf((float)(s.lg[t] - s.lg[i]));
}

// max(m, m of the lane that the DPP control CTRL names, inside the lane's
// 16-lane row) for m the bits of a non-negative float (such floats order
// like their bit patterns): one DPP-modified v_max_u32, with no
// canonicalization of the operands as a float maximum would need.
template <int CTRL>
__device__ __forceinline__ uint32_t row_max_step(uint32_t m) {
    const uint32_t o = (uint32_t)__builtin_amdgcn_mov_dpp((int)m, CTRL, 0xf, 0xf, true);
    return m > o ? m : o;
}

// One step of the decay-prefix scans: la += la of the DPP source lane (0.0
// where the lane has none), z = max(z, z of that lane) (-1 where none).
template <int CTRL, int ROWS>
__device__ __forceinline__ void scan_step(double &la, int &z) {
    const uint64_t b = __builtin_bit_cast(uint64_t, la);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)b, CTRL, ROWS, 0xf, false);
    const uint32_t hi =
        (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(b >> 32), CTRL, ROWS, 0xf, false);
    const int zo = __builtin_amdgcn_update_dpp(-1, z, CTRL, ROWS, 0xf, false);
    la += __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
    z = max(z, zo);
}

// a / b from y = RN(1/b): q = RN(a y) is within one ulp of a / b, the
// residual a - b q is exact in one FMA, and RN(q + r y) is the correctly
// rounded quotient (Markstein's theorem) unless a y or the residual falls
// below the normal range, where it is within an ulp of it.  Three
// instructions in place of the IEEE divide's ten; y is formed once per
// column.
__device__ __forceinline__ float div_by_recip(float a, float b, float y) {
    const float q = a * y;
    const float r = __builtin_fmaf(-b, q, a);
    return __builtin_fmaf(r, y, q);
}

// One input element at byte offset off of a buffer (zero outside its range);
// bf16 widens exactly to FP32.
template <int IN_BF16>
__device__ __forceinline__ float ld_buf(__amdgpu_buffer_rsrc_t r, int off) {
    if (IN_BF16) {
        const uint16_t bits = __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, kStream);
        return __builtin_bit_cast(float, (uint32_t)bits << 16);
    }
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, kStream));
}

// The masked, decayed tile: element (t, i) = r(t, i) acc for i < t (STRICT)
// or i <= t, zero elsewhere; r as ratio() gives it.  Branch-free, with the
// lane's log-prefix loads issued together: the lane's column i and its four
// rows t.
template <bool STRICT>
__device__ __forceinline__ void gram_store(const PrefillSmem &s, float *dst, v4f acc, int tb,
                                           int sb, int l16, int g) {
    const int i = 16 * sb + l16;
    const double li = s.lg[i];
    float e[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) e[r] = expf((float)(s.lg[16 * tb + 4 * g + r] - li));
    // all four are evaluated on every lane (no branch around each exp)
    asm volatile("" : "+v"(e[0]), "+v"(e[1]), "+v"(e[2]), "+v"(e[3]));
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int t = 16 * tb + 4 * g + r;
        const bool keep = STRICT ? (i < t) : (i <= t);
        const float rt = s.zi[t] > i ? 0.f : e[r];   // ratio(s, t, i)
        dst[t * LDM + i] = keep ? rt * acc[r] : 0.f;
    }
}

// 16x16 tile of the masked Gram matrix  A[t][i] = r(t, i) * (X_t . K_i)  for
// i < t (STRICT) or i <= t, zero elsewhere, rows t in [16 tb, +16), columns i
// in [16 sb, +16); X = K or Q from LDS.  Written to dst (row stride LDM).
template <bool STRICT>
__device__ __forceinline__ void gram_tile(PrefillSmem &s, const float *X, float *dst, int tb,
                                          int sb, int l16, int g) {
    v4f acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < 8; ++kb) {
        const v4f a = lds4(X + (16 * tb + l16) * LDK + 16 * kb + 4 * g);
        const v4f b = lds4(s.K + (16 * sb + l16) * LDK + 16 * kb + 4 * g);
        acc = mfma4(a.x, b.x, acc);
        acc = mfma4(a.y, b.y, acc);
        acc = mfma4(a.z, b.z, acc);
        acc = mfma4(a.w, b.w, acc);
    }
    gram_store<STRICT>(s, dst, acc, tb, sb, l16, g);
}

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// Eight LDS values that are exact bf16 numbers (bf16 inputs widened to FP32:
// the low 16 bits are zero) as the bf16 operand of one MFMA: the high half of
// each, two per v_perm.
__device__ __forceinline__ bf16x8 to_bf16x8(v4f lo, v4f hi) {
    typedef uint32_t u32x4_ __attribute__((ext_vector_type(4)));
    const auto b = [](float x) { return __builtin_bit_cast(uint32_t, x); };
    const u32x4_ w = {__builtin_amdgcn_perm(b(lo.y), b(lo.x), 0x07060302u),
                      __builtin_amdgcn_perm(b(lo.w), b(lo.z), 0x07060302u),
                      __builtin_amdgcn_perm(b(hi.y), b(hi.x), 0x07060302u),
                      __builtin_amdgcn_perm(b(hi.w), b(hi.z), 0x07060302u)};
    return __builtin_bit_cast(bf16x8, w);
}

// gram_tile for bf16 inputs: the same masked tile from the same LDS rows, on
// bf16 matrix cores (v_mfma_f32_16x16x32_bf16: lane l supplies row l & 15 and
// the 8 contraction indices 8 (l >> 4) .. + 7 of each operand; the result has
// the layout of the FP32 16x16x4 product).  Products of bf16 numbers are exact
// in FP32 and accumulate in FP32, so the tile differs from the FP32 matrix
// cores' only by the order of the FP32 accumulation; 4 instructions per tile
// instead of 32.
template <bool STRICT>
__device__ __forceinline__ void gram_tile_bf16(PrefillSmem &s, const float *X, float *dst, int tb,
                                               int sb, int l16, int g) {
    v4f acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
        const float *xa = X + (16 * tb + l16) * LDK + 32 * kk + 8 * g;
        const float *kb = s.K + (16 * sb + l16) * LDK + 32 * kk + 8 * g;
        const bf16x8 a = to_bf16x8(lds4(xa), lds4(xa + 4));
        const bf16x8 b = to_bf16x8(lds4(kb), lds4(kb + 4));
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
    }
    gram_store<STRICT>(s, dst, acc, tb, sb, l16, g);
}

}  // namespace

// FMT: QRS_FMT_FP32 (0), QRS_FMT_I8F16 (1) or QRS_FMT_U8H16 (2) pool; IN_BF16:
// q, k, v in bf16.
template <int FMT, int IN_BF16>
__global__ __launch_bounds__(PT) void prefill_kernel(PoolView pool, const int32_t *__restrict__ slots,
                                                     int T, int chunk, const void *__restrict__ q,
                                                     const void *__restrict__ k,
                                                     const void *__restrict__ v,
                                                     const float *__restrict__ alpha,
                                                     const float *__restrict__ beta,
                                                     float *__restrict__ o, int init_from_pool) {
    extern __shared__ __align__(16) uint8_t smem_raw[];
    PrefillSmem &s = *reinterpret_cast<PrefillSmem *>(smem_raw);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = tid >> 6;  // wave: value columns [32 w, 32 w + 32)
    const int l16 = lane & 15;
    const int g = lane >> 4;
    const int H = pool.num_heads;
    const int uu = blockIdx.x;  // b * H + h
    const int b = uu / H;
    const int h = uu - b * H;
    const int slot = slots[b];
    const size_t unit_bytes = FMT != 0 ? (size_t)UNIT_BYTES : (size_t)F32_UNIT_BYTES;

    if (slot < 0 || slot >= pool.num_slots) {
        for (int e = tid; e < T * DV; e += PT) {
            const int t = e >> 7, j = e & (DV - 1);
            o[(((size_t)b * T + t) * H + h) * DV + j] = __builtin_nanf("");
        }
        return;
    }
    uint8_t *unit = pool.base + ((size_t)slot * H + h) * unit_bytes;
    const int in_col = tid & (DK - 1);  // column this thread owns in the LDS-only phases
    if (tid < DK) s.inv[pool.perm[h * DK + tid]] = tid;
    __syncthreads();
    float c_out[2];
    c_out[0] = pool.smooth[h * DV + 32 * w + l16];
    c_out[1] = pool.smooth[h * DV + 32 * w + 16 + l16];

    // ---- initial state, in the accumulator layout: S[rb][cb][r] holds row
    //      16 rb + 4 g + r, column 32 w + 16 cb + l16 ----
    v4f S[8][2];
#pragma unroll
    for (int rb = 0; rb < 8; ++rb)
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) S[rb][cb] = v4f{0.f, 0.f, 0.f, 0.f};
    if (init_from_pool) {
        if (FMT != 0) {
            uint8_t *stg = reinterpret_cast<uint8_t *>(s.Q);
            const __amdgpu_buffer_rsrc_t ru = make_rsrc(unit, UNIT_BYTES);
            U4 part[(UNIT_BYTES / 16 + PT - 1) / PT];
#pragma unroll
            for (int i = 0; i < (UNIT_BYTES / 16 + PT - 1) / PT; ++i)
                part[i] = buf_load16(ru, (tid + PT * i) * 16, 0);   // past the unit: zeros
#pragma unroll
            for (int i = 0; i < (UNIT_BYTES / 16 + PT - 1) / PT; ++i)
                if (tid + PT * i < UNIT_BYTES / 16) reinterpret_cast<U4 *>(stg)[tid + PT * i] = part[i];
            __syncthreads();
#pragma unroll
            for (int rb = 0; rb < 8; ++rb)
#pragma unroll
                for (int cb = 0; cb < 2; ++cb)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int row = 16 * rb + 4 * g + r, col = 32 * w + 16 * cb + l16;
                        if (rb == 0) {
                            S[rb][cb][r] = f16_bits_to_f32(
                                reinterpret_cast<const uint16_t *>(stg + HI_OFF)[row * DV + col]);
                        } else if (FMT == 1) {
                            const int lr = row - KHI;
                            const float sc = reinterpret_cast<const float *>(stg + SC_OFF)[lr * NGRP + w];
                            S[rb][cb][r] =
                                sc * (float)reinterpret_cast<const int8_t *>(stg + LO_OFF)[lr * DV + col];
                        } else {
                            // transformed-domain value s16 (code - z16); the
                            // inverse transform follows once both halves are in
                            const int lr = row - KHI;
                            const uint32_t m = reinterpret_cast<const uint32_t *>(stg + SC_OFF)[lr * NGRP + w];
                            const uint32_t cw = reinterpret_cast<const uint8_t *>(stg + LO_OFF)[lr * DV + col];
                            S[rb][cb][r] = u8_dequant(cw, 0, f16_bits_to_f32(m & 0xffffu),
                                                      f16_bits_to_f32(m >> 16));
                        }
                    }
            if (FMT == 2) {
#pragma unroll
                for (int rb = 1; rb < 8; ++rb)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        float x0 = S[rb][0][r], x1 = S[rb][1][r];
                        hadamard32_row(x0, x1, l16);
                        S[rb][0][r] = x0;
                        S[rb][1][r] = x1;
                    }
            }
            __syncthreads();
        } else {
            const float *u = reinterpret_cast<const float *>(unit);
#pragma unroll
            for (int rb = 0; rb < 8; ++rb)
#pragma unroll
                for (int cb = 0; cb < 2; ++cb)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        S[rb][cb][r] = u[(16 * rb + 4 * g + r) * DV + 32 * w + 16 * cb + l16];
        }
    }

    const int nchunks = (T + chunk - 1) / chunk;
    // One chunk's inputs in registers, read as 16-byte pieces of token rows
    // in model order: thread tid holds model columns [lc, lc + VPL) of tokens
    // lt + RPP j.  pi is applied when k and q are written to LDS (stored row
    // inv[c] of model channel c), and v is divided by c there.  Wave 0's lane
    // t also holds alpha and beta of token t.  Each input is read through a
    // buffer resource that ends at the chunk's last real token, so rows
    // t >= ceff read as zero (and alpha as 1).
    constexpr int ESZ = IN_BF16 ? 2 : 4;
    constexpr int VPL = 16 / ESZ;        // values per 16-byte piece
    constexpr int LPR = DK / VPL;        // pieces per token row
    constexpr int RPP = PT / LPR;        // token rows per pass of the workgroup
    constexpr int NLD = CT / RPP;        // pieces per thread per input
    // lc, lt and the per-thread pi / c entries are re-derived where they are
    // used from an opaque copy of the thread id: held across the chunk loop
    // they were spilled and reloaded every chunk (first revision's tier).
    auto piece_col = [&]() {
        int t2 = tid;
        asm volatile("" : "+v"(t2));
        return (t2 % LPR) * VPL;
    };
    auto piece_row = [&]() {
        int t2 = tid;
        asm volatile("" : "+v"(t2));
        return t2 / LPR;
    };
    U4 kr4[NLD], qr4[NLD], vr4[NLD];
    float a_in = 1.f, b_in = 0.f;
    // Part 0: k and the gates; part 1: q; part 2: v.  The parts are issued
    // at different points of the previous chunk.
    auto load_part = [&](int ch, int part) {
        const int t0 = ch * chunk;
        const int ceff = min(chunk, T - t0);
        const size_t row0 = ((size_t)b * T + t0) * H + h;         // token t0 of (b, h)
        const int rstride = H * DK * ESZ;                         // bytes between tokens
        const int bytes = (ceff - 1) * rstride + DK * ESZ;
        const void *src = part == 0 ? k : part == 1 ? q : v;
        const __amdgpu_buffer_rsrc_t rs = make_rsrc((const uint8_t *)src + row0 * DK * ESZ, bytes);
        U4 *dst = part == 0 ? kr4 : part == 1 ? qr4 : vr4;
        const int lc = piece_col(), lt = piece_row();
#pragma unroll
        for (int j = 0; j < NLD; ++j) dst[j] = buf_load16(rs, (lt + RPP * j) * rstride + lc * ESZ, 0);
        if (part == 0 && tid < CT) {
            const size_t gi = ((size_t)b * T + (t0 + tid)) * H + h;
            a_in = tid < ceff ? alpha[gi] : 1.f;
            b_in = tid < ceff ? beta[gi] : 0.f;
        }
    };
    // element i of a 16-byte piece, widened to FP32 (bf16 widens exactly)
    auto elem = [](const U4 &u, int i) -> float {
        const uint32_t w4[4] = {u.x, u.y, u.z, u.w};
        if (IN_BF16) return __builtin_bit_cast(float, (w4[i >> 1] >> (16 * (i & 1))) << 16);
        return __builtin_bit_cast(float, w4[i]);
    };
    load_part(0, 0);
    load_part(0, 1);
    load_part(0, 2);
    for (int ch = 0; ch < nchunks; ++ch) {
        const int t0 = ch * chunk;
        const int ceff = min(chunk, T - t0);
        // ---- 1. chunk operands into LDS (loaded during the previous chunk) ----
        const int lc = piece_col(), lt = piece_row();
        int inv_c[VPL];
        float c_c[VPL], y_c[VPL];
#pragma unroll
        for (int i = 0; i < VPL; ++i) {
            inv_c[i] = s.inv[lc + i];
            c_c[i] = pool.smooth[h * DV + lc + i];
            y_c[i] = 1.0f / c_c[i];   // RN(1/c)
        }
#pragma unroll
        for (int j = 0; j < NLD; ++j) {
            const int t = lt + RPP * j;
            float vv[VPL];
#pragma unroll
            for (int i = 0; i < VPL; ++i) {
                s.K[t * LDK + inv_c[i]] = elem(kr4[j], i);
                s.Q[t * LDK + inv_c[i]] = elem(qr4[j], i);
                vv[i] = div_by_recip(elem(vr4[j], i), c_c[i], y_c[i]);  // v' = D_c^{-1} v
            }
            // v' in model column order: whole 16-byte writes, each lane of a
            // 16-lane group on its own banks (single floats four columns apart
            // met four to a bank)
#pragma unroll
            for (int i = 0; i < VPL; i += 4)
                *reinterpret_cast<v4f *>(&s.VU[t * LDK + lc + i]) =
                    v4f{vv[i], vv[i + 1], vv[i + 2], vv[i + 3]};
        }
        // ---- 2. decay prefix sums (wave 0: lane = token) ----
        if (tid < CT) {
            const int t = tid;
            const float a = a_in;
            double la = a > 0.f ? log((double)a) : 0.0;
            int z = a > 0.f ? -1 : t;
            // inclusive scans over the 64 lanes with DPP: shifts by 1, 2, 4
            // and 8 inside each 16-lane row, then lane 15 of a row into the
            // next row and lane 31 into the upper half (the lanes without a
            // source take the identity)
            scan_step<0x111, 0xf>(la, z);   // row_shr:1
            scan_step<0x112, 0xf>(la, z);   // row_shr:2
            scan_step<0x114, 0xf>(la, z);   // row_shr:4
            scan_step<0x118, 0xf>(la, z);   // row_shr:8
            scan_step<0x142, 0xa>(la, z);   // row_bcast:15 into rows 1 and 3
            scan_step<0x143, 0xc>(la, z);   // row_bcast:31 into rows 2 and 3
            s.lg[t] = la;
            s.zi[t] = z;
            s.gam[t] = z >= 0 ? 0.f : expf((float)la);
            s.bet[t] = b_in;
        }
        __syncthreads();
        if (tid < CT) {
            const int t = tid;
            s.rc[t] = t == CT - 1 ? 1.f : ratio(s, CT - 1, t);
        }

        // ---- 3. the masked Gram matrices, 20 lower 16x16 tiles over 4 waves:
        //      M = strict-lower decayed K K^T, A_qk = inclusive-lower decayed
        //      Q K^T (in the W tile, free during the chunk); then per wave, on
        //      its 32 value columns, Y = V' - Gamma K S0 in the accumulator
        //      layout ----
        float *const Aqk = s.W;
        for (int tile = w; tile < 20; tile += 4) {
            const int tt = tile < 10 ? tile : tile - 10;
            const int tb = tt >= 6 ? 3 : tt >= 3 ? 2 : tt >= 1 ? 1 : 0;
            const int sb = tt - tb * (tb + 1) / 2;
            if (IN_BF16) {   // q and k are exact bf16 numbers: bf16 matrix cores
                if (tile < 10)
                    gram_tile_bf16<true>(s, s.K, s.M, tb, sb, l16, g);
                else
                    gram_tile_bf16<false>(s, s.Q, Aqk, tb, sb, l16, g);
            } else {
                if (tile < 10)
                    gram_tile<true>(s, s.K, s.M, tb, sb, l16, g);
                else
                    gram_tile<false>(s, s.Q, Aqk, tb, sb, l16, g);
            }
        }
        v4f D[4][2];
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) {
            v4f acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb < 8; ++kb) {
                const v4f a = lds4(s.K + (16 * tb + l16) * LDK + 16 * kb + 4 * g);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    acc0 = mfma4(a[j], S[kb][0][j], acc0);
                    acc1 = mfma4(a[j], S[kb][1][j], acc1);
                }
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = 16 * tb + 4 * g + r;
                const float gm = s.gam[row];
                const float *u = s.VU + row * LDK + 32 * w + l16;
                D[tb][0][r] = u[0] - gm * acc0[r];
                D[tb][1][r] = u[16] - gm * acc1[r];
            }
        }
        __syncthreads();

        // ---- 4. Wave 0 inverts the four unit lower triangular 16x16 diagonal
        //      blocks of I + B M, times B: lane 16 d + j forward-substitutes
        //      column j of D_d = (I + B M)_dd^-1 B_d. ----
        if (w == 0) {
            const int d = lane >> 4, j = lane & 15;
            const float *Md = s.M + 16 * d * LDM + 16 * d;
            float bt[16], y[16];
#pragma unroll
            for (int t = 0; t < 16; ++t) bt[t] = s.bet[16 * d + t];
#pragma unroll
            for (int t = 0; t < 16; ++t) {
                // two interleaved partial sums halve the dependent chain
                float acc0 = 0.f, acc1 = 0.f;
#pragma unroll
                for (int i = 0; i < t; ++i) {
                    if (i & 1)
                        acc1 = __builtin_fmaf(Md[t * LDM + i], y[i], acc1);
                    else
                        acc0 = __builtin_fmaf(Md[t * LDM + i], y[i], acc0);
                }
                float acc = acc0 + acc1;
                // every lane evaluates the row (no branch around it), so the
                // next rows' reads can be issued early
                asm volatile("" : "+v"(acc));
                y[t] = t < j ? 0.f : t == j ? bt[t] : -bt[t] * acc;
            }
#pragma unroll
            for (int t = 0; t < 16; ++t) s.Dinv[(16 * d + t) * LDI + j] = y[t];
        }
        __syncthreads();

        // ---- 5. per wave: (I + B M) Delta = B Y on its 32 columns, block by
        //      block on the matrix cores in registers: Delta_d = D_d Y_d, then
        //      Y_e -= M_ed Delta_d for the later blocks.  This is the Delta of
        //      (I + B M) [W | U] = B [Gamma K | V], Delta = U - W S0, with half
        //      the right-hand-side columns; the accumulator layout of each
        //      product is the next one's B operand. ----
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            const v4f a = lds4(s.Dinv + (16 * d + l16) * LDI + 4 * g);
#pragma unroll
            for (int ct = 0; ct < 2; ++ct) {
                v4f acc = {0.f, 0.f, 0.f, 0.f};
                acc = mfma4(a.x, D[d][ct][0], acc);
                acc = mfma4(a.y, D[d][ct][1], acc);
                acc = mfma4(a.z, D[d][ct][2], acc);
                acc = mfma4(a.w, D[d][ct][3], acc);
                D[d][ct] = acc;
            }
#pragma unroll
            for (int e = d + 1; e < 4; ++e) {
                const v4f m = lds4(s.M + (16 * e + l16) * LDM + 16 * d + 4 * g);
#pragma unroll
                for (int ct = 0; ct < 2; ++ct) {
                    v4f acc = {0.f, 0.f, 0.f, 0.f};
                    acc = mfma4(m.x, D[d][ct][0], acc);
                    acc = mfma4(m.y, D[d][ct][1], acc);
                    acc = mfma4(m.z, D[d][ct][2], acc);
                    acc = mfma4(m.w, D[d][ct][3], acc);
                    D[e][ct] -= acc;
                }
            }
        }

        // ---- 6. O = Gamma Q S0 + A_qk Delta, written as o = c (.) O; the
        //      output rows of the chunk through a buffer resource that ends at
        //      its last real token (padding rows write nothing) ----
        const int ostride = H * DV * 4;   // bytes between tokens
        const __amdgpu_buffer_rsrc_t ro =
            make_rsrc(o + (((size_t)b * T + t0) * H + h) * DV, (ceff - 1) * ostride + DV * 4);
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) {
            v4f acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb < 8; ++kb) {
                const v4f a = lds4(s.Q + (16 * tb + l16) * LDK + 16 * kb + 4 * g);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    acc0 = mfma4(a[j], S[kb][0][j], acc0);
                    acc1 = mfma4(a[j], S[kb][1][j], acc1);
                }
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float gm = s.gam[16 * tb + 4 * g + r];
                acc0[r] *= gm;
                acc1[r] *= gm;
            }
#pragma unroll
            for (int sb = 0; sb <= tb; ++sb) {
                const v4f a = lds4(Aqk + (16 * tb + l16) * LDM + 16 * sb + 4 * g);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    acc0 = mfma4(a[j], D[sb][0][j], acc0);
                    acc1 = mfma4(a[j], D[sb][1][j], acc1);
                }
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int off = (16 * tb + 4 * g + r) * ostride + (32 * w + l16) * 4;
                buf_storef(ro, c_out[0] * acc0[r], off, 0);
                buf_storef(ro, c_out[1] * acc1[r], off + 64, 0);
            }
        }

        // ---- 7. S_C = g_C S0 + K^T diag(r(C, t)) Delta; the next chunk's
        //      inputs are loaded meanwhile ----
        if (ch + 1 < nchunks) load_part(ch + 1, 0);
        {
            const float gc = s.gam[CT - 1];
#pragma unroll
            for (int rb = 0; rb < 8; ++rb)
#pragma unroll
                for (int cb = 0; cb < 2; ++cb) S[rb][cb] *= gc;
#pragma unroll
            for (int tb = 0; tb < 4; ++tb)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float f = s.rc[16 * tb + 4 * g + r];
                    D[tb][0][r] *= f;
                    D[tb][1][r] *= f;
                }
#pragma unroll
            for (int rb = 0; rb < 8; ++rb)
#pragma unroll
                for (int kb = 0; kb < 4; ++kb) {
                    float a[4];
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        a[j] = s.K[(16 * kb + 4 * g + j) * LDK + 16 * rb + l16];
#pragma unroll
                    for (int cb = 0; cb < 2; ++cb) {
                        S[rb][cb] = mfma4(a[0], D[kb][cb][0], S[rb][cb]);
                        S[rb][cb] = mfma4(a[1], D[kb][cb][1], S[rb][cb]);
                        S[rb][cb] = mfma4(a[2], D[kb][cb][2], S[rb][cb]);
                        S[rb][cb] = mfma4(a[3], D[kb][cb][3], S[rb][cb]);
                    }
                }
        }
        __syncthreads();  // every wave is done with s.Q and s.K

        // ---- 8. chunk end: store the state, continue from what was stored ----
        if (ch + 1 < nchunks) load_part(ch + 1, 1);
        if (FMT != 0) {
            uint8_t *stg = reinterpret_cast<uint8_t *>(s.Q);
            // FP32 rows 16..127 of the state for the INT8+Hadamard tier's
            // pass; VU and W (adjacent) are free from here to the next chunk
            float *F = reinterpret_cast<float *>(smem_raw + offsetof(PrefillSmem, VU));
#pragma unroll
            for (int rb = 0; rb < 8; ++rb)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int row = 16 * rb + 4 * g + r;
                    float v0 = S[rb][0][r], v1 = S[rb][1][r];
                    const int c0 = 32 * w + l16, c1 = c0 + 16;
                    if (rb == 0) {
                        const uint32_t h0 = f32_to_f16_bits(v0), h1 = f32_to_f16_bits(v1);
                        uint16_t *hp = reinterpret_cast<uint16_t *>(stg + HI_OFF);
                        hp[row * DV + c0] = (uint16_t)h0;
                        hp[row * DV + c1] = (uint16_t)h1;
                        S[rb][0][r] = f16_bits_to_f32(h0);
                        S[rb][1][r] = f16_bits_to_f32(h1);
                    } else if (FMT == 2) {
                        // INT8+Hadamard rows go through LDS (pass below)
                        F[(row - KHI) * LDK + c0] = v0;
                        F[(row - KHI) * LDK + c1] = v1;
                    }
                }
            if (FMT == 1) {
                // INT8 rows: each row's group maximum over its 16 lanes (the
                // row16_max steps, each step taken for all 28 rows of the
                // lane before the next, so no DPP read waits on the VALU
                // write just before it), then scale, codes and the
                // reconstruction the next chunk starts from
                uint32_t m[7][4];
#pragma unroll
                for (int rb = 1; rb < 8; ++rb)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        m[rb - 1][r] = __builtin_bit_cast(
                            uint32_t, fmaxf(fabsf(S[rb][0][r]), fabsf(S[rb][1][r])));
#pragma unroll
                for (int rb = 0; rb < 7; ++rb)
#pragma unroll
                    for (int r = 0; r < 4; ++r) m[rb][r] = row_max_step<0xb1>(m[rb][r]);
#pragma unroll
                for (int rb = 0; rb < 7; ++rb)
#pragma unroll
                    for (int r = 0; r < 4; ++r) m[rb][r] = row_max_step<0x4e>(m[rb][r]);
#pragma unroll
                for (int rb = 0; rb < 7; ++rb)
#pragma unroll
                    for (int r = 0; r < 4; ++r) m[rb][r] = row_max_step<0x141>(m[rb][r]);
#pragma unroll
                for (int rb = 0; rb < 7; ++rb)
#pragma unroll
                    for (int r = 0; r < 4; ++r) m[rb][r] = row_max_step<0x140>(m[rb][r]);
                int8_t *cp = reinterpret_cast<int8_t *>(stg + LO_OFF);
                const int c0 = 32 * w + l16, c1 = c0 + 16;
#pragma unroll
                for (int rb = 1; rb < 8; ++rb)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int lr = 16 * rb + 4 * g + r - KHI;
                        const float sc = group_scale(__builtin_bit_cast(float, m[rb - 1][r]));
                        const double rinv = scale_reciprocal(sc);
                        const float q0 = rintf(quant_quotient(S[rb][0][r], rinv));
                        const float q1 = rintf(quant_quotient(S[rb][1][r], rinv));
                        cp[lr * DV + c0] = (int8_t)(int)q0;
                        cp[lr * DV + c1] = (int8_t)(int)q1;
                        if (l16 == 0) reinterpret_cast<float *>(stg + SC_OFF)[lr * NGRP + w] = sc;
                        S[rb][0][r] = sc * q0;
                        S[rb][1][r] = sc * q1;
                    }
            }
            __syncthreads();
            if (FMT == 2) {
                // Each 32-value group on a lane pair, 16 values per lane (the
                // codec's mapping): forward transform, codes and (s16, z16)
                // into the staged unit, reconstruction, inverse transform.
                // Task e: group (row KHI + e/2 mod 112, group e/224), half e&1,
                // so the lanes of a pair are adjacent and consecutive pairs
                // read consecutive rows (distinct LDS banks).
                for (int e = tid; e < KLO * NGRP * 2; e += PT) {
                    const int gi = e >> 1, half = e & 1;
                    const int lr = gi % KLO, gq = gi / KLO;
                    float *x = F + lr * LDK + GRP * gq + 16 * half;
                    float y[16];
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const v4f t4 = lds4(x + 4 * j);
                        y[4 * j] = t4.x;
                        y[4 * j + 1] = t4.y;
                        y[4 * j + 2] = t4.z;
                        y[4 * j + 3] = t4.w;
                    }
                    hadamard32_pair(y, half);
                    float lo = y[0], hi = y[0];
#pragma unroll
                    for (int j = 1; j < 16; ++j) {
                        lo = fminf(lo, y[j]);
                        hi = fmaxf(hi, y[j]);
                    }
                    const U8Params pr = u8_params(lo, hi);
                    uint32_t wd[4];
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const float q0 = u8_code(y[4 * j], pr), q1 = u8_code(y[4 * j + 1], pr);
                        const float q2 = u8_code(y[4 * j + 2], pr), q3 = u8_code(y[4 * j + 3], pr);
                        wd[j] = pack4_u8(q0, q1, q2, q3);
                        y[4 * j] = pr.sh * (q0 - pr.zh);
                        y[4 * j + 1] = pr.sh * (q1 - pr.zh);
                        y[4 * j + 2] = pr.sh * (q2 - pr.zh);
                        y[4 * j + 3] = pr.sh * (q3 - pr.zh);
                    }
                    *reinterpret_cast<U4 *>(stg + LO_OFF + lr * DV + GRP * gq + 16 * half) =
                        U4{wd[0], wd[1], wd[2], wd[3]};
                    if (!half) reinterpret_cast<uint32_t *>(stg + SC_OFF)[lr * NGRP + gq] = pr.meta;
                    // the reconstruction transformed back: on the integer codes
                    // when every group of the wave is in the exact range (the
                    // same bits), else in FP64
                    if (__builtin_amdgcn_ballot_w64(!u8_group_exact(pr.sh, pr.zh)) == 0)
                        hadamard32_pair_codes(wd, pr.sh, pr.zh, half != 0, y);
                    else
                        hadamard32_pair(y, half);
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        *reinterpret_cast<v4f *>(x + 4 * j) =
                            v4f{y[4 * j], y[4 * j + 1], y[4 * j + 2], y[4 * j + 3]};
                }
                __syncthreads();
#pragma unroll
                for (int rb = 1; rb < 8; ++rb)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int lr = 16 * rb + 4 * g + r - KHI;
                        S[rb][0][r] = F[lr * LDK + 32 * w + l16];
                        S[rb][1][r] = F[lr * LDK + 32 * w + 16 + l16];
                    }
            }
            if (ch + 1 < nchunks) load_part(ch + 1, 2);
            for (int e = tid; e < UNIT_BYTES / 16; e += PT)
                reinterpret_cast<U4 *>(unit)[e] = reinterpret_cast<const U4 *>(stg)[e];
        } else {
            if (ch + 1 < nchunks) load_part(ch + 1, 2);
            float *u = reinterpret_cast<float *>(unit);
#pragma unroll
            for (int rb = 0; rb < 8; ++rb)
#pragma unroll
                for (int cb = 0; cb < 2; ++cb)
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        u[(16 * rb + 4 * g + r) * DV + 32 * w + 16 * cb + l16] = S[rb][cb][r];
        }
        __syncthreads();  // the staging copy is read out before the next chunk's loads
    }
}

// The kernel's dynamic LDS (about 152 KB) needs the function attribute raised,
// once per device; host threads that get here together set it twice, which is
// harmless.
hipError_t launch_prefill(int fmt, const PoolView &pool, const int32_t *slots, int n, int T,
                          int chunk, int in_bf16, const void *q, const void *k, const void *v,
                          const float *alpha, const float *beta, float *o, int init_from_pool,
                          hipStream_t stream) {
    const size_t smem = sizeof(PrefillSmem);
    dim3 grid((unsigned)(n * pool.num_heads)), block(PT);
#define QRS_PREFILL_CASE(F, B)                                                                    \
    if (fmt == F && in_bf16 == B) {                                                               \
        static std::atomic<bool> attr_set[16];                                                    \
        int dev = 0;                                                                              \
        const hipError_t de = hipGetDevice(&dev);                                                 \
        if (de != hipSuccess) return de;                                                          \
        if (dev < 0 || dev >= 16 || !attr_set[dev].load(std::memory_order_acquire)) {             \
            hipError_t e = hipFuncSetAttribute(                                                   \
                reinterpret_cast<const void *>(&prefill_kernel<F, B>),                            \
                hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);                           \
            if (e != hipSuccess) return e;                                                        \
            if (dev >= 0 && dev < 16) attr_set[dev].store(true, std::memory_order_release);       \
        }                                                                                         \
        hipLaunchKernelGGL((prefill_kernel<F, B>), grid, block, smem, stream, pool, slots, T,     \
                           chunk, q, k, v, alpha, beta, o, init_from_pool);                       \
        return hipGetLastError();                                                                 \
    }
    QRS_PREFILL_CASE(1, 0)
    QRS_PREFILL_CASE(1, 1)
    QRS_PREFILL_CASE(2, 0)
    QRS_PREFILL_CASE(2, 1)
    QRS_PREFILL_CASE(0, 0)
    QRS_PREFILL_CASE(0, 1)
#undef QRS_PREFILL_CASE
    return hipErrorInvalidValue;
}

}  // namespace qrs
