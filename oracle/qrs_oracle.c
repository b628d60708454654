/*
 * qrs_oracle.c -- plain, slow CPU oracle for the compressed recurrent-state
 * decode update of Gated DeltaNet (GDN) and Kimi Delta Attention (KDA).
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header, table or helper with the HIP library; the two meet only through
 * seeded input arrays.
 *
 * Sources (web pages; cited by title and section/equation):
 *   [DAMP]  "DAMP: Decay-Aware Mixed-Precision Recurrent-State Quantization",
 *           arXiv 2608.27513 (HTML, first version).
 *   [DAMP2] Reading notes on DAMP arXiv 2608.27513v2 (Chinese), the
 *           revision whose quantizer this oracle follows.
 *
 * What is computed, step by step (all arithmetic FP32 unless a function says
 * FP64; the pages fix FP32 for the recurrence -- [DAMP2] section 2.2 and
 * [DAMP] Appendix A.5 "Fused decode executor"):
 *
 *  - Stored coordinates ([DAMP2] section 2.7, Eqs.(17)-(18) of v2):
 *      T = P_K S D_c^{-1}; stored key row i holds model key channel perm[i];
 *      value column j is divided by the smoothing scale c[j].
 *      The value permutation P_V is the identity here.
 *  - Storage of one (slot, head) unit ([DAMP] Appendix A.5 Eq.(17) layout,
 *    with the v2 quantizer of [DAMP2] section 2.2 Eqs.(5)-(6)):
 *      rows 0..15   : FP16, round to nearest even;
 *      rows 16..127 : INT8 codes, one FP32 scale per 32 consecutive values of
 *                     the row: s = max|x| / 127, code = round(x / s),
 *                     symmetric, no zero point.
 *  - One decode step, delta form ([DAMP] section 3.1 Eq.(1)):
 *      Tbar = Lambda That,  w = Tbar^T k',  delta = v' - w,
 *      T = Tbar + beta k' delta^T,  o = c (.) (T^T q')
 *    with Lambda = alpha I (GDN) or diag(exp(g')) (KDA), k' = k[perm],
 *    q' = q[perm], g' = g[perm], v' = v / c.  The readout uses the FP32 state
 *    of this step before requantization ([DAMP2] section 2.2: dequantize,
 *    FP32 recurrence and readout, then compress).
 *
 * Readings where the pages are silent (each is listed in the design notes):
 *  - round() is round-half-to-even on the correctly rounded FP32 quotient x/s;
 *  - s = amax/127 is a correctly rounded FP32 division and is stored as is;
 *  - a group whose scale is zero (all values zero, or amax so small that
 *    amax/127 underflows to zero) stores s = 0 and all codes 0;
 *  - codes are clamped to [-127, 127] (never -128);
 *  - sums run in increasing stored-row order as separate multiply and add.
 *
 * Build: gcc -O2 -fno-fast-math -ffp-contract=off -fopenmp -shared -fPIC.
 * OpenMP only splits independent (slot, head) units across threads.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define DK 128          /* key dimension d_k */
#define DV 128          /* value dimension d_v */
#define KHI 16          /* FP16 key rows per head */
#define KLO (DK - KHI)  /* INT8 key rows per head */
#define GRP 32          /* values per INT8 scale group */
#define NGRP (DV / GRP) /* scale groups per row */

/* ------------------------------------------------------------------ */
/* IEEE 754 binary16 conversions, written from the format's definition: */
/* 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits; subnormals  */
/* have exponent field 0 and value fraction * 2^-24.                   */
/* ------------------------------------------------------------------ */

uint16_t orc_f32_to_f16(float f)
{
    uint32_t bits;
    memcpy(&bits, &f, sizeof bits);
    uint16_t sign = (uint16_t)((bits >> 16) & 0x8000u);
    if (isnan(f))
        return (uint16_t)(sign | 0x7e00u);
    double a = fabs((double)f);          /* exact: every float is a double */
    /* Largest finite half is 65504 = (2 - 2^-10) 2^15; the next step would
     * be 65536, so everything at or above the midpoint 65520 rounds to inf
     * (the tie goes to the even neighbour, which is the infinity). */
    if (a >= 65520.0)
        return (uint16_t)(sign | 0x7c00u);
    if (a == 0.0)
        return sign;
    int e2;
    frexp(a, &e2);                        /* a = m 2^e2, m in [0.5, 1) */
    int E = e2 - 1;                       /* floor(log2 a) */
    if (E < -14)
        E = -14;                          /* subnormal range shares 2^-24 spacing */
    double quantum = ldexp(1.0, E - 10);  /* spacing of halves in this binade */
    double n = rint(a / quantum);         /* exact quotient, round half to even */
    double r = n * quantum;               /* the rounded magnitude, exact */
    if (r < ldexp(1.0, -14)) {            /* subnormal half */
        return (uint16_t)(sign | (uint16_t)rint(r / ldexp(1.0, -24)));
    }
    int er;
    frexp(r, &er);
    int Er = er - 1;                      /* rounding may have carried into the next binade */
    uint16_t expf16 = (uint16_t)(Er + 15);
    uint16_t frac = (uint16_t)(r / ldexp(1.0, Er - 10) - 1024.0);
    return (uint16_t)(sign | (uint16_t)(expf16 << 10) | frac);
}

float orc_f16_to_f32(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int m = h & 0x3ff;
    float v;
    if (e == 0)
        v = (float)ldexp((double)m, -24);
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = (float)ldexp((double)(1024 + m), e - 25);
    return sign ? -v : v;
}

void orc_f32_to_f16_array(const float *x, uint16_t *h, int64_t n)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i)
        h[i] = orc_f32_to_f16(x[i]);
}

void orc_f16_to_f32_array(const uint16_t *h, float *x, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        x[i] = orc_f16_to_f32(h[i]);
}

/* ------------------------------------------------------------------ */
/* INT8 group codec ([DAMP2] section 2.2 Eqs.(5)-(6)).                */
/* ------------------------------------------------------------------ */

/* Quantize `len` values sharing one scale. */
void orc_quantize_group(const float *x, int len, int8_t *code, float *scale)
{
    float amax = 0.0f;
    for (int j = 0; j < len; ++j) {
        float a = fabsf(x[j]);
        if (a > amax)
            amax = a;
    }
    float s = amax / 127.0f;
    *scale = s;
    for (int j = 0; j < len; ++j) {
        if (s == 0.0f) {
            code[j] = 0;
            continue;
        }
        float r = rintf(x[j] / s);
        if (r > 127.0f)
            r = 127.0f;
        if (r < -127.0f)
            r = -127.0f;
        code[j] = (int8_t)r;
    }
}

/* Dequantized value of one code ([DAMP2] section 2.2 Eq.(6): Q(x) = s round(x/s)). */
static float dequant_code(float s, int8_t code)
{
    return s * (float)code;
}

/* Encode one unit held in stored coordinates. */
static void store_unit(const float *T /*[DK][DV]*/, uint16_t *hi, int8_t *lo, float *sc)
{
    for (int i = 0; i < KHI; ++i)
        for (int j = 0; j < DV; ++j)
            hi[i * DV + j] = orc_f32_to_f16(T[i * DV + j]);
    for (int i = KHI; i < DK; ++i)
        for (int g = 0; g < NGRP; ++g)
            orc_quantize_group(&T[i * DV + g * GRP], GRP,
                               &lo[(i - KHI) * DV + g * GRP],
                               &sc[(i - KHI) * NGRP + g]);
}

/* Decode one unit into stored coordinates. */
static void dequant_unit(const uint16_t *hi, const int8_t *lo, const float *sc, float *T)
{
    for (int i = 0; i < KHI; ++i)
        for (int j = 0; j < DV; ++j)
            T[i * DV + j] = orc_f16_to_f32(hi[i * DV + j]);
    for (int i = KHI; i < DK; ++i)
        for (int j = 0; j < DV; ++j)
            T[i * DV + j] = dequant_code(sc[(i - KHI) * NGRP + j / GRP], lo[(i - KHI) * DV + j]);
}

/* ------------------------------------------------------------------ */
/* Pool-level store / dequant.  The oracle pool is three arrays indexed */
/* by unit u = slot * num_heads + head:                                  */
/*   hi [U][16][128] uint16 (FP16 bits), lo [U][112][128] int8,          */
/*   sc [U][112][4] float.                                               */
/* space 0 = model coordinates (apply perm and c), 1 = stored.          */
/* ------------------------------------------------------------------ */

void orc_store(uint16_t *hi, int8_t *lo, float *sc, int num_heads,
               const int32_t *perm /*[H][DK]*/, const float *c /*[H][DV]*/,
               const int32_t *slots, int n, const float *S /*[n][H][DK][DV]*/, int space)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t uu = 0; uu < (int64_t)n * num_heads; ++uu) {
        int b = (int)(uu / num_heads), h = (int)(uu % num_heads);
        int64_t u = (int64_t)slots[b] * num_heads + h;
        const float *Sm = S + uu * DK * DV;
        float *T = (float *)malloc(sizeof(float) * DK * DV);
        for (int i = 0; i < DK; ++i)
            for (int j = 0; j < DV; ++j)
                T[i * DV + j] = space ? Sm[i * DV + j]
                                      : Sm[perm[h * DK + i] * DV + j] / c[h * DV + j];
        store_unit(T, hi + u * KHI * DV, lo + u * KLO * DV, sc + u * KLO * NGRP);
        free(T);
    }
}

void orc_dequant(const uint16_t *hi, const int8_t *lo, const float *sc, int num_heads,
                 const int32_t *perm, const float *c, const int32_t *slots, int n,
                 float *S /*[n][H][DK][DV]*/, int space)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t uu = 0; uu < (int64_t)n * num_heads; ++uu) {
        int b = (int)(uu / num_heads), h = (int)(uu % num_heads);
        int64_t u = (int64_t)slots[b] * num_heads + h;
        float *Sm = S + uu * DK * DV;
        float *T = (float *)malloc(sizeof(float) * DK * DV);
        dequant_unit(hi + u * KHI * DV, lo + u * KLO * DV, sc + u * KLO * NGRP, T);
        for (int i = 0; i < DK; ++i)
            for (int j = 0; j < DV; ++j) {
                if (space)
                    Sm[i * DV + j] = T[i * DV + j];
                else
                    Sm[perm[h * DK + i] * DV + j] = T[i * DV + j] * c[h * DV + j];
            }
        free(T);
    }
}

/* ------------------------------------------------------------------ */
/* One delta-rule step of one unit in stored coordinates, FP32          */
/* ([DAMP] section 3.1 Eq.(1); coordinates of [DAMP2] section 2.7).     */
/*   Th    : dequantized state before the step [DK][DV] (read)          */
/*   T     : FP32 state after the step [DK][DV] (written)               */
/*   lam   : per-row decay of this step [DK] (alpha for every row in    */
/*           GDN, exp(g'_i) in KDA)                                     */
/*   kp,qp : permuted key and query [DK]; vp = v / c [DV]               */
/*   o     : readout in model value order [DV]                          */
/* ------------------------------------------------------------------ */
static void step_unit_f32(const float *Th, float *T, const float *lam, const float *kp,
                          const float *qp, const float *vp, float beta, const float *c, float *o)
{
    float *Tbar = (float *)malloc(sizeof(float) * DK * DV);
    float delta[DV];
    for (int i = 0; i < DK; ++i)
        for (int j = 0; j < DV; ++j)
            Tbar[i * DV + j] = lam[i] * Th[i * DV + j];        /* decay */
    for (int j = 0; j < DV; ++j) {
        float w = 0.0f;
        for (int i = 0; i < DK; ++i)
            w = w + kp[i] * Tbar[i * DV + j];                   /* key readout of the decayed state */
        delta[j] = vp[j] - w;                                    /* delta-rule residual */
    }
    for (int i = 0; i < DK; ++i)
        for (int j = 0; j < DV; ++j)
            T[i * DV + j] = Tbar[i * DV + j] + kp[i] * (beta * delta[j]);  /* rank-1 write */
    for (int j = 0; j < DV; ++j) {
        float acc = 0.0f;
        for (int i = 0; i < DK; ++i)
            acc = acc + qp[i] * T[i * DV + j];                  /* readout o = T^T q' */
        o[j] = c[j] * acc;                                       /* undo value smoothing */
    }
    free(Tbar);
}

/* FP64 twin of step_unit_f32, same operation order. */
static void step_unit_f64(const double *Th, double *T, const double *lam, const double *kp,
                          const double *qp, const double *vp, double beta, const double *c,
                          double *o)
{
    double *Tbar = (double *)malloc(sizeof(double) * DK * DV);
    double delta[DV];
    for (int i = 0; i < DK; ++i)
        for (int j = 0; j < DV; ++j)
            Tbar[i * DV + j] = lam[i] * Th[i * DV + j];
    for (int j = 0; j < DV; ++j) {
        double w = 0.0;
        for (int i = 0; i < DK; ++i)
            w = w + kp[i] * Tbar[i * DV + j];
        delta[j] = vp[j] - w;
    }
    for (int i = 0; i < DK; ++i)
        for (int j = 0; j < DV; ++j)
            T[i * DV + j] = Tbar[i * DV + j] + kp[i] * (beta * delta[j]);
    for (int j = 0; j < DV; ++j) {
        double acc = 0.0;
        for (int i = 0; i < DK; ++i)
            acc = acc + qp[i] * T[i * DV + j];
        o[j] = c[j] * acc;
    }
    free(Tbar);
}

/* Gather the per-step operands of unit (b, h) into stored key order.
 * kind 0: GDN, gate = alpha [n][H]; kind 1: KDA, gate = g [n][H][DK]
 * (Lambda = diag(exp(g)), HTML section 3.1); kind 2: KDA with the decay
 * factors exp(g) given directly, gate = lambda [n][H][DK] (the per-window
 * method's recorded decays). */
static void gather_operands(int kind, int b, int h, int num_heads, const int32_t *perm,
                            const float *c, const float *q, const float *k, const float *v,
                            const float *gate, float *qp, float *kp, float *vp, float *lam)
{
    int64_t base = ((int64_t)b * num_heads + h) * DK;
    for (int i = 0; i < DK; ++i) {
        int src = perm[h * DK + i];
        qp[i] = q[base + src];
        kp[i] = k[base + src];
        lam[i] = kind == 0   ? gate[(int64_t)b * num_heads + h]
                 : kind == 1 ? expf(gate[base + src])
                             : gate[base + src];
    }
    for (int j = 0; j < DV; ++j)
        vp[j] = v[base + j] / c[h * DV + j];                      /* v' = D_c^{-1} v */
}

/* One compressed decode step for n slots x H heads:
 * dequantize -> FP32 delta-rule step and readout -> requantize in place. */
void orc_i8_decode(uint16_t *hi, int8_t *lo, float *sc, int num_heads, const int32_t *perm,
                   const float *c, const int32_t *slots, int n, int kind, const float *q,
                   const float *k, const float *v, const float *gate, const float *beta,
                   float *o /*[n][H][DV]*/)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t uu = 0; uu < (int64_t)n * num_heads; ++uu) {
        int b = (int)(uu / num_heads), h = (int)(uu % num_heads);
        int64_t u = (int64_t)slots[b] * num_heads + h;
        float qp[DK], kp[DK], vp[DV], lam[DK];
        gather_operands(kind, b, h, num_heads, perm, c, q, k, v, gate, qp, kp, vp, lam);
        float *Th = (float *)malloc(sizeof(float) * DK * DV);
        float *T = (float *)malloc(sizeof(float) * DK * DV);
        uint16_t *uhi = hi + u * KHI * DV;
        int8_t *ulo = lo + u * KLO * DV;
        float *usc = sc + u * KLO * NGRP;
        dequant_unit(uhi, ulo, usc, Th);
        step_unit_f32(Th, T, lam, kp, qp, vp, beta[uu], c + h * DV, o + uu * DV);
        store_unit(T, uhi, ulo, usc);
        free(Th);
        free(T);
    }
}

/* Same step on an uncompressed FP32 state held in stored coordinates,
 * pool T [U][DK][DV] (compression disabled). */
void orc_f32_decode(float *Tpool, int num_heads, const int32_t *perm, const float *c,
                    const int32_t *slots, int n, int kind, const float *q, const float *k,
                    const float *v, const float *gate, const float *beta, float *o)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t uu = 0; uu < (int64_t)n * num_heads; ++uu) {
        int b = (int)(uu / num_heads), h = (int)(uu % num_heads);
        int64_t u = (int64_t)slots[b] * num_heads + h;
        float qp[DK], kp[DK], vp[DV], lam[DK];
        gather_operands(kind, b, h, num_heads, perm, c, q, k, v, gate, qp, kp, vp, lam);
        float *T = (float *)malloc(sizeof(float) * DK * DV);
        float *Tu = Tpool + u * DK * DV;
        step_unit_f32(Tu, T, lam, kp, qp, vp, beta[uu], c + h * DV, o + uu * DV);
        memcpy(Tu, T, sizeof(float) * DK * DV);
        free(T);
    }
}

/* FP64 twin of orc_f32_decode (pool and outputs in double; inputs are the
 * same FP32 arrays, widened exactly; the KDA decay uses exp in double). */
void orc_f64_decode(double *Tpool, int num_heads, const int32_t *perm, const float *c,
                    const int32_t *slots, int n, int kind, const float *q, const float *k,
                    const float *v, const float *gate, const float *beta, double *o)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t uu = 0; uu < (int64_t)n * num_heads; ++uu) {
        int b = (int)(uu / num_heads), h = (int)(uu % num_heads);
        int64_t u = (int64_t)slots[b] * num_heads + h;
        int64_t base = uu * DK;
        double qp[DK], kp[DK], vp[DV], lam[DK], cc[DV];
        for (int i = 0; i < DK; ++i) {
            int src = perm[h * DK + i];
            qp[i] = q[base + src];
            kp[i] = k[base + src];
            lam[i] = kind == 0   ? (double)gate[uu]
                     : kind == 1 ? exp((double)gate[base + src])
                                 : (double)gate[base + src];
        }
        for (int j = 0; j < DV; ++j) {
            cc[j] = c[h * DV + j];
            vp[j] = (double)v[base + j] / cc[j];
        }
        double *T = (double *)malloc(sizeof(double) * DK * DV);
        double *Tu = Tpool + u * DK * DV;
        step_unit_f64(Tu, T, lam, kp, qp, vp, (double)beta[uu], cc, o + uu * DV);
        memcpy(Tu, T, sizeof(double) * DK * DV);
        free(T);
    }
}

/* ------------------------------------------------------------------ */
/* Chunked prefill ([DAMP] Appendix A.5 "Prefill path"; [DAMP2] section */
/* 2.2): FP32 recurrence token by token inside a chunk with no codec,   */
/* outputs from the FP32 in-chunk state, and at every chunk end the     */
/* state is written in packed form; the next chunk starts from that     */
/* packed state.  GDN gating (alpha per token and head).                */
/*   q, k, v : [n][Tlen][H][128] FP32;  alpha, beta : [n][Tlen][H]       */
/*   o       : [n][Tlen][H][128]                                        */
/*   init_from_pool: 1 = start from the slot's packed state, 0 = zero.  */
/* ------------------------------------------------------------------ */
void orc_i8_prefill(uint16_t *hi, int8_t *lo, float *sc, int num_heads, const int32_t *perm,
                    const float *c, const int32_t *slots, int n, int Tlen, int chunk,
                    const float *q, const float *k, const float *v, const float *alpha,
                    const float *beta, float *o, int init_from_pool)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t uu = 0; uu < (int64_t)n * num_heads; ++uu) {
        int b = (int)(uu / num_heads), h = (int)(uu % num_heads);
        int64_t u = (int64_t)slots[b] * num_heads + h;
        uint16_t *uhi = hi + u * KHI * DV;
        int8_t *ulo = lo + u * KLO * DV;
        float *usc = sc + u * KLO * NGRP;
        float *Tcur = (float *)malloc(sizeof(float) * DK * DV);
        float *Tnext = (float *)malloc(sizeof(float) * DK * DV);
        if (init_from_pool)
            dequant_unit(uhi, ulo, usc, Tcur);
        else
            memset(Tcur, 0, sizeof(float) * DK * DV);
        for (int t = 0; t < Tlen; ++t) {
            /* operands of token t, viewed as a one-slot step */
            int64_t tok = ((int64_t)b * Tlen + t) * num_heads + h;     /* [n][Tlen][H] index */
            float qp[DK], kp[DK], vp[DV], lam[DK];
            for (int i = 0; i < DK; ++i) {
                int src = perm[h * DK + i];
                qp[i] = q[tok * DK + src];
                kp[i] = k[tok * DK + src];
                lam[i] = alpha[tok];
            }
            for (int j = 0; j < DV; ++j)
                vp[j] = v[tok * DV + j] / c[h * DV + j];
            step_unit_f32(Tcur, Tnext, lam, kp, qp, vp, beta[tok], c + h * DV, o + tok * DV);
            float *tmp = Tcur;
            Tcur = Tnext;
            Tnext = tmp;
            if ((t + 1) % chunk == 0 || t + 1 == Tlen) {
                store_unit(Tcur, uhi, ulo, usc);           /* chunk-end write */
                dequant_unit(uhi, ulo, usc, Tcur);         /* the next chunk reads it back */
            }
        }
        free(Tcur);
        free(Tnext);
    }
}

/* Sizes of the oracle's representation of one unit, in bytes. */
/* ------------------------------------------------------------------ */
/* The first revision's low tier ([DAMP] section 3.2 Eq.(3); Appendix   */
/* A.1 and Table 3, "INT8+Hadamard"; Appendix A.5 Eq.(17)): a normalized */
/* block-32 Hadamard transform along d_v, then asymmetric UINT8 codes    */
/* with an FP16 scale and zero point per 32 values.  Same unit size as   */
/* the INT8 tier above (4 bytes of metadata per group).                  */
/* ------------------------------------------------------------------ */

/* Normalized block-32 Hadamard, y = H x / sqrt(32) with H[i][j] =
 * (-1)^popcount(i & j) (Sylvester order).  Each output is the FP64 sum over
 * j in increasing order, times RN64(2^-2.5) (= RN64(sqrt 2) / 8, the
 * correctly rounded 1/sqrt(32)), rounded once to FP32.  The transform is its
 * own inverse. */
void orc_hadamard32(const float *x, float *y)
{
    const double inv = sqrt(2.0) * 0.125;
    for (int i = 0; i < GRP; ++i) {
        double acc = 0.0;
        for (int j = 0; j < GRP; ++j) {
            const int neg = __builtin_popcount((unsigned)(i & j)) & 1;
            acc += neg ? -(double)x[j] : (double)x[j];
        }
        y[i] = (float)(acc * inv);
    }
}

/* Eq.(3) with b = 8 on one transformed group y[32]:
 *   s = (y_max - y_min) / 255, stored as FP16 s16 (round to nearest even);
 *   z = round(-y_min / s16), stored as FP16 z16;
 *   q_i = round(y_i / s16) + z16, saturated to [0, 255];
 *   reconstruction y_hat_i = s16 (q_i - z16).
 * Quantization uses the stored FP16 values, so codes and reconstruction
 * agree.  All arithmetic FP32 (correctly rounded divides, round half to
 * even).  A group whose stored scale is zero (constant group, or a scale
 * below the FP16 range) stores s16 = z16 = 0 and codes 0. */
void orc_quantize_group_u8(const float *y, uint8_t *q, uint16_t *s16, uint16_t *z16)
{
    float lo = y[0], hi = y[0];
    for (int j = 1; j < GRP; ++j) {
        if (y[j] < lo)
            lo = y[j];
        if (y[j] > hi)
            hi = y[j];
    }
    const float s = (hi - lo) / 255.0f;
    const uint16_t sb = orc_f32_to_f16(s);
    const float sh = orc_f16_to_f32(sb);
    if (sh == 0.0f) {
        *s16 = 0;
        *z16 = 0;
        for (int j = 0; j < GRP; ++j)
            q[j] = 0;
        return;
    }
    const uint16_t zb = orc_f32_to_f16(rintf(-lo / sh));
    const float zh = orc_f16_to_f32(zb);
    for (int j = 0; j < GRP; ++j) {
        float c = rintf(y[j] / sh) + zh;
        if (c < 0.0f)
            c = 0.0f;
        if (c > 255.0f)
            c = 255.0f;
        q[j] = (uint8_t)c;
    }
    *s16 = sb;
    *z16 = zb;
}

static void store_unit_u8(const float *T, uint16_t *hi, uint8_t *lo, uint16_t *meta)
{
    for (int i = 0; i < KHI; ++i)
        for (int j = 0; j < DV; ++j)
            hi[i * DV + j] = orc_f32_to_f16(T[i * DV + j]);
    for (int i = KHI; i < DK; ++i)
        for (int g = 0; g < NGRP; ++g) {
            float y[GRP];
            orc_hadamard32(&T[i * DV + g * GRP], y);
            uint16_t *m = meta + ((i - KHI) * NGRP + g) * 2;
            orc_quantize_group_u8(y, &lo[(i - KHI) * DV + g * GRP], &m[0], &m[1]);
        }
}

static void dequant_unit_u8(const uint16_t *hi, const uint8_t *lo, const uint16_t *meta, float *T)
{
    for (int i = 0; i < KHI; ++i)
        for (int j = 0; j < DV; ++j)
            T[i * DV + j] = orc_f16_to_f32(hi[i * DV + j]);
    for (int i = KHI; i < DK; ++i)
        for (int g = 0; g < NGRP; ++g) {
            const uint16_t *m = meta + ((i - KHI) * NGRP + g) * 2;
            const float sh = orc_f16_to_f32(m[0]), zh = orc_f16_to_f32(m[1]);
            float yh[GRP];
            for (int j = 0; j < GRP; ++j)
                yh[j] = sh * ((float)lo[(i - KHI) * DV + g * GRP + j] - zh);
            orc_hadamard32(yh, &T[i * DV + g * GRP]);
        }
}

/* Pool-level calls of the v1 tier; arrays as for the INT8 tier except
 * lo [U][112][128] uint8 and meta [U][112][4][2] uint16 (FP16 s, z). */
void orc_u8_store(uint16_t *hi, uint8_t *lo, uint16_t *meta, int num_heads, const int32_t *perm,
                  const float *c, const int32_t *slots, int n, const float *S, int space)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t uu = 0; uu < (int64_t)n * num_heads; ++uu) {
        int b = (int)(uu / num_heads), h = (int)(uu % num_heads);
        int64_t u = (int64_t)slots[b] * num_heads + h;
        const float *Sm = S + uu * DK * DV;
        float *T = (float *)malloc(sizeof(float) * DK * DV);
        for (int i = 0; i < DK; ++i)
            for (int j = 0; j < DV; ++j)
                T[i * DV + j] = space ? Sm[i * DV + j]
                                      : Sm[perm[h * DK + i] * DV + j] / c[h * DV + j];
        store_unit_u8(T, hi + u * KHI * DV, lo + u * KLO * DV, meta + u * KLO * NGRP * 2);
        free(T);
    }
}

void orc_u8_dequant(const uint16_t *hi, const uint8_t *lo, const uint16_t *meta, int num_heads,
                    const int32_t *perm, const float *c, const int32_t *slots, int n, float *S,
                    int space)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t uu = 0; uu < (int64_t)n * num_heads; ++uu) {
        int b = (int)(uu / num_heads), h = (int)(uu % num_heads);
        int64_t u = (int64_t)slots[b] * num_heads + h;
        float *Sm = S + uu * DK * DV;
        float *T = (float *)malloc(sizeof(float) * DK * DV);
        dequant_unit_u8(hi + u * KHI * DV, lo + u * KLO * DV, meta + u * KLO * NGRP * 2, T);
        for (int i = 0; i < DK; ++i)
            for (int j = 0; j < DV; ++j) {
                if (space)
                    Sm[i * DV + j] = T[i * DV + j];
                else
                    Sm[perm[h * DK + i] * DV + j] = T[i * DV + j] * c[h * DV + j];
            }
        free(T);
    }
}

/* The same compressed decode step with the v1 tier. */
void orc_u8_decode(uint16_t *hi, uint8_t *lo, uint16_t *meta, int num_heads, const int32_t *perm,
                   const float *c, const int32_t *slots, int n, int kind, const float *q,
                   const float *k, const float *v, const float *gate, const float *beta,
                   float *o /*[n][H][DV]*/)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t uu = 0; uu < (int64_t)n * num_heads; ++uu) {
        int b = (int)(uu / num_heads), h = (int)(uu % num_heads);
        int64_t u = (int64_t)slots[b] * num_heads + h;
        float qp[DK], kp[DK], vp[DV], lam[DK];
        gather_operands(kind, b, h, num_heads, perm, c, q, k, v, gate, qp, kp, vp, lam);
        float *Th = (float *)malloc(sizeof(float) * DK * DV);
        float *T = (float *)malloc(sizeof(float) * DK * DV);
        uint16_t *uhi = hi + u * KHI * DV;
        uint8_t *ulo = lo + u * KLO * DV;
        uint16_t *umeta = meta + u * KLO * NGRP * 2;
        dequant_unit_u8(uhi, ulo, umeta, Th);
        step_unit_f32(Th, T, lam, kp, qp, vp, beta[uu], c + h * DV, o + uu * DV);
        store_unit_u8(T, uhi, ulo, umeta);
        free(Th);
        free(T);
    }
}

/* Chunked prefill on the first revision's low tier, GDN gating: the
 * recurrence of orc_i8_prefill (FP32 inside a chunk, sequential), with the
 * chunk-end state written in the INT8+Hadamard format and read back from it
 * ([DAMP] Appendix A.5 "Prefill path"). */
void orc_u8_prefill(uint16_t *hi, uint8_t *lo, uint16_t *meta, int num_heads, const int32_t *perm,
                    const float *c, const int32_t *slots, int n, int Tlen, int chunk,
                    const float *q, const float *k, const float *v, const float *alpha,
                    const float *beta, float *o, int init_from_pool)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t uu = 0; uu < (int64_t)n * num_heads; ++uu) {
        int b = (int)(uu / num_heads), h = (int)(uu % num_heads);
        int64_t u = (int64_t)slots[b] * num_heads + h;
        uint16_t *uhi = hi + u * KHI * DV;
        uint8_t *ulo = lo + u * KLO * DV;
        uint16_t *umeta = meta + u * KLO * NGRP * 2;
        float *Tcur = (float *)malloc(sizeof(float) * DK * DV);
        float *Tnext = (float *)malloc(sizeof(float) * DK * DV);
        if (init_from_pool)
            dequant_unit_u8(uhi, ulo, umeta, Tcur);
        else
            memset(Tcur, 0, sizeof(float) * DK * DV);
        for (int t = 0; t < Tlen; ++t) {
            int64_t tok = ((int64_t)b * Tlen + t) * num_heads + h;     /* [n][Tlen][H] index */
            float qp[DK], kp[DK], vp[DV], lam[DK];
            for (int i = 0; i < DK; ++i) {
                int src = perm[h * DK + i];
                qp[i] = q[tok * DK + src];
                kp[i] = k[tok * DK + src];
                lam[i] = alpha[tok];
            }
            for (int j = 0; j < DV; ++j)
                vp[j] = v[tok * DV + j] / c[h * DV + j];
            step_unit_f32(Tcur, Tnext, lam, kp, qp, vp, beta[tok], c + h * DV, o + tok * DV);
            float *tmp = Tcur;
            Tcur = Tnext;
            Tnext = tmp;
            if ((t + 1) % chunk == 0 || t + 1 == Tlen) {
                store_unit_u8(Tcur, uhi, ulo, umeta);          /* chunk-end write */
                dequant_unit_u8(uhi, ulo, umeta, Tcur);        /* the next chunk reads it back */
            }
        }
        free(Tcur);
        free(Tnext);
    }
}

/* ------------------------------------------------------------------ */
/* Key-channel selection: quantization-error energy of each key channel */
/* ([DAMP] section 4 "Accumulated-error risk", Eq.(8), and Appendix A.2 */
/* Eq.(14); [DAMP2] section 2.5, e_{t,u}).                              */
/* ------------------------------------------------------------------ */

/* For n calibration states S [n][H][DK][DV] in model coordinates, the squared
 * error of row u under the low-precision storage mapping: the row is taken to
 * stored value coordinates (x_j = S[u][j] / c[j], FP32 divide), every 32-value
 * group is quantized and dequantized with the INT8 codec above, the result is
 * mapped back (x_hat_j * c[j], FP32 multiply), and
 *     e[n][H][u] = sum_j (x_hat_j c_j - S[u][j])^2
 * is accumulated in FP64 over increasing j.  Every key channel is measured
 * under the INT8 mapping, since the statistic ranks candidates for the FP16
 * tier.  c == NULL means unit smoothing. */
void orc_channel_error(const float *S, int n, int num_heads, const float *c, double *e)
{
#pragma omp parallel for schedule(static)
    for (int64_t sh = 0; sh < (int64_t)n * num_heads; ++sh) {
        const int h = (int)(sh % num_heads);
        const float *Su = S + sh * DK * DV;
        for (int u = 0; u < DK; ++u) {
            float x[DV];
            int8_t code[DV];
            float sc[NGRP];
            for (int j = 0; j < DV; ++j)
                x[j] = Su[u * DV + j] / (c ? c[h * DV + j] : 1.0f);
            for (int g = 0; g < NGRP; ++g)
                orc_quantize_group(&x[g * GRP], GRP, &code[g * GRP], &sc[g]);
            double acc = 0.0;
            for (int j = 0; j < DV; ++j) {
                const float back = dequant_code(sc[j / GRP], code[j]) * (c ? c[h * DV + j] : 1.0f);
                const double d = (double)back - (double)Su[u * DV + j];
                acc += d * d;
            }
            e[sh * DK + u] = acc;
        }
    }
}

int64_t orc_unit_bytes(void)
{
    return (int64_t)KHI * DV * 2 + (int64_t)KLO * DV * 1 + (int64_t)KLO * NGRP * 4;
}

/* Threads the OpenMP loops above use (reported beside the oracle's timings). */
int orc_max_threads(void)
{
    return omp_get_max_threads();
}
