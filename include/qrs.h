/*
 * qrs.h -- C ABI of libqrs: compressed recurrent-state decode for Gated
 * DeltaNet (GDN) and Kimi Delta Attention (KDA) on AMD Instinct MI355X
 * (gfx950).
 *
 * The method follows "DAMP: Decay-Aware Mixed-Precision Recurrent-State
 * Quantization" (arXiv 2608.27513; HTML version and the reading notes on its
 * v2).  Each (request slot, head) state S in R^{128x128} (rows = key channels,
 * columns = value dimensions) is kept in stored coordinates
 *     T = P_K S D_c^{-1}                      (v2 notes, section 2.7, Eq.(17) of v2)
 * i.e. stored row i holds model key channel perm[h][i] and value column j is
 * divided by the smoothing scale c[h][j] > 0.  The first 16 stored rows are
 * FP16, the other 112 are INT8 with one FP32 scale per 32 values
 * (s = max|x| / 127, code = round-half-even(x / s), no zero point; v2 notes
 * section 2.2, Eqs.(5)-(6)), packed contiguously per unit (HTML, Appendix A.5,
 * Eq.(17)): 9.875 bits per state value (HTML, Eq.(12)).
 *
 * A decode step reads the packed state, dequantizes it, applies the
 * delta-rule update in FP32
 *     S_t = (I - beta k k^T) Lambda_t S_{t-1} + beta k v^T,  o_t = S_t^T q_t
 * (HTML section 3.1, Eqs.(1)-(2); Lambda_t = alpha_t I for GDN,
 * diag(exp(g_t)) for KDA), reads out from the FP32 state of this step, then
 * recomputes the group scales, requantizes and writes back in place (v2 notes
 * section 2.2; HTML Appendix A.5 "Fused decode executor").
 *
 * Conventions for every entry point:
 *  - Pointers named *_host are host memory; every other pointer is HIP device
 *    memory on the device that was current when the pool was created.
 *  - Work is enqueued asynchronously on `stream` (0 = the null stream);
 *    inputs must stay valid and unmodified until the work completes.
 *  - The caller owns all memory.  The library never allocates device memory;
 *    it owns only the small host-side pool handle.
 *  - Return value: QRS_OK, or a negative status (qrs_status_string names
 *    it).  QRS_EINVAL: null pointer, negative size, bad enum, a perm that is
 *    not a permutation, a non-positive or non-finite smoothing scale, a buffer
 *    too small.  QRS_EUNSUPPORTED: a shape other than d_k = d_v = 128,
 *    k_hi = 16, group = 32 (FP32 pools: k_hi = group = 0), or a call a pool
 *    format does not support.  QRS_EDEVICE: a HIP
 *    launch or copy failed (asynchronous faults surface at the caller's next
 *    synchronization).  Nothing is enqueued when the call returns an error.
 *  - Slot ids: int32 device array of length n.  Ids must be distinct within
 *    one call (duplicates race on the same state).  A slot id outside
 *    [0, num_slots) is skipped on the device: its state is not touched and
 *    its output rows are filled with NaN.
 *  - Operands are FP32, C-contiguous, in model key order; the library gathers
 *    them through perm.  Calls on disjoint slots of one pool may overlap.
 */
#ifndef QRS_H
#define QRS_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct qrs_pool_s *qrs_pool;

/* Pool formats. */
enum {
    QRS_FMT_FP32 = 0,  /* uncompressed FP32 state (compression disabled) */
    QRS_FMT_I8F16 = 1, /* 16 FP16 rows + 112 INT8 rows, FP32 scale per 32 values */
    QRS_FMT_U8H16 = 2  /* 16 FP16 rows + 112 UINT8 rows of the block-32 Hadamard transform,
                          FP16 scale and zero point per 32 values (the first revision's tier) */
};

/* Coordinate spaces for store / dequant. */
enum {
    QRS_SPACE_MODEL = 0,  /* S in model key order, unsmoothed */
    QRS_SPACE_STORED = 1  /* T = P_K S D_c^{-1}, stored row order */
};

/* Status codes. */
enum {
    QRS_OK = 0,
    QRS_EINVAL = -1,
    QRS_EUNSUPPORTED = -2,
    QRS_EDEVICE = -3
};

/*
 * QRS_FMT_U8H16 ([DAMP] HTML section 3.2 Eq.(3); Appendix A.1, Table 3
 * "INT8+Hadamard"; Appendix A.5 Eq.(17)): each 32-value group x of an
 * INT8-tier row is transformed, y = H_32 x / sqrt(32) (Sylvester order; FP64
 * sums, times RN64(2^-2.5), rounded once to FP32), then coded as
 *   s = RN32((max y - min y) / 255) -> FP16 s16;  z = round(-min y / s16) -> FP16 z16;
 *   code = min(max(round(y / s16) + z16, 0), 255)   (round half to even),
 * and read back as x = H_32 (s16 (code - z16)) / sqrt(32).  A zero s16
 * stores s16 = z16 = 0 and codes 0.  Same unit size and offsets as
 * QRS_FMT_I8F16; the 4-byte word of a group holds s16 in bits 0..15 and z16
 * in bits 16..31.  Decode, store/dequant and chunked prefill support it;
 * the per-window decode step returns QRS_EUNSUPPORTED.
 */

/*
 * Layout of one unit u = slot * num_heads + head, at byte offset
 * u * unit_bytes from the pool base (unit_bytes is a multiple of 256):
 *   QRS_FMT_I8F16 (20224 bytes):
 *     [0, 4096)       FP16 rows 0..15, row-major [16][128] (IEEE binary16 bits)
 *     [4096, 18432)   INT8 codes of rows 16..127, row-major [112][128]
 *     [18432, 20224)  FP32 scales [112][4]; scale g of a row covers
 *                     columns 32g..32g+31
 *   QRS_FMT_FP32 (65536 bytes): FP32 [128][128] row-major.
 * After the num_slots * num_heads units: perm int32 [H][128] and c FP32
 * [H][128], each starting on a 256-byte boundary.
 */
#define QRS_I8F16_UNIT_BYTES 20224
#define QRS_I8F16_HI_OFFSET 0
#define QRS_I8F16_LO_OFFSET 4096
#define QRS_I8F16_SCALE_OFFSET 18432
#define QRS_FP32_UNIT_BYTES 65536

/*
 * Bytes of device memory a pool needs (state units plus the perm / smoothing
 * tail).  Returns 0 for an invalid or unsupported shape.
 */
size_t qrs_state_pool_bytes(int fmt, int num_slots, int num_heads, int d_k, int d_v, int k_hi,
                            int group);

/*
 * Create a pool over caller-owned device memory `dev_mem` of `dev_bytes`
 * (>= qrs_state_pool_bytes(...), 256-byte aligned).  Copies perm_host
 * ([H][128], stored row i <- model key channel perm_host[h][i]; NULL =
 * identity) and smooth_host ([H][128], c > 0; NULL = ones) into the pool tail
 * and zero-fills the state region (the tables synchronously, the fill on
 * `stream`).  FP32 pools hold the state uncompressed in the same stored
 * coordinates (compression disabled).  The key permutation is a
 * static per-head layout stored once with the model (HTML section 5.2 and
 * Appendix A.5); smoothing is the per-value-column scaling of v2 (notes
 * section 2.7).  On success *out receives the handle.
 */
int qrs_create_state_pool(int fmt, int num_slots, int num_heads, int d_k, int d_v, int k_hi,
                          int group, void *dev_mem, size_t dev_bytes, const int32_t *perm_host,
                          const float *smooth_host, hipStream_t stream, qrs_pool *out);

/* Release the host handle (the device memory stays the caller's).  NULL is a no-op. */
int qrs_destroy_state_pool(qrs_pool pool);

/* Geometry of a pool: any output pointer may be NULL. */
int qrs_pool_info(qrs_pool pool, int *fmt, int *num_slots, int *num_heads, size_t *unit_bytes,
                  size_t *perm_offset, size_t *smooth_offset);

/*
 * Write states into the given slots.  S: FP32 [n][H][128][128].
 * space QRS_SPACE_MODEL: T[i][j] = S[perm[i]][j] / c[j] (IEEE FP32 divide),
 * then encode; QRS_SPACE_STORED: S is already T.  Encoding: rows 0..15
 * FP16 round-to-nearest-even; rows 16..127 per 32-value group
 * s = RN(amax / 127) and code = RN_int(RN(x / s)), s = 0 and codes 0 when
 * the scale is zero (v2 notes section 2.2, Eqs.(5)-(6)).  FP32 pools copy.
 */
int qrs_store_state(qrs_pool pool, const int32_t *slots, int n, const float *S, int space,
                    hipStream_t stream);

/*
 * Read states back.  S_out: FP32 [n][H][128][128].  Dequantization is
 * T = f32(fp16) on rows 0..15 and T = s * f32(code) on rows 16..127 (v2 notes
 * section 2.2, Eq.(6)); QRS_SPACE_MODEL then writes S[perm[i]][j] = T[i][j] * c[j].
 */
int qrs_dequant_state(qrs_pool pool, const int32_t *slots, int n, float *S_out, int space,
                      hipStream_t stream);

/*
 * One GDN decode step on n slots x H heads, in place (HTML section 3.1,
 * Eq.(1), Lambda = alpha I):
 *   q, k, v: FP32 [n][H][128] in model order; alpha, beta: FP32 [n][H];
 *   o: FP32 [n][H][128] output, model value order, o = S_t^T q from the FP32
 *   state of this step before requantization.
 * Compressed pools: dequantize -> FP32 update and readout -> requantize
 * (one fused kernel); FP32 pools: the same update on the FP32 state.
 */
int qrs_gdn_decode_step(qrs_pool pool, const int32_t *slots, int n, const float *q,
                        const float *k, const float *v, const float *alpha, const float *beta,
                        float *o, hipStream_t stream);

/*
 * One KDA decode step: as qrs_gdn_decode_step with per-key-channel decay
 * Lambda = diag(exp(g)) (HTML section 3.1); g: FP32 [n][H][128] log-decay in
 * model key order (exp is evaluated on the device).
 */
int qrs_kda_decode_step(qrs_pool pool, const int32_t *slots, int n, const float *q,
                        const float *k, const float *v, const float *g, const float *beta,
                        float *o, hipStream_t stream);

/*
 * General decode step: GDN (kind 0) or KDA (kind 1) on heads
 * [head_begin, head_begin + head_count) of n slots, with q, k, v and o in
 * FP32 (io_dtype 0) or bf16 (io_dtype 1; inputs widen exactly to FP32, o is
 * rounded to nearest even from the FP32 readout).  Operands keep their full
 * [n][H][128] layout (gate: alpha [n][H] or g [n][H][128], FP32; beta [n][H],
 * FP32) and only the selected heads are read and written, so one slot can
 * hold GDN heads and KDA heads updated by two calls (the mixed-pool reading
 * of a GDN/KDA model).  The arithmetic is that of qrs_gdn_decode_step /
 * qrs_kda_decode_step, which are this call with io_dtype 0 and all heads.
 * QRS_EINVAL: kind or io_dtype not 0/1, an empty or out-of-range head range.
 * QRS_EUNSUPPORTED: bf16 I/O on an FP32 pool.
 */
int qrs_decode_step_ex(qrs_pool pool, int kind, int io_dtype, const int32_t *slots, int n,
                       int head_begin, int head_count, const void *q, const void *k, const void *v,
                       const float *gate, const float *beta, void *o, hipStream_t stream);

/*
 * A GDN decode step and a KDA decode step on disjoint slots of one pool, as
 * one call: the two request groups of a model with GDN and KDA layers, or of a
 * pool whose slots serve both kinds (one packed cache per request slot, DAMP
 * arXiv HTML, Appendix A.5 "Persistent representation"; the updates of
 * section 3.1 Eq.(1) and the v2 notes' Eqs.(5)-(6), as in
 * qrs_gdn_decode_step and qrs_kda_decode_step).  The results, outputs and
 * stored bytes, are those of qrs_gdn_decode_step(pool, slots_gdn, n_gdn, ...)
 * followed by qrs_kda_decode_step(pool, slots_kda, n_kda, ...) on the same
 * stream; on a QRS_FMT_I8F16 pool the two run in one kernel launch, which pays
 * the launch's ramp and drain once (small grids and the other formats make
 * the two calls), and deals each group's slots whole to the XCDs, which
 * suits slots scattered over the pool; the results do not depend on it.  Arguments of each group as for those calls (FP32, all
 * heads); a group with n = 0 may pass NULL pointers.  A slot id in both groups
 * is undefined behaviour (the two updates of its units would race).
 * QRS_EINVAL: a NULL pool, a negative n, a NULL pointer of a non-empty group,
 * or (n_gdn + n_kda) * num_heads beyond 2^31 - 1.  Nothing is enqueued on an
 * error return.
 */
int qrs_decode_step_pair(qrs_pool pool, const int32_t *slots_gdn, int n_gdn, const float *q_gdn,
                         const float *k_gdn, const float *v_gdn, const float *alpha,
                         const float *beta_gdn, float *o_gdn, const int32_t *slots_kda, int n_kda,
                         const float *q_kda, const float *k_kda, const float *v_kda, const float *g,
                         const float *beta_kda, float *o_kda, hipStream_t stream);

/*
 * Per-window quantization ("LeapQuant: Efficient Linear Attention with
 * Accurate Recurrent State Quantization", section 3.2, Figure 2; buffer size
 * of section 4.3) on a QRS_FMT_I8F16 pool.  The stored state of a slot stays
 * fixed for `window` tokens (1..32; the pages use 16 and find no gain at 32).  Each token of the
 * window is recorded in a caller-owned update buffer with k and v rounded to
 * FP16 (nearest even), KDA's decay factors exp(g) taken in FP64 and rounded
 * once to FP16 (nearest even), and beta and GDN's alpha in FP32; the output of token j
 * is that of the FP32 recurrence of qrs_gdn_decode_step / qrs_kda_decode_step
 * started from the dequantized window-start state and run through the
 * window's tokens 0..j (their recorded values), read out with this token's q.  The
 * token at position window - 1 writes the requantized end state into the
 * pool, which starts the next window; the others write only their record.
 *   kind: 0 GDN (gate = alpha [n][H]), 1 KDA (gate = g [n][H][128]);
 *   buffer: device memory of >= qrs_window_buffer_bytes(kind, num_slots,
 *     num_heads, window) bytes, 16-byte aligned, laid out as
 *     [num_slots][num_heads][window] records of 528 B (GDN: k FP16[128],
 *     v FP16[128], beta, alpha) or 784 B (KDA: k, v, exp(g) FP16[128], beta);
 *   pos: int32 [n] device, the index of this token in slot b's window.
 *     Calls must visit positions 0, 1, ..., window - 1 of a slot in order
 *     (position 0 starts from the pool's stored state); a slot id or
 *     position out of range leaves everything untouched and gives NaN
 *     outputs.
 * q, k, v, o: FP32 [n][H][128] as for the other decode calls.
 * Scheduling: the window's last token replays the window's updates and takes
 * several times longer than the others.  When n <= 1024 and the first, middle
 * and last requests (pos[0], pos[n / 2], pos[n - 1]) are not all at one
 * position, the kernel runs the requests at position window - 1 first and the
 * rest after them, each part in batch order; other calls run in batch order,
 * where listing the window-end requests first has the same effect.  The
 * results do not depend on the order.
 * QRS_EUNSUPPORTED on other pool formats.
 */
size_t qrs_window_buffer_bytes(int kind, int num_slots, int num_heads, int window);
int qrs_window_decode_step(qrs_pool pool, int kind, int window, void *buffer, size_t buffer_bytes,
                           const int32_t *slots, const int32_t *pos, int n, const float *q,
                           const float *k, const float *v, const float *gate, const float *beta,
                           float *o, hipStream_t stream);

/*
 * Chunked prefill with GDN gating, writing the compressed state (DAMP arXiv
 * HTML, Appendix A.5 "Prefill path"; v2 reading notes, section 2.2): for each
 * of n sequences (slots[b]) x H heads, runs T tokens through the recurrence
 * of qrs_gdn_decode_step in FP32 one chunk of `chunk` tokens at a time (the
 * last chunk may be shorter) and writes the chunk-final state into the slot
 * at every chunk end; the next chunk continues from the stored (requantized)
 * state.  Outputs come from the FP32 state inside the chunk.
 *   q, k, v: [n][T][H][128] in model key order, FP32 (in_dtype 0) or bf16
 *            (in_dtype 1, widened exactly to FP32 on load);
 *   alpha, beta: FP32 [n][T][H];  o: FP32 [n][T][H][128], model value order;
 *   chunk: 1..64;  init_from_pool: 1 = start from the slot's stored state,
 *   0 = start from zero.
 * All contractions run on FP32 matrix cores.  FP32 pools store the chunk-end
 * state uncompressed (compression disabled); QRS_FMT_U8H16 pools write and
 * read it back through the block-32 transform.  Out-of-range slot ids leave
 * their state untouched and fill their outputs with NaN.  n = 0 or T = 0 is
 * a no-op.
 */
int qrs_chunked_prefill(qrs_pool pool, const int32_t *slots, int n, int T, int chunk,
                        int in_dtype, const void *q, const void *k, const void *v,
                        const float *alpha, const float *beta, float *o, int init_from_pool,
                        hipStream_t stream);

/*
 * Key-channel selection: the offline construction of perm (DAMP arXiv HTML,
 * section 4 "Key-channel budget", "Accumulated-error risk", "Budgeted
 * selection", Eqs.(7)-(10); Appendix A.2 Eqs.(13)-(15); Appendix A.4
 * Algorithm 1; v2 reading notes, section 2.5).  Calibration statistics come
 * from FP32 state trajectories; the result is the perm of
 * qrs_create_state_pool.  These calls need no pool and run on the current
 * device.
 */

/*
 * Quantization-error energy of every key channel of n calibration states
 * (Eq.(14) integrand; v2 notes e_{t,u}):
 *   S: FP32 [n][H][128][128], model coordinates, 16-byte aligned;
 *   smooth: FP32 [H][128] value-column scales c (NULL = ones), 16-byte aligned;
 *   e: FP64 [n][H][128] output,
 *   e[s][h][u] = sum_j (Q(S[s][h][u][j] / c[h][j]) * c[h][j] - S[s][h][u][j])^2
 * where Q quantizes and dequantizes each 32-value group with the INT8 codec of
 * qrs_store_state (every row is measured under INT8, the tier the selection
 * protects channels from).  The squares are summed in FP64.
 */
int qrs_channel_error(int n, int num_heads, const float *S, const float *smooth, double *e,
                      hipStream_t stream);

/*
 * Finite-horizon persistence weight of each sampled state write (v2 notes
 * section 2.5):
 *   W[s][h][u] = 1 + sum_{j=1..horizon} prod_{r=1..j} a[q][t+r][h][u]^2,
 * with q = sample_seq[s], t = sample_t[s]; the sum stops at the end of the
 * trajectory (t + j <= T - 1).
 *   a: FP32 [n_seq][T][H][128] per-step decays (GDN: alpha repeated over
 *      the key channels; KDA: exp(g));
 *   sample_seq, sample_t: int32 [n] device arrays;  W: FP64 [n][H][128].
 * A sample whose sequence or step is out of range gets NaN.  FP64 products
 * and sums in step order.
 */
int qrs_persistence_window(int n_seq, int T, int num_heads, const float *a, int n,
                           const int32_t *sample_seq, const int32_t *sample_t, int horizon,
                           double *W, hipStream_t stream);

/*
 * Geometric-mean persistence (Eq.(15)):
 *   a_eff[h][u] = exp(sum_s weight[s] log a[q_s][t_s][h][u]),
 *   P[h][u] = 1 / max(1 - a_eff^2, tau)    (the pages use tau = 1e-4),
 * weight: FP64 [n] device (the domain-balanced mean of Eq.(13) has
 * weight[s] = 1 / (|D| |Omega_d(s)|)); samples with weight 0 are skipped; an
 * out-of-range sample makes its head's P NaN.  P: FP64 [H][128].
 */
int qrs_persistence_geometric(int n_seq, int T, int num_heads, const float *a, int n,
                              const int32_t *sample_seq, const int32_t *sample_t,
                              const double *weight, double tau, double *P, hipStream_t stream);

/*
 * Key-channel risk C: FP64 [H][128] (device), from e [n][H][128] and weight
 * [n]; exactly one of W and P is given:
 *   W (v2 notes):  C[h][u] = sum_s weight[s] e[s][h][u] W[s][h][u];
 *   P (Eq.(10) with Eqs.(14)-(15)):  C[h][u] = (sum_s weight[s] e[s][h][u]) P[h][u].
 * Sums run in sample order, without fused multiply-adds.
 */
int qrs_channel_scores(int n, int num_heads, const double *e, const double *W, const double *P,
                       const double *weight, double *C, hipStream_t stream);

/*
 * Protected channels and the permutation (Algorithm 1), on the host:
 * score_host FP64 [H][128] (host), perm_host int32 [H][128] (host output).
 * Per head, the k_hi channels of largest score (equal scores: lower index
 * first; NaN ranks last) are placed first, then the rest, each in ascending
 * channel order.  k_hi is 16 for the pool formats of this library.
 */
int qrs_select_protected_channels(int num_heads, const double *score_host, int k_hi,
                                  int32_t *perm_host);

/*
 * Which kernel the QRS_FMT_I8F16 decode steps (qrs_gdn_decode_step,
 * qrs_kda_decode_step, qrs_decode_step_ex) launch.  Every step of the update
 * stays within a value column (DAMP HTML, section 3.1 Eq.(1); the v2 notes'
 * 32-value groups run along the value axis), so a unit can be split into two
 * workgroups, one per 64-column half, with no exchange between them.  Both
 * kernels perform the same operations in the same order and give the same
 * bits; they differ only in speed:
 *   QRS_DECODE_SPLIT_WHOLE:  one workgroup per (slot, head) unit;
 *   QRS_DECODE_SPLIT_HALVES: two workgroups per unit, for grids too small to
 *     fill the GPU (a whole-unit workgroup's lifetime then sets the step);
 *   QRS_DECODE_SPLIT_AUTO (the default): the halves below 1,024 units per call
 *     (n * head count), where on MI355X they are faster; above, whole units,
 *     and for grids of at least 4/3 of a generation of resident workgroups
 *     the last eighth of a generation's units as halves, at the end of the
 *     same launch, which shortens its drain.
 * The setting is process-wide, applies to calls enqueued after it returns,
 * and is a tuning choice only.  Returns the previous mode (>= 0), or
 * QRS_EINVAL for another value (the setting is then unchanged).  Other pool
 * formats and the per-window step ignore it.
 */
enum {
    QRS_DECODE_SPLIT_AUTO = 0,
    QRS_DECODE_SPLIT_WHOLE = 1,
    QRS_DECODE_SPLIT_HALVES = 2
};
int qrs_set_decode_split(int mode);

/* Name of a status code (static string). */
const char *qrs_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* QRS_H */
