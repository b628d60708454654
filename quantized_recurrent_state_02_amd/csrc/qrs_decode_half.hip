// qrs_decode_half.hip -- the fused compressed-state decode step (GDN and KDA,
// INT8 tier) with two workgroups per (slot, head) unit, one per 64-column half
// of the value axis, for grids too small to fill the GPU.  The per-half body
// and its derivation are in qrs_decode_half.h.
#include "qrs_decode_half.h"

namespace qrs {

using half_unit::HCOLS;

// KIND 0: GDN (gate = alpha [n][H]); KIND 1: KDA (gate = g [n][H][128]).
// IO 0: q, k, v, o in FP32; IO 1: in bf16 (gates and beta stay FP32).
template <int KIND, int IO>
__global__ __launch_bounds__(THREADS) void decode_half_kernel(
    PoolView pool, const int32_t *__restrict__ slots, int units, int h0, int hc,
    const void *__restrict__ q, const void *__restrict__ k, const void *__restrict__ v,
    const float *__restrict__ gate, const float *__restrict__ beta, void *__restrict__ o) {
    __shared__ float s_k[DK];
    __shared__ float s_q[DK];
    __shared__ float s_dec[DK];
    __shared__ float s_bd[HCOLS];
    __shared__ float s_vp[HCOLS];
    __shared__ float s_kraw[DK];
    __shared__ float s_qraw[DK];
    __shared__ float s_graw[DK];
    __shared__ float s_qk[2];
    __shared__ float4 red_w[16][HCOLS / 4];
    __shared__ float4 red_z[16][HCOLS / 4];

    const HalfLds L{s_k, s_q, s_dec, s_bd, s_vp, s_kraw, s_qraw, s_graw, s_qk, &red_w[0][0], &red_z[0][0]};
    decode_half_unit<KIND, IO>(pool, slots, units, h0, hc, (int)blockIdx.x, 0, q, k, v, gate, beta,
                               o, L);
}

// Launcher: units = n * hc; the grid holds whole groups of 16 workgroups (8
// units x 2 halves), so the rounded-up tail exits at once.
hipError_t launch_decode_half(int kind, int io, const PoolView &pool, const int32_t *slots, int n,
                              int h0, int hc, const void *q, const void *k, const void *v,
                              const float *gate, const float *beta, void *o, hipStream_t stream) {
    const int units = n * hc;
    const int groups = (units + 7) / 8;
    dim3 grid((unsigned)(16 * groups)), block(THREADS);
#define QRS_HALF_CASE(K, I)                                                                      \
    if (kind == K && io == I) {                                                                  \
        hipLaunchKernelGGL((decode_half_kernel<K, I>), grid, block, 0, stream, pool, slots,      \
                           units, h0, hc, q, k, v, gate, beta, o);                               \
        return hipGetLastError();                                                                \
    }
    QRS_HALF_CASE(0, 0)
    QRS_HALF_CASE(1, 0)
    QRS_HALF_CASE(0, 1)
    QRS_HALF_CASE(1, 1)
#undef QRS_HALF_CASE
    return hipErrorInvalidValue;
}

}  // namespace qrs
