// qrs_api.hip -- the C ABI declared in include/qrs.h: argument validation,
// pool handles and kernel launches.  Every check happens on the host before
// anything is enqueued, so an error return leaves the stream untouched.
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <new>
#include <algorithm>
#include <atomic>
#include <numeric>
#include <vector>

#include "../../include/qrs.h"
#include "qrs_internal.h"
#include "qrs_window.h"

namespace qrs {
hipError_t launch_decode_half(int kind, int io, const PoolView &pool, const int32_t *slots, int n,
                              int h0, int hc, const void *q, const void *k, const void *v,
                              const float *gate, const float *beta, void *o, hipStream_t stream);
hipError_t launch_decode_packed(int kind, int codec, int io, const PoolView &pool,
                                const int32_t *slots, int n, int h0, int hc, const void *q,
                                const void *k, const void *v, const float *gate, const float *beta,
                                void *o, bool half_tail, hipStream_t stream);
hipError_t launch_decode_pair(const PoolView &pool, const int32_t *slots_g, int n_g,
                              const float *q_g, const float *k_g, const float *v_g,
                              const float *alpha, const float *beta_g, float *o_g,
                              const int32_t *slots_k, int n_k, const float *q_k, const float *k_k,
                              const float *v_k, const float *g, const float *beta_k, float *o_k,
                              bool half_tail, hipStream_t stream);
hipError_t launch_decode_f32(int kind, const PoolView &pool, const int32_t *slots, int n, int h0,
                             int hc, const float *q, const float *k, const float *v,
                             const float *gate, const float *beta, float *o, hipStream_t stream);
hipError_t launch_store(int fmt, const PoolView &pool, const int32_t *slots, int n, const float *S,
                        int space, hipStream_t stream);
hipError_t launch_dequant(int fmt, const PoolView &pool, const int32_t *slots, int n, float *S,
                          int space, hipStream_t stream);
hipError_t launch_prefill(int fmt, const PoolView &pool, const int32_t *slots, int n, int T,
                          int chunk, int in_bf16, const void *q, const void *k, const void *v,
                          const float *alpha, const float *beta, float *o, int init_from_pool,
                          hipStream_t stream);
hipError_t launch_window(int kind, const PoolView &pool, uint8_t *buf, int window,
                         const int32_t *slots, const int32_t *pos, int n, const float *q,
                         const float *k, const float *v, const float *gate, const float *beta,
                         float *o, hipStream_t stream);
hipError_t launch_channel_error(int n, int num_heads, const float *S, const float *smooth,
                                double *e, hipStream_t stream);
hipError_t launch_persistence_window(int n_seq, int T, int num_heads, const float *a, int n,
                                     const int32_t *sample_seq, const int32_t *sample_t,
                                     int horizon, double *W, hipStream_t stream);
hipError_t launch_persistence_geometric(int n_seq, int T, int num_heads, const float *a, int n,
                                        const int32_t *sample_seq, const int32_t *sample_t,
                                        const double *weight, double tau, double *P,
                                        hipStream_t stream);
hipError_t launch_channel_scores(int n, int num_heads, const double *e, const double *W,
                                 const double *P, const double *weight, double *C,
                                 hipStream_t stream);
}  // namespace qrs

struct qrs_pool_s {
    int fmt;
    int num_slots;
    int num_heads;
    size_t unit_bytes;
    size_t perm_offset;
    size_t smooth_offset;
    size_t total_bytes;
    uint8_t *base;
    int device;
};

namespace {

constexpr size_t kAlign = 256;

size_t round_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool shape_ok(int fmt, int d_k, int d_v, int k_hi, int group) {
    if (d_k != qrs::DK || d_v != qrs::DV) return false;
    if (fmt == QRS_FMT_I8F16 || fmt == QRS_FMT_U8H16) return k_hi == qrs::KHI && group == qrs::GRP;
    if (fmt == QRS_FMT_FP32) return k_hi == 0 && group == 0;
    return false;
}

// Layout of a pool; returns false for invalid sizes.
bool layout(int fmt, int num_slots, int num_heads, size_t *unit_bytes, size_t *perm_off,
            size_t *smooth_off, size_t *total) {
    if (num_slots <= 0 || num_heads <= 0) return false;
    const size_t ub = fmt == QRS_FMT_FP32 ? (size_t)qrs::F32_UNIT_BYTES : (size_t)qrs::UNIT_BYTES;
    const size_t units = (size_t)num_slots * (size_t)num_heads;
    if (units > ((size_t)1 << 40) / ub) return false;
    const size_t meta = round_up((size_t)num_heads * qrs::DK * sizeof(int32_t));
    *unit_bytes = ub;
    *perm_off = round_up(units * ub);
    *smooth_off = *perm_off + meta;
    *total = *smooth_off + round_up((size_t)num_heads * qrs::DV * sizeof(float));
    return true;
}

qrs::PoolView view(const qrs_pool_s *p) {
    qrs::PoolView v;
    v.base = p->base;
    v.perm = reinterpret_cast<const int32_t *>(p->base + p->perm_offset);
    v.smooth = reinterpret_cast<const float *>(p->base + p->smooth_offset);
    v.num_slots = p->num_slots;
    v.num_heads = p->num_heads;
    return v;
}

// Launches must happen with the pool's device current.
struct DeviceGuard {
    int prev = -1;
    bool ok = true;
    explicit DeviceGuard(int dev) {
        if (hipGetDevice(&prev) != hipSuccess) {
            ok = false;
            return;
        }
        if (prev != dev && hipSetDevice(dev) != hipSuccess) ok = false;
    }
    ~DeviceGuard() {
        int cur = -1;
        if (prev >= 0 && hipGetDevice(&cur) == hipSuccess && cur != prev) (void)hipSetDevice(prev);
    }
};

// Which INT8-tier decode kernel runs: one workgroup per unit, or two per unit
// (value-column halves) for grids too small to fill the GPU.
// QRS_DECODE_SPLIT_AUTO picks the halves below kDecodeSplitUnits units, and
// above lets the whole-unit kernel end a large grid with half-unit
// workgroups; QRS_DECODE_SPLIT_WHOLE uses whole-unit workgroups only.  At
// exactly 1,024 units the better kernel depends on the layout on MI355X:
// halves 11.25 against 11.55 us for 32 slots x 32 heads, but 11.66 against
// 10.87 for 256 slots x 4 heads (scattered units), so whole units stay there.
std::atomic<int> g_decode_split{QRS_DECODE_SPLIT_AUTO};
constexpr int kDecodeSplitUnits = 1024;

bool use_half_kernel(int units) {
    const int mode = g_decode_split.load(std::memory_order_relaxed);
    if (mode == QRS_DECODE_SPLIT_AUTO) return units < kDecodeSplitUnits;
    return mode == QRS_DECODE_SPLIT_HALVES;
}

int decode_common(int kind, int io, qrs_pool pool, const int32_t *slots, int n, int h0, int hc,
                  const void *q, const void *k, const void *v, const float *gate,
                  const float *beta, void *o, hipStream_t stream) {
    if (!pool || n < 0 || (kind != 0 && kind != 1) || (io != 0 && io != 1)) return QRS_EINVAL;
    if (h0 < 0 || hc < 1 || h0 > pool->num_heads - hc) return QRS_EINVAL;
    if (pool->fmt == QRS_FMT_FP32 && io != 0) return QRS_EUNSUPPORTED;
    if (n == 0) return QRS_OK;
    if (!slots || !q || !k || !v || !gate || !beta || !o) return QRS_EINVAL;
    if ((size_t)n * (size_t)pool->num_heads > 0x7fffffffu) return QRS_EINVAL;
    DeviceGuard g(pool->device);
    if (!g.ok) return QRS_EDEVICE;
    const qrs::PoolView pv = view(pool);
    hipError_t e =
        pool->fmt == QRS_FMT_FP32
            ? qrs::launch_decode_f32(kind, pv, slots, n, h0, hc, static_cast<const float *>(q),
                                     static_cast<const float *>(k), static_cast<const float *>(v),
                                     gate, beta, static_cast<float *>(o), stream)
        : pool->fmt == QRS_FMT_I8F16 && use_half_kernel(n * hc)
            ? qrs::launch_decode_half(kind, io, pv, slots, n, h0, hc, q, k, v, gate, beta, o, stream)
            : qrs::launch_decode_packed(
                  kind, pool->fmt == QRS_FMT_U8H16 ? 1 : 0, io, pv, slots, n, h0, hc, q, k, v, gate,
                  beta, o,
                  g_decode_split.load(std::memory_order_relaxed) == QRS_DECODE_SPLIT_AUTO, stream);
    return e == hipSuccess ? QRS_OK : QRS_EDEVICE;
}

}  // namespace

extern "C" {

size_t qrs_state_pool_bytes(int fmt, int num_slots, int num_heads, int d_k, int d_v, int k_hi,
                            int group) {
    if (!shape_ok(fmt, d_k, d_v, k_hi, group)) return 0;
    size_t ub, po, so, total;
    if (!layout(fmt, num_slots, num_heads, &ub, &po, &so, &total)) return 0;
    return total;
}

int qrs_create_state_pool(int fmt, int num_slots, int num_heads, int d_k, int d_v, int k_hi,
                          int group, void *dev_mem, size_t dev_bytes, const int32_t *perm_host,
                          const float *smooth_host, hipStream_t stream, qrs_pool *out) {
    if (!out) return QRS_EINVAL;
    *out = nullptr;
    if (fmt != QRS_FMT_FP32 && fmt != QRS_FMT_I8F16 && fmt != QRS_FMT_U8H16) return QRS_EINVAL;
    if (!shape_ok(fmt, d_k, d_v, k_hi, group)) return QRS_EUNSUPPORTED;
    size_t ub, po, so, total;
    if (!layout(fmt, num_slots, num_heads, &ub, &po, &so, &total)) return QRS_EINVAL;
    if (!dev_mem || dev_bytes < total) return QRS_EINVAL;
    if (reinterpret_cast<uintptr_t>(dev_mem) % kAlign != 0) return QRS_EINVAL;

    std::vector<int32_t> perm((size_t)num_heads * qrs::DK);
    std::vector<float> smooth((size_t)num_heads * qrs::DV);
    for (int h = 0; h < num_heads; ++h) {
        std::vector<char> seen(qrs::DK, 0);
        for (int i = 0; i < qrs::DK; ++i) {
            const int32_t p = perm_host ? perm_host[(size_t)h * qrs::DK + i] : i;
            if (p < 0 || p >= qrs::DK || seen[p]) return QRS_EINVAL;
            seen[p] = 1;
            perm[(size_t)h * qrs::DK + i] = p;
        }
        for (int j = 0; j < qrs::DV; ++j) {
            const float c = smooth_host ? smooth_host[(size_t)h * qrs::DV + j] : 1.0f;
            if (!(c > 0.0f) || !std::isfinite(c)) return QRS_EINVAL;
            smooth[(size_t)h * qrs::DV + j] = c;
        }
    }
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return QRS_EDEVICE;
    qrs_pool_s *p = new (std::nothrow) qrs_pool_s;
    if (!p) return QRS_EDEVICE;
    p->fmt = fmt;
    p->num_slots = num_slots;
    p->num_heads = num_heads;
    p->unit_bytes = ub;
    p->perm_offset = po;
    p->smooth_offset = so;
    p->total_bytes = total;
    p->base = static_cast<uint8_t *>(dev_mem);
    p->device = dev;
    // Synchronous copies of the small tables (the host vectors die on return),
    // then the state region is zero-filled on the caller's stream.
    if (hipMemcpy(p->base + po, perm.data(), perm.size() * sizeof(int32_t),
                  hipMemcpyHostToDevice) != hipSuccess ||
        hipMemcpy(p->base + so, smooth.data(), smooth.size() * sizeof(float),
                  hipMemcpyHostToDevice) != hipSuccess ||
        hipMemsetAsync(p->base, 0, po, stream) != hipSuccess) {
        delete p;
        return QRS_EDEVICE;
    }
    *out = p;
    return QRS_OK;
}

int qrs_destroy_state_pool(qrs_pool pool) {
    delete pool;
    return QRS_OK;
}

int qrs_pool_info(qrs_pool pool, int *fmt, int *num_slots, int *num_heads, size_t *unit_bytes,
                  size_t *perm_offset, size_t *smooth_offset) {
    if (!pool) return QRS_EINVAL;
    if (fmt) *fmt = pool->fmt;
    if (num_slots) *num_slots = pool->num_slots;
    if (num_heads) *num_heads = pool->num_heads;
    if (unit_bytes) *unit_bytes = pool->unit_bytes;
    if (perm_offset) *perm_offset = pool->perm_offset;
    if (smooth_offset) *smooth_offset = pool->smooth_offset;
    return QRS_OK;
}

int qrs_store_state(qrs_pool pool, const int32_t *slots, int n, const float *S, int space,
                    hipStream_t stream) {
    if (!pool || n < 0 || (space != QRS_SPACE_MODEL && space != QRS_SPACE_STORED))
        return QRS_EINVAL;
    if (n == 0) return QRS_OK;
    if (!slots || !S) return QRS_EINVAL;
    if ((size_t)n * (size_t)pool->num_heads > 0x7fffffffu) return QRS_EINVAL;
    DeviceGuard g(pool->device);
    if (!g.ok) return QRS_EDEVICE;
    return qrs::launch_store(pool->fmt, view(pool), slots, n, S, space, stream) == hipSuccess
               ? QRS_OK
               : QRS_EDEVICE;
}

int qrs_dequant_state(qrs_pool pool, const int32_t *slots, int n, float *S_out, int space,
                      hipStream_t stream) {
    if (!pool || n < 0 || (space != QRS_SPACE_MODEL && space != QRS_SPACE_STORED))
        return QRS_EINVAL;
    if (n == 0) return QRS_OK;
    if (!slots || !S_out) return QRS_EINVAL;
    if ((size_t)n * (size_t)pool->num_heads > 0x7fffffffu) return QRS_EINVAL;
    DeviceGuard g(pool->device);
    if (!g.ok) return QRS_EDEVICE;
    return qrs::launch_dequant(pool->fmt, view(pool), slots, n, S_out, space, stream) == hipSuccess
               ? QRS_OK
               : QRS_EDEVICE;
}

int qrs_gdn_decode_step(qrs_pool pool, const int32_t *slots, int n, const float *q,
                        const float *k, const float *v, const float *alpha, const float *beta,
                        float *o, hipStream_t stream) {
    return decode_common(0, 0, pool, slots, n, 0, pool ? pool->num_heads : 1, q, k, v, alpha, beta,
                         o, stream);
}

int qrs_kda_decode_step(qrs_pool pool, const int32_t *slots, int n, const float *q,
                        const float *k, const float *v, const float *g, const float *beta,
                        float *o, hipStream_t stream) {
    return decode_common(1, 0, pool, slots, n, 0, pool ? pool->num_heads : 1, q, k, v, g, beta, o,
                         stream);
}

int qrs_decode_step_pair(qrs_pool pool, const int32_t *slots_gdn, int n_gdn, const float *q_gdn,
                         const float *k_gdn, const float *v_gdn, const float *alpha,
                         const float *beta_gdn, float *o_gdn, const int32_t *slots_kda, int n_kda,
                         const float *q_kda, const float *k_kda, const float *v_kda, const float *g,
                         const float *beta_kda, float *o_kda, hipStream_t stream) {
    if (!pool || n_gdn < 0 || n_kda < 0) return QRS_EINVAL;
    if (n_gdn > 0 && (!slots_gdn || !q_gdn || !k_gdn || !v_gdn || !alpha || !beta_gdn || !o_gdn))
        return QRS_EINVAL;
    if (n_kda > 0 && (!slots_kda || !q_kda || !k_kda || !v_kda || !g || !beta_kda || !o_kda))
        return QRS_EINVAL;
    if (((size_t)n_gdn + (size_t)n_kda) * (size_t)pool->num_heads > 0x7fffffffu) return QRS_EINVAL;
    const int units = (n_gdn + n_kda) * pool->num_heads;
    const int mode = g_decode_split.load(std::memory_order_relaxed);
    if (pool->fmt != QRS_FMT_I8F16 || n_gdn == 0 || n_kda == 0 ||
        mode == QRS_DECODE_SPLIT_HALVES ||
        (mode == QRS_DECODE_SPLIT_AUTO && units < kDecodeSplitUnits)) {
        // the two calls, as a caller would make them (every argument is valid
        // by the checks above, so neither returns an argument error)
        const int st = decode_common(0, 0, pool, slots_gdn, n_gdn, 0, pool->num_heads, q_gdn, k_gdn,
                                     v_gdn, alpha, beta_gdn, o_gdn, stream);
        if (st != QRS_OK) return st;
        return decode_common(1, 0, pool, slots_kda, n_kda, 0, pool->num_heads, q_kda, k_kda, v_kda,
                             g, beta_kda, o_kda, stream);
    }
    DeviceGuard dg(pool->device);
    if (!dg.ok) return QRS_EDEVICE;
    return qrs::launch_decode_pair(view(pool), slots_gdn, n_gdn, q_gdn, k_gdn, v_gdn, alpha,
                                   beta_gdn, o_gdn, slots_kda, n_kda, q_kda, k_kda, v_kda, g,
                                   beta_kda, o_kda, mode == QRS_DECODE_SPLIT_AUTO,
                                   stream) == hipSuccess
               ? QRS_OK
               : QRS_EDEVICE;
}

int qrs_decode_step_ex(qrs_pool pool, int kind, int io_dtype, const int32_t *slots, int n,
                       int head_begin, int head_count, const void *q, const void *k, const void *v,
                       const float *gate, const float *beta, void *o, hipStream_t stream) {
    return decode_common(kind, io_dtype, pool, slots, n, head_begin, head_count, q, k, v, gate,
                         beta, o, stream);
}

size_t qrs_window_buffer_bytes(int kind, int num_slots, int num_heads, int window) {
    if ((kind != 0 && kind != 1) || num_slots <= 0 || num_heads <= 0 || window < 1 || window > 32)
        return 0;
    const size_t rec = (size_t)qrs::window_record_bytes(kind);
    const size_t units = (size_t)num_slots * (size_t)num_heads;
    if (units > ((size_t)1 << 40) / (rec * (size_t)window)) return 0;
    return units * (size_t)window * rec;
}

int qrs_window_decode_step(qrs_pool pool, int kind, int window, void *buffer, size_t buffer_bytes,
                           const int32_t *slots, const int32_t *pos, int n, const float *q,
                           const float *k, const float *v, const float *gate, const float *beta,
                           float *o, hipStream_t stream) {
    if (!pool || n < 0 || (kind != 0 && kind != 1) || window < 1 || window > 32) return QRS_EINVAL;
    if (pool->fmt != QRS_FMT_I8F16) return QRS_EUNSUPPORTED;
    const size_t need = qrs_window_buffer_bytes(kind, pool->num_slots, pool->num_heads, window);
    if (!buffer || need == 0 || buffer_bytes < need) return QRS_EINVAL;
    if (reinterpret_cast<uintptr_t>(buffer) % 16 != 0) return QRS_EINVAL;
    if (n == 0) return QRS_OK;
    if (!slots || !pos || !q || !k || !v || !gate || !beta || !o) return QRS_EINVAL;
    if ((size_t)n * (size_t)pool->num_heads > 0x7fffffffu) return QRS_EINVAL;
    DeviceGuard g(pool->device);
    if (!g.ok) return QRS_EDEVICE;
    return qrs::launch_window(kind, view(pool), static_cast<uint8_t *>(buffer), window, slots, pos,
                              n, q, k, v, gate, beta, o, stream) == hipSuccess
               ? QRS_OK
               : QRS_EDEVICE;
}

int qrs_chunked_prefill(qrs_pool pool, const int32_t *slots, int n, int T, int chunk,
                        int in_dtype, const void *q, const void *k, const void *v,
                        const float *alpha, const float *beta, float *o, int init_from_pool,
                        hipStream_t stream) {
    if (!pool || n < 0 || T < 0 || chunk < 1 || chunk > 64 || (in_dtype != 0 && in_dtype != 1) ||
        (init_from_pool != 0 && init_from_pool != 1))
        return QRS_EINVAL;
    if (n == 0 || T == 0) return QRS_OK;
    if (!slots || !q || !k || !v || !alpha || !beta || !o) return QRS_EINVAL;
    if ((size_t)n * (size_t)pool->num_heads > 0x7fffffffu || T > (1 << 24)) return QRS_EINVAL;
    DeviceGuard g(pool->device);
    if (!g.ok) return QRS_EDEVICE;
    return qrs::launch_prefill(pool->fmt, view(pool), slots, n, T, chunk, in_dtype, q, k, v, alpha,
                               beta, o, init_from_pool, stream) == hipSuccess
               ? QRS_OK
               : QRS_EDEVICE;
}

int qrs_channel_error(int n, int num_heads, const float *S, const float *smooth, double *e,
                      hipStream_t stream) {
    if (n < 0 || num_heads < 1) return QRS_EINVAL;
    if (n == 0) return QRS_OK;
    if (!S || !e) return QRS_EINVAL;
    if ((reinterpret_cast<uintptr_t>(S) | reinterpret_cast<uintptr_t>(smooth)) % 16 != 0)
        return QRS_EINVAL;
    if ((size_t)n * (size_t)num_heads > 0x7fffffffu) return QRS_EINVAL;
    return qrs::launch_channel_error(n, num_heads, S, smooth, e, stream) == hipSuccess
               ? QRS_OK
               : QRS_EDEVICE;
}

int qrs_persistence_window(int n_seq, int T, int num_heads, const float *a, int n,
                           const int32_t *sample_seq, const int32_t *sample_t, int horizon,
                           double *W, hipStream_t stream) {
    if (n < 0 || n_seq < 1 || T < 1 || num_heads < 1 || horizon < 0) return QRS_EINVAL;
    if (n == 0) return QRS_OK;
    if (!a || !sample_seq || !sample_t || !W) return QRS_EINVAL;
    if ((size_t)n * (size_t)num_heads > 0x7fffffffu) return QRS_EINVAL;
    return qrs::launch_persistence_window(n_seq, T, num_heads, a, n, sample_seq, sample_t, horizon,
                                          W, stream) == hipSuccess
               ? QRS_OK
               : QRS_EDEVICE;
}

int qrs_persistence_geometric(int n_seq, int T, int num_heads, const float *a, int n,
                              const int32_t *sample_seq, const int32_t *sample_t,
                              const double *weight, double tau, double *P, hipStream_t stream) {
    if (n < 0 || n_seq < 1 || T < 1 || num_heads < 1 || !(tau > 0.0) || !std::isfinite(tau))
        return QRS_EINVAL;
    if (!P || (n > 0 && (!a || !sample_seq || !sample_t || !weight))) return QRS_EINVAL;
    return qrs::launch_persistence_geometric(n_seq, T, num_heads, a, n, sample_seq, sample_t,
                                             weight, tau, P, stream) == hipSuccess
               ? QRS_OK
               : QRS_EDEVICE;
}

int qrs_channel_scores(int n, int num_heads, const double *e, const double *W, const double *P,
                       const double *weight, double *C, hipStream_t stream) {
    if (n < 0 || num_heads < 1 || (W == nullptr) == (P == nullptr) || !C) return QRS_EINVAL;
    if (n > 0 && (!e || !weight)) return QRS_EINVAL;
    return qrs::launch_channel_scores(n, num_heads, e, W, P, weight, C, stream) == hipSuccess
               ? QRS_OK
               : QRS_EDEVICE;
}

int qrs_select_protected_channels(int num_heads, const double *score_host, int k_hi,
                                  int32_t *perm_host) {
    if (num_heads < 1 || k_hi < 0 || k_hi > qrs::DK || !score_host || !perm_host)
        return QRS_EINVAL;
    std::vector<int> order(qrs::DK);
    std::vector<char> chosen(qrs::DK);
    for (int h = 0; h < num_heads; ++h) {
        const double *sc = score_host + (size_t)h * qrs::DK;
        // a NaN score ranks below every number
        auto key = [&](int u) { return std::isnan(sc[u]) ? -INFINITY : sc[u]; };
        std::iota(order.begin(), order.end(), 0);
        std::stable_sort(order.begin(), order.end(),
                         [&](int x, int y) { return key(x) > key(y); });
        std::fill(chosen.begin(), chosen.end(), 0);
        for (int i = 0; i < k_hi; ++i) chosen[order[i]] = 1;
        int32_t *pm = perm_host + (size_t)h * qrs::DK;
        int pos = 0;
        for (int u = 0; u < qrs::DK; ++u)
            if (chosen[u]) pm[pos++] = u;
        for (int u = 0; u < qrs::DK; ++u)
            if (!chosen[u]) pm[pos++] = u;
    }
    return QRS_OK;
}

int qrs_set_decode_split(int mode) {
    if (mode != QRS_DECODE_SPLIT_AUTO && mode != QRS_DECODE_SPLIT_WHOLE &&
        mode != QRS_DECODE_SPLIT_HALVES)
        return QRS_EINVAL;
    return g_decode_split.exchange(mode, std::memory_order_relaxed);
}

const char *qrs_status_string(int status) {
    switch (status) {
    case QRS_OK: return "QRS_OK";
    case QRS_EINVAL: return "QRS_EINVAL: invalid argument";
    case QRS_EUNSUPPORTED: return "QRS_EUNSUPPORTED: unsupported shape or format";
    case QRS_EDEVICE: return "QRS_EDEVICE: HIP runtime error";
    default: return "unknown qrs status";
    }
}

}  // extern "C"
