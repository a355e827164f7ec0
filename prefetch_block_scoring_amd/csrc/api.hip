// extern "C" entry points of liboasis: argument checks, pointer resolution,
// stream / event ordering, then the kernel launchers.  The semantics of each
// call are documented in include/oasis.h.
#include "oasis_internal.h"

#include <cmath>
#include <cstdio>
#include <mutex>
#include <vector>

namespace oasis {

namespace {
thread_local std::string g_error;

struct DevInfo {
    int cu = 0;
};
std::mutex g_dev_mu;
std::vector<DevInfo> g_dev;

}  // namespace

void set_error(const std::string &msg) { g_error = msg; }
void clear_error() { g_error.clear(); }

int hip_check(hipError_t e, const char *what) {
    if (e == hipSuccess) return OASIS_OK;
    set_error(std::string(what) + ": " + hipGetErrorName(e) + " (" + hipGetErrorString(e) + ")");
    return OASIS_EHIP;
}

int device_cu_count() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
    std::lock_guard<std::mutex> lk(g_dev_mu);
    if ((int)g_dev.size() <= dev) g_dev.resize(dev + 1);
    if (g_dev[dev].cu == 0) {
        int cu = 0;
        if (hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cu <= 0)
            cu = 256;
        g_dev[dev].cu = cu;
    }
    return g_dev[dev].cu;
}

int device_view(const void *p, const void **out, const char *name) {
    hipPointerAttribute_t at;
    hipError_t e = hipPointerGetAttributes(&at, p);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        set_error(std::string(name) + ": not a HIP allocation (pageable host memory?)");
        return OASIS_EINVAL;
    }
    if (at.type == hipMemoryTypeDevice || at.type == hipMemoryTypeManaged) {
        *out = p;
        return OASIS_OK;
    }
    if (at.type == hipMemoryTypeHost) {
        void *dp = nullptr;
        e = hipHostGetDevicePointer(&dp, const_cast<void *>(p), 0);
        if (e != hipSuccess || dp == nullptr) {
            (void)hipGetLastError();
            set_error(std::string(name) + ": pinned host memory without a device mapping");
            return OASIS_EINVAL;
        }
        *out = dp;
        return OASIS_OK;
    }
    set_error(std::string(name) + ": not device or pinned host memory");
    return OASIS_EINVAL;
}

}  // namespace oasis

using namespace oasis;

#define FAIL(code, ...)                                   \
    do {                                                  \
        char _buf[512];                                   \
        snprintf(_buf, sizeof _buf, __VA_ARGS__);         \
        set_error(_buf);                                  \
        return (code);                                    \
    } while (0)

#define NEED(ptr)                                                         \
    do {                                                                  \
        if ((ptr) == nullptr) FAIL(OASIS_EINVAL, "%s is NULL", #ptr);     \
    } while (0)

// Common shape checks of every call.
int oasis::check_dims(const oasis_dims *d) {
    if (!d) FAIL(OASIS_EINVAL, "dims is NULL");
    if (d->B < 0) FAIL(OASIS_EINVAL, "B = %d < 0", d->B);
    if (d->H_q < 1 || d->H_kv < 1) FAIL(OASIS_EINVAL, "H_q = %d, H_kv = %d must be >= 1", d->H_q, d->H_kv);
    if (d->H_q % d->H_kv) FAIL(OASIS_EINVAL, "H_q = %d is not a multiple of H_kv = %d", d->H_q, d->H_kv);
    if (d->D != kD) FAIL(OASIS_EUNSUPPORTED, "D = %d (only %d is supported)", d->D, kD);
    if (d->bs != kBs) FAIL(OASIS_EUNSUPPORTED, "bs = %d (only %d is supported)", d->bs, kBs);
    if (d->H_q / d->H_kv > kMaxG)
        FAIL(OASIS_EUNSUPPORTED, "H_q / H_kv = %d (at most %d)", d->H_q / d->H_kv, kMaxG);
    if (d->NB_max < 1) FAIL(OASIS_EINVAL, "NB_max = %d < 1", d->NB_max);
    if (d->NB_max > kMaxNB) FAIL(OASIS_EUNSUPPORTED, "NB_max = %d (at most %d)", d->NB_max, kMaxNB);
    if ((int64_t)d->B * d->H_kv > (int64_t)INT32_MAX / 2) FAIL(OASIS_EUNSUPPORTED, "B * H_kv too large");
    return OASIS_OK;
}

extern "C" {

const char *oasis_version(void) { return "oasis 0.1.0 gfx950"; }

const char *oasis_last_error(void) { return g_error.c_str(); }

int oasis_host_alloc(size_t bytes, void **ptr) {
    clear_error();
    if (!ptr) FAIL(OASIS_EINVAL, "ptr is NULL");
    *ptr = nullptr;
    if (bytes == 0) FAIL(OASIS_EINVAL, "bytes = 0");
    OASIS_HIP(hipHostMalloc(ptr, bytes, hipHostMallocDefault));
    prefault_host(*ptr, bytes);
    return OASIS_OK;
}

int oasis_host_free(void *ptr) {
    clear_error();
    if (!ptr) return OASIS_OK;
    OASIS_HIP(hipHostFree(ptr));
    return OASIS_OK;
}

int32_t oasis_fetch_cap_blocks(double cap, int32_t K_b) {
    if (K_b < 1) return -1;
    if (!(cap > 0.0)) return 0;
    if (cap >= 1.0) return K_b;
    const double c = std::floor(cap * (double)K_b);
    return c < 1.0 ? 1 : (int32_t)c;
}

int oasis_build_summaries(const oasis_dims *dims, const uint16_t *kv, const int32_t *ctx_len,
                          uint16_t *kminmax, void *stream) {
    clear_error();
    int rc = check_dims(dims);
    if (rc) return rc;
    if (dims->B == 0) return OASIS_OK;
    NEED(kv);
    NEED(ctx_len);
    NEED(kminmax);
    const void *kv_dev = nullptr;
    if ((rc = device_view(kv, &kv_dev, "kv"))) return rc;
    OASIS_HIP(launch_build_summaries(*dims, static_cast<const uint16_t *>(kv_dev), ctx_len, kminmax,
                                     static_cast<hipStream_t>(stream)));
    return OASIS_OK;
}

int oasis_score_blocks(const oasis_dims *dims, const uint16_t *q_look, int32_t J,
                       const uint16_t *kminmax, const int32_t *ctx_len, float *scores, void *stream) {
    return score_blocks(dims, q_look, J, kminmax, ctx_len, scores, stream, nullptr);
}

int oasis_select_topk(const oasis_dims *dims, const float *scores, const int32_t *ctx_len, int32_t K_b,
                      int32_t *sel, int32_t *n_sel, void *stream) {
    return select_topk(dims, scores, ctx_len, K_b, sel, n_sel, stream, nullptr);
}

}  // extern "C"

namespace oasis {

int score_blocks(const oasis_dims *dims, const uint16_t *q_look, int32_t J, const uint16_t *kminmax,
                 const int32_t *ctx_len, float *scores, void *stream, hipEvent_t done) {
    clear_error();
    int rc = check_dims(dims);
    if (rc) return rc;
    if (J < 1) FAIL(OASIS_EINVAL, "J = %d < 1", J);
    if (J > 64) FAIL(OASIS_EUNSUPPORTED, "J = %d (at most 64)", J);
    if ((int64_t)dims->B * dims->H_kv * ((dims->NB_max + 63) / 64) > INT32_MAX)
        FAIL(OASIS_EUNSUPPORTED, "B * H_kv * ceil(NB_max / 64) exceeds 2^31 - 1");
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (dims->B == 0) {
        OASIS_HIP(record_done(done, s));
        return OASIS_OK;
    }
    NEED(q_look);
    NEED(kminmax);
    NEED(ctx_len);
    NEED(scores);
    OASIS_HIP(launch_score(*dims, q_look, J, kminmax, ctx_len, scores, s, done));
    return OASIS_OK;
}

int select_topk(const oasis_dims *dims, const float *scores, const int32_t *ctx_len, int32_t K_b, int32_t *sel,
                int32_t *n_sel, void *stream, hipEvent_t done) {
    clear_error();
    int rc = check_dims(dims);
    if (rc) return rc;
    if (K_b < 1) FAIL(OASIS_EINVAL, "K_b = %d < 1", K_b);
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (dims->B == 0) {
        OASIS_HIP(record_done(done, s));
        return OASIS_OK;
    }
    NEED(scores);
    NEED(ctx_len);
    NEED(sel);
    NEED(n_sel);
    OASIS_HIP(launch_topk(*dims, scores, ctx_len, K_b, sel, n_sel, s, done));
    return OASIS_OK;
}

}  // namespace oasis

extern "C" {

int oasis_append_kv(const oasis_dims *dims, const uint16_t *k_new, const uint16_t *v_new, int32_t *ctx_len,
                    uint16_t *kminmax, void *pool, uint16_t *ws_pool, const int32_t *slot_block, int32_t S,
                    void *stream) {
    clear_error();
    int rc = check_dims(dims);
    if (rc) return rc;
    if (ws_pool && (S < 1 || S > 2048))
        FAIL(S < 1 ? OASIS_EINVAL : OASIS_EUNSUPPORTED, "S = %d (1 .. 2048 with a working set)", S);
    if (dims->B == 0) return OASIS_OK;
    NEED(k_new);
    NEED(v_new);
    NEED(ctx_len);
    NEED(kminmax);
    NEED(pool);
    if (ws_pool) NEED(slot_block);
    const void *pool_dev = nullptr;
    if ((rc = device_view(pool, &pool_dev, "pool"))) return rc;
    OASIS_HIP(launch_append(*dims, k_new, v_new, ctx_len, kminmax, const_cast<void *>(pool_dev), ws_pool,
                            slot_block, ws_pool ? S : 0, static_cast<hipStream_t>(stream)));
    return OASIS_OK;
}

size_t oasis_block_mass_workspace_bytes(const oasis_dims *dims) {
    if (check_dims(dims) != OASIS_OK) return 0;
    return block_mass_ws_bytes(*dims);
}

int oasis_block_attention_mass(const oasis_dims *dims, const uint16_t *q, const uint16_t *kv_pool,
                               const int32_t *ctx_len, float sm_scale, float *mass, void *ws, size_t ws_bytes,
                               void *stream) {
    clear_error();
    int rc = check_dims(dims);
    if (rc) return rc;
    if (!std::isfinite(sm_scale)) FAIL(OASIS_EINVAL, "sm_scale is not finite");
    if (dims->B == 0) return OASIS_OK;
    NEED(q);
    NEED(kv_pool);
    NEED(ctx_len);
    NEED(mass);
    NEED(ws);
    const size_t need = block_mass_ws_bytes(*dims);
    if (ws_bytes < need) FAIL(OASIS_ENOSPACE, "block-mass workspace %zu bytes < %zu", ws_bytes, need);
    const void *kv_dev = nullptr;
    if ((rc = device_view(kv_pool, &kv_dev, "kv_pool"))) return rc;
    OASIS_HIP(launch_block_mass(*dims, q, kv_dev, ctx_len, sm_scale, mass, ws, static_cast<hipStream_t>(stream)));
    return OASIS_OK;
}

int oasis_topk_overlap(const oasis_dims *dims, const int32_t *sel_a, const int32_t *n_a, const int32_t *sel_b,
                       const int32_t *n_b, int32_t K, int32_t *overlap, void *stream) {
    clear_error();
    int rc = check_dims(dims);
    if (rc) return rc;
    if (K < 1) FAIL(OASIS_EINVAL, "K = %d < 1", K);
    if (dims->B == 0) return OASIS_OK;
    NEED(sel_a);
    NEED(n_a);
    NEED(sel_b);
    NEED(n_b);
    NEED(overlap);
    OASIS_HIP(launch_topk_overlap(dims->B * dims->H_kv, sel_a, n_a, sel_b, n_b, K, overlap,
                                  static_cast<hipStream_t>(stream)));
    return OASIS_OK;
}

size_t oasis_stage_plan_bytes(const oasis_dims *dims, int32_t C) {
    if (!dims || dims->B < 0 || dims->H_kv < 1) return 0;
    return sizeof(int32_t) * plan_ints(dims->B * dims->H_kv, C);
}

size_t oasis_stage_buffer_bytes(const oasis_dims *dims, int32_t n_blocks) {
    if (!dims || n_blocks < 0 || dims->bs < 1 || dims->D < 1) return 0;
    return (size_t)n_blocks * 2 * dims->bs * dims->D * sizeof(uint16_t);
}

// Arguments of the plan phase.
static int check_plan_args(const oasis_dims *dims, const oasis_stage_args *a) {
    int rc = check_dims(dims);
    if (rc) return rc;
    if (!a) FAIL(OASIS_EINVAL, "args is NULL");
    if (a->K_b < 1) FAIL(OASIS_EINVAL, "K_b = %d < 1", a->K_b);
    if (a->K_sel < 1) FAIL(OASIS_EINVAL, "K_sel = %d < 1", a->K_sel);
    if (a->C < 0 || a->C > a->K_b) FAIL(OASIS_EINVAL, "C = %d outside [0, K_b = %d]", a->C, a->K_b);
    if (a->S < a->K_b) FAIL(OASIS_EINVAL, "S = %d < K_b = %d", a->S, a->K_b);
    if (a->S > 2048 || a->K_sel > 1024)
        FAIL(OASIS_EUNSUPPORTED, "S = %d, K_sel = %d (at most 2048, 1024)", a->S, a->K_sel);
    if (a->step < 0) FAIL(OASIS_EINVAL, "step = %d < 0", a->step);
    if (dims->B == 0) return OASIS_OK;
    NEED(a->sel);
    NEED(a->n_sel);
    NEED(a->scores);
    NEED(a->slot_block);
    NEED(a->slot_stamp);
    NEED(a->ctx_len);
    NEED(a->tbl_slot);
    NEED(a->tbl_block);
    NEED(a->tbl_n);
    NEED(a->plan);
    const size_t need = oasis_stage_plan_bytes(dims, a->C);
    if (a->plan_bytes < need) FAIL(OASIS_ENOSPACE, "plan workspace %zu bytes < %zu", a->plan_bytes, need);
    return OASIS_OK;
}

// Arguments of the copy phase (host checks only).
static int check_copy_args(const oasis_dims *dims, const oasis_stage_args *a) {
    int rc = check_dims(dims);
    if (rc) return rc;
    if (!a) FAIL(OASIS_EINVAL, "args is NULL");
    if (a->C < 0 || a->C > 16384) FAIL(OASIS_EINVAL, "C = %d", a->C);
    if (a->S < 1 || a->S > 2048) FAIL(a->S < 1 ? OASIS_EINVAL : OASIS_EUNSUPPORTED, "S = %d", a->S);
    if (a->copy_mode != OASIS_COPY_KERNEL && a->copy_mode != OASIS_COPY_DMA)
        FAIL(OASIS_EINVAL, "copy_mode = %d", a->copy_mode);
    if (dims->B == 0) return OASIS_OK;
    NEED(a->plan);
    NEED(a->host_pool);
    NEED(a->ws_pool);
    const size_t need = oasis_stage_plan_bytes(dims, a->C);
    if (a->plan_bytes < need) FAIL(OASIS_ENOSPACE, "plan workspace %zu bytes < %zu", a->plan_bytes, need);
    if (a->copy_mode == OASIS_COPY_DMA) {
        NEED(a->host_plan);
        NEED(a->stage_host);
        NEED(a->stage_dev);
        if (a->host_plan_bytes < need)
            FAIL(OASIS_ENOSPACE, "host plan %zu bytes < %zu", a->host_plan_bytes, need);
        if (a->C > 0 && (a->stage_host_bytes < kBlockBytes || a->stage_dev_bytes < kBlockBytes))
            FAIL(OASIS_ENOSPACE, "staging buffers (%zu, %zu bytes) hold no block", a->stage_host_bytes,
                 a->stage_dev_bytes);
        if (a->host_threads < 0 || a->host_threads > 256)
            FAIL(OASIS_EINVAL, "host_threads = %d outside [0, 256]", a->host_threads);
    }
    return OASIS_OK;
}

// `plan_event` is bound to the prefix kernel that ends the plan.
static int stage_plan_phase(const oasis_dims *dims, const oasis_stage_args *a) {
    hipStream_t s = static_cast<hipStream_t>(a->stream);
    OASIS_HIP(launch_stage_plan(*dims, *a, s));
    OASIS_HIP(launch_stage_prefix(*dims, *a, s, static_cast<hipEvent_t>(a->plan_event)));
    return OASIS_OK;
}

// Pointer checks of the copy phase that need the runtime: the pool must be
// device memory or pinned host memory with a device mapping (pageable host
// memory is refused), the DMA engine's host buffers pinned.  Done before
// anything is enqueued.
static int resolve_copy_args(const oasis_stage_args *a, const void **pool_dev) {
    int rc;
    if ((rc = device_view(a->host_pool, pool_dev, "host_pool"))) return rc;
    if (a->copy_mode == OASIS_COPY_DMA) {
        for (const void *hb : {a->host_plan, a->stage_host}) {
            hipPointerAttribute_t at;
            if (hipPointerGetAttributes(&at, hb) != hipSuccess || at.type != hipMemoryTypeHost) {
                (void)hipGetLastError();
                FAIL(OASIS_EINVAL, "%s is not pinned host memory", hb == a->host_plan ? "host_plan" : "stage_host");
            }
        }
    }
    return OASIS_OK;
}

static int stage_copy_phase(const oasis_dims *dims, const oasis_stage_args *a, const void *pool_dev) {
    int rc;
    hipStream_t s = static_cast<hipStream_t>(a->stream);
    hipStream_t cs = a->copy_stream ? static_cast<hipStream_t>(a->copy_stream) : s;
    // the plan this copy uses: `plan_event` if given, else everything on `stream` so far
    // (a gather on that same stream follows it in stream order)
    const bool in_order = cs == s && a->copy_mode == OASIS_COPY_KERNEL;
    hipEvent_t plan_ready = static_cast<hipEvent_t>(a->plan_event);
    if (!plan_ready && !in_order) {
        if ((rc = ring_event(&plan_ready))) return rc;
        OASIS_HIP(hipEventRecord(plan_ready, s));
    }
    hipEvent_t done = static_cast<hipEvent_t>(a->done_event);
    if (a->copy_mode == OASIS_COPY_KERNEL) {
        if (!in_order) OASIS_HIP(stream_wait(cs, plan_ready));
        if (a->wait_event) OASIS_HIP(stream_wait(cs, static_cast<hipEvent_t>(a->wait_event)));
        OASIS_HIP(launch_stage_gather(*dims, *a, pool_dev, cs, done));
    } else {
        if ((rc = stage_dma(*dims, *a, plan_ready, cs))) return rc;
        if (done) OASIS_HIP(hipEventRecord(done, cs));
    }
    return OASIS_OK;
}

int oasis_stage_plan(const oasis_dims *dims, const oasis_stage_args *a) {
    clear_error();
    int rc = check_plan_args(dims, a);
    if (rc) return rc;
    if (dims->B == 0) {
        OASIS_HIP(record_done(static_cast<hipEvent_t>(a->plan_event), static_cast<hipStream_t>(a->stream)));
        return OASIS_OK;
    }
    return stage_plan_phase(dims, a);
}

int oasis_stage_copy(const oasis_dims *dims, const oasis_stage_args *a) {
    clear_error();
    int rc = check_copy_args(dims, a);
    if (rc || dims->B == 0) return rc;
    const void *pool_dev = nullptr;
    if ((rc = resolve_copy_args(a, &pool_dev))) return rc;
    return stage_copy_phase(dims, a, pool_dev);
}

// Reads the step totals at the end of a plan (the stream's work is done).
static int read_plan_totals(const oasis_dims *dims, int C, const int32_t *plan, hipStream_t s,
                            oasis_stage_stats *out) {
    int32_t tail[kPlanTail] = {0, 0, 0, 0};
    const size_t off = (size_t)dims->B * dims->H_kv * plan_row(C);
    OASIS_HIP(hipMemcpyAsync(tail, plan + off, sizeof(tail), hipMemcpyDeviceToHost, s));
    OASIS_HIP(hipStreamSynchronize(s));
    out->admits = tail[0];
    out->evictions = tail[1];
    out->deferred = tail[2];
    out->capped_pairs = tail[3];
    out->bytes = (int64_t)tail[0] * 2 * dims->bs * dims->D * (int64_t)sizeof(uint16_t);
    return OASIS_OK;
}

int oasis_stage_read_stats(const oasis_dims *dims, int32_t C, const int32_t *plan, oasis_stage_stats *stats,
                           void *stream) {
    clear_error();
    int rc = check_dims(dims);
    if (rc) return rc;
    if (C < 0) FAIL(OASIS_EINVAL, "C = %d < 0", C);
    NEED(stats);
    *stats = oasis_stage_stats{0, 0, 0, 0, 0};
    if (dims->B == 0) return OASIS_OK;
    NEED(plan);
    return read_plan_totals(dims, C, plan, static_cast<hipStream_t>(stream), stats);
}

int oasis_stage_blocks(const oasis_dims *dims, const oasis_stage_args *a, oasis_stage_stats *stats) {
    clear_error();
    int rc = check_plan_args(dims, a);
    if (rc) return rc;
    if ((rc = check_copy_args(dims, a))) return rc;
    if (stats) *stats = oasis_stage_stats{0, 0, 0, 0, 0};
    if (dims->B == 0) return OASIS_OK;
    const void *pool_dev = nullptr;
    if ((rc = resolve_copy_args(a, &pool_dev))) return rc;  // before the plan changes any state
    if ((rc = stage_plan_phase(dims, a))) return rc;
    if ((rc = stage_copy_phase(dims, a, pool_dev))) return rc;
    if (stats) return read_plan_totals(dims, a->C, a->plan, static_cast<hipStream_t>(a->stream), stats);
    return OASIS_OK;
}

size_t oasis_attn_workspace_bytes(const oasis_dims *dims, int32_t T, int32_t n_split) {
    if (check_dims(dims) != OASIS_OK || T < 0 || n_split < 0) return 0;
    return attn_ws_bytes(*dims, 1, T, n_split);
}

size_t oasis_lookahead_attn_workspace_bytes(const oasis_dims *dims, int32_t n_q, int32_t T, int32_t n_split) {
    if (check_dims(dims) != OASIS_OK || n_q < 1 || T < 0 || n_split < 0) return 0;
    return attn_ws_bytes(*dims, n_q, T, n_split);
}

int32_t oasis_attn_num_splits(const oasis_dims *dims, int32_t T, int32_t n_split) {
    if (check_dims(dims) != OASIS_OK || T < 0 || n_split < 0) return -1;
    return attn_splits(*dims, 1, T, n_split);
}

int oasis_attn_launch_shape(const oasis_dims *dims, int32_t n_q, int32_t T, int32_t n_split, int32_t *splits,
                            int32_t *waves) {
    clear_error();
    int rc = check_dims(dims);
    if (rc) return rc;
    NEED(splits);
    NEED(waves);
    if (n_q < 1) FAIL(OASIS_EINVAL, "n_q = %d < 1", n_q);
    if ((int64_t)n_q * (dims->H_q / dims->H_kv) > kMaxG)
        FAIL(OASIS_EUNSUPPORTED, "n_q * H_q / H_kv = %lld (at most %d)",
             (long long)n_q * (dims->H_q / dims->H_kv), kMaxG);
    if (T < 0) FAIL(OASIS_EINVAL, "T = %d < 0", T);
    if (n_split < 0 || n_split > 64) FAIL(OASIS_EINVAL, "n_split = %d outside [0, 64]", n_split);
    *splits = attn_splits(*dims, n_q, T, n_split);
    *waves = attn_waves(*dims, n_q, T, *splits);
    return OASIS_OK;
}

int oasis_lookahead_attn(const oasis_dims *dims, int32_t n_q, const uint16_t *q, const uint16_t *kv_pool,
                         int32_t P, const int32_t *tbl_slot, const int32_t *tbl_block, const int32_t *tbl_n,
                         int32_t T, const int32_t *ctx_len, float sm_scale, uint16_t *out, float *lse, void *ws,
                         size_t ws_bytes, int32_t n_split, void *stream) {
    return lookahead_attn(dims, n_q, q, kv_pool, P, tbl_slot, tbl_block, tbl_n, T, ctx_len, sm_scale, out, lse, ws,
                          ws_bytes, n_split, stream, nullptr);
}

}  // extern "C"

int oasis::lookahead_attn(const oasis_dims *dims, int32_t n_q, const uint16_t *q, const uint16_t *kv_pool, int32_t P,
                          const int32_t *tbl_slot, const int32_t *tbl_block, const int32_t *tbl_n, int32_t T,
                          const int32_t *ctx_len, float sm_scale, uint16_t *out, float *lse, void *ws,
                          size_t ws_bytes, int32_t n_split, void *stream, hipEvent_t done) {
    clear_error();
    int rc = check_dims(dims);
    if (rc) return rc;
    if (n_q < 1) FAIL(OASIS_EINVAL, "n_q = %d < 1", n_q);
    if ((int64_t)n_q * (dims->H_q / dims->H_kv) > kMaxG)
        FAIL(OASIS_EUNSUPPORTED, "n_q * H_q / H_kv = %lld (at most %d)",
             (long long)n_q * (dims->H_q / dims->H_kv), kMaxG);
    if (P < 1) FAIL(OASIS_EINVAL, "P = %d < 1", P);
    if (T < 0) FAIL(OASIS_EINVAL, "T = %d < 0", T);
    if (n_split < 0 || n_split > 64) FAIL(OASIS_EINVAL, "n_split = %d outside [0, 64]", n_split);
    if (!std::isfinite(sm_scale)) FAIL(OASIS_EINVAL, "sm_scale is not finite");
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (dims->B == 0) {
        OASIS_HIP(record_done(done, s));
        return OASIS_OK;
    }
    NEED(q);
    NEED(kv_pool);
    NEED(tbl_n);
    NEED(ctx_len);
    NEED(out);
    if (T > 0) {
        NEED(tbl_slot);
        NEED(tbl_block);
    }
    const int splits = attn_splits(*dims, n_q, T, n_split);
    const size_t need = attn_ws_bytes(*dims, n_q, T, n_split);
    if (need > 0) {
        NEED(ws);
        if (ws_bytes < need) FAIL(OASIS_ENOSPACE, "attention workspace %zu bytes < %zu", ws_bytes, need);
    }
    OASIS_HIP(launch_attn(*dims, n_q, q, kv_pool, P, tbl_slot, tbl_block, tbl_n, T, ctx_len, sm_scale, out, lse,
                          static_cast<float *>(ws), splits, s, done));
    return OASIS_OK;
}

extern "C" {

size_t oasis_sparse_decode_attn_static_bytes(void) { return attn_static_scratch_bytes(); }

int oasis_sparse_decode_attn_static(const oasis_dims *dims, const uint16_t *q, const uint16_t *kv_pool, int32_t P,
                                    const int32_t *tbl_slot, const int32_t *tbl_block, const int32_t *tbl_n,
                                    int32_t T, const int32_t *ctx_len, float sm_scale, uint16_t *out, float *lse,
                                    int32_t n_split, void *stream) {
    clear_error();
    int rc = check_dims(dims);
    if (rc) return rc;
    if (P < 1) FAIL(OASIS_EINVAL, "P = %d < 1", P);
    if (T < 0) FAIL(OASIS_EINVAL, "T = %d < 0", T);
    if (n_split < 0 || n_split > 64) FAIL(OASIS_EINVAL, "n_split = %d outside [0, 64]", n_split);
    if (!std::isfinite(sm_scale)) FAIL(OASIS_EINVAL, "sm_scale is not finite");
    if (dims->B == 0) return OASIS_OK;
    NEED(q);
    NEED(kv_pool);
    NEED(tbl_n);
    NEED(ctx_len);
    NEED(out);
    if (T > 0) {
        NEED(tbl_slot);
        NEED(tbl_block);
    }
    const int splits = attn_splits(*dims, 1, T, n_split);
    const size_t need = attn_ws_bytes(*dims, 1, T, n_split);
    const size_t have = attn_static_scratch_bytes();
    if (need > have)
        FAIL(OASIS_ENOSPACE,
             "split-K partials need %zu bytes, more than the %zu bytes of fixed scratch (B * H_q * splits * "
             "(D + 2) * 4); use oasis_sparse_decode_attn with a workspace, or fewer splits",
             need, have);
    void *ws = nullptr;
    if (need > 0) OASIS_HIP(attn_static_scratch(&ws));
    OASIS_HIP(launch_attn(*dims, 1, q, kv_pool, P, tbl_slot, tbl_block, tbl_n, T, ctx_len, sm_scale, out, lse,
                          static_cast<float *>(ws), splits, static_cast<hipStream_t>(stream)));
    return OASIS_OK;
}

int oasis_sparse_decode_attn(const oasis_dims *dims, const uint16_t *q, const uint16_t *kv_pool, int32_t P,
                             const int32_t *tbl_slot, const int32_t *tbl_block, const int32_t *tbl_n, int32_t T,
                             const int32_t *ctx_len, float sm_scale, uint16_t *out, float *lse, void *ws,
                             size_t ws_bytes, int32_t n_split, void *stream) {
    return oasis_lookahead_attn(dims, 1, q, kv_pool, P, tbl_slot, tbl_block, tbl_n, T, ctx_len, sm_scale, out, lse,
                                ws, ws_bytes, n_split, stream);
}

}  // extern "C"
