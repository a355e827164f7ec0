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

// Per-thread, per-device event that orders the copy stream after the plan.
thread_local std::vector<hipEvent_t> t_plan_event;
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

static int plan_event(hipEvent_t *ev) {
    int dev = 0;
    OASIS_HIP(hipGetDevice(&dev));
    if ((int)t_plan_event.size() <= dev) t_plan_event.resize(dev + 1, nullptr);
    if (!t_plan_event[dev]) OASIS_HIP(hipEventCreateWithFlags(&t_plan_event[dev], hipEventDisableTiming));
    *ev = t_plan_event[dev];
    return OASIS_OK;
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

// Common shape checks.  needs_nb: the call indexes [0, NB_max) arrays.
static int check_dims(const oasis_dims *d) {
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
    clear_error();
    int rc = check_dims(dims);
    if (rc) return rc;
    if (J < 1) FAIL(OASIS_EINVAL, "J = %d < 1", J);
    if (J > 64) FAIL(OASIS_EUNSUPPORTED, "J = %d (at most 64)", J);
    if (dims->B == 0) return OASIS_OK;
    NEED(q_look);
    NEED(kminmax);
    NEED(ctx_len);
    NEED(scores);
    OASIS_HIP(launch_score(*dims, q_look, J, kminmax, ctx_len, scores, static_cast<hipStream_t>(stream)));
    return OASIS_OK;
}

int oasis_select_topk(const oasis_dims *dims, const float *scores, const int32_t *ctx_len, int32_t K_b,
                      int32_t *sel, int32_t *n_sel, void *stream) {
    clear_error();
    int rc = check_dims(dims);
    if (rc) return rc;
    if (K_b < 1) FAIL(OASIS_EINVAL, "K_b = %d < 1", K_b);
    if (dims->B == 0) return OASIS_OK;
    NEED(scores);
    NEED(ctx_len);
    NEED(sel);
    NEED(n_sel);
    OASIS_HIP(launch_topk(*dims, scores, ctx_len, K_b, sel, n_sel, static_cast<hipStream_t>(stream)));
    return OASIS_OK;
}

size_t oasis_stage_plan_bytes(const oasis_dims *dims, int32_t C) {
    if (!dims || dims->B < 0 || dims->H_kv < 1) return 0;
    return sizeof(int32_t) * (size_t)dims->B * dims->H_kv * plan_row(C);
}

size_t oasis_stage_host_plan_bytes(const oasis_dims *dims, int32_t C) { return oasis_stage_plan_bytes(dims, C); }

int oasis_stage_blocks(const oasis_dims *dims, const oasis_stage_args *a) {
    clear_error();
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
    if (a->copy_mode != OASIS_COPY_KERNEL && a->copy_mode != OASIS_COPY_DMA)
        FAIL(OASIS_EINVAL, "copy_mode = %d", a->copy_mode);
    if (dims->B == 0) return OASIS_OK;
    NEED(a->sel);
    NEED(a->n_sel);
    NEED(a->scores);
    NEED(a->slot_block);
    NEED(a->slot_stamp);
    NEED(a->ctx_len);
    NEED(a->host_pool);
    NEED(a->ws_pool);
    NEED(a->tbl_slot);
    NEED(a->tbl_block);
    NEED(a->tbl_n);
    NEED(a->plan);
    const size_t need = oasis_stage_plan_bytes(dims, a->C);
    if (a->plan_bytes < need) FAIL(OASIS_ENOSPACE, "plan workspace %zu bytes < %zu", a->plan_bytes, need);
    if (a->copy_mode == OASIS_COPY_DMA) {
        NEED(a->host_plan);
        if (a->host_plan_bytes < need)
            FAIL(OASIS_ENOSPACE, "host plan %zu bytes < %zu", a->host_plan_bytes, need);
    }
    const void *pool_dev = nullptr;
    if ((rc = device_view(a->host_pool, &pool_dev, "host_pool"))) return rc;
    if (a->copy_mode == OASIS_COPY_DMA) {
        hipPointerAttribute_t at;
        if (hipPointerGetAttributes(&at, a->host_plan) != hipSuccess || at.type != hipMemoryTypeHost) {
            (void)hipGetLastError();
            FAIL(OASIS_EINVAL, "host_plan is not pinned host memory");
        }
    }

    hipStream_t s = static_cast<hipStream_t>(a->stream);
    hipStream_t cs = a->copy_stream ? static_cast<hipStream_t>(a->copy_stream) : s;
    OASIS_HIP(launch_stage_plan(*dims, *a, s));

    if (a->copy_mode == OASIS_COPY_KERNEL) {
        if (cs != s) {
            hipEvent_t ev;
            if ((rc = plan_event(&ev))) return rc;
            OASIS_HIP(hipEventRecord(ev, s));
            OASIS_HIP(hipStreamWaitEvent(cs, ev, 0));
        }
        if (a->wait_event) OASIS_HIP(hipStreamWaitEvent(cs, static_cast<hipEvent_t>(a->wait_event), 0));
        OASIS_HIP(launch_stage_gather(*dims, *a, pool_dev, cs));
    } else {
        OASIS_HIP(hipMemcpyAsync(a->host_plan, a->plan, need, hipMemcpyDeviceToHost, s));
        OASIS_HIP(hipStreamSynchronize(s));
        if (a->wait_event) OASIS_HIP(hipStreamWaitEvent(cs, static_cast<hipEvent_t>(a->wait_event), 0));
        const int row = plan_row(a->C);
        const int32_t *hp = static_cast<const int32_t *>(a->host_plan);
        const char *src0 = static_cast<const char *>(a->host_pool);
        char *dst0 = static_cast<char *>(a->ws_pool);
        const int pairs = dims->B * dims->H_kv;
        for (int rh = 0; rh < pairs; rh++) {
            const int32_t *p = hp + (size_t)rh * row;
            const int n = p[0] < a->C ? p[0] : a->C;
            int i = 0;
            while (i < n) {
                const int slot = p[2 + 2 * i], blk = p[3 + 2 * i];
                if (slot < 0 || slot >= a->S || blk < 0 || blk >= dims->NB_max) { i++; continue; }
                int run = 1;  // merge admits that are adjacent in both pool and working set
                while (i + run < n && p[2 + 2 * (i + run)] == slot + run && p[3 + 2 * (i + run)] == blk + run &&
                       slot + run < a->S && blk + run < dims->NB_max)
                    run++;
                const char *src = src0 + ((size_t)rh * dims->NB_max + blk) * kBlockBytes;
                char *dst = dst0 + ((size_t)rh * a->S + slot) * kBlockBytes;
                OASIS_HIP(hipMemcpyAsync(dst, src, run * kBlockBytes, hipMemcpyHostToDevice, cs));
                i += run;
            }
        }
    }
    if (a->done_event) OASIS_HIP(hipEventRecord(static_cast<hipEvent_t>(a->done_event), cs));
    return OASIS_OK;
}

size_t oasis_attn_workspace_bytes(const oasis_dims *dims, int32_t T, int32_t n_split) {
    if (check_dims(dims) != OASIS_OK || T < 0 || n_split < 0) return 0;
    return attn_ws_bytes(*dims, T, n_split);
}

int32_t oasis_attn_num_splits(const oasis_dims *dims, int32_t T, int32_t n_split) {
    if (check_dims(dims) != OASIS_OK || T < 0 || n_split < 0) return -1;
    return attn_splits(*dims, T, n_split);
}

int oasis_sparse_decode_attn(const oasis_dims *dims, const uint16_t *q, const uint16_t *kv_pool, int32_t P,
                             const int32_t *tbl_slot, const int32_t *tbl_block, const int32_t *tbl_n, int32_t T,
                             const int32_t *ctx_len, float sm_scale, uint16_t *out, float *lse, void *ws,
                             size_t ws_bytes, int32_t n_split, void *stream) {
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
    const int splits = attn_splits(*dims, T, n_split);
    const size_t need = attn_ws_bytes(*dims, T, n_split);
    if (need > 0) {
        NEED(ws);
        if (ws_bytes < need) FAIL(OASIS_ENOSPACE, "attention workspace %zu bytes < %zu", ws_bytes, need);
    }
    OASIS_HIP(launch_attn(*dims, q, kv_pool, P, tbl_slot, tbl_block, tbl_n, T, ctx_len, sm_scale, out, lse,
                          static_cast<float *>(ws), splits, static_cast<hipStream_t>(stream)));
    return OASIS_OK;
}

}  // extern "C"
