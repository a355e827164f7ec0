// Host half of the DMA copy engine of oasis_stage_blocks.
//
// OasisKV (arXiv 2608.08097), paperlayer summary, section 4: the admitted
// blocks move from host memory into HBM in the background, overlapped with
// the current step; only the next step's attention waits for them.
//
// The admitted blocks of one step are scattered over the pinned pool (one
// 8 KiB block per (request, KV head, admit)).  One hipMemcpyAsync per block
// costs microseconds of runtime work each, thousands of times per step, so
// instead a pool of worker threads packs them into a pinned staging buffer in
// plan order, a single hipMemcpyAsync moves the packed buffer over PCIe on the
// DMA engines, and a scatter kernel places the blocks into their slots.  The
// DMA engines do not use the compute units or their memory path, so the
// HBM-bound kernels of the same step keep their bandwidth.
#include "oasis_internal.h"
#include "worker_pool.h"

#include <atomic>
#include <cstring>
#include <thread>
#include <vector>

namespace oasis {

namespace {

// ------------------------------------------------------------ worker pool

WorkerPool &workers() {
    static WorkerPool w;
    return w;
}

// One 8 KiB block with streaming (non-temporal) stores: the staging buffer
// is only read by the copy engine, so its lines need not be read into the
// CPU caches first nor kept there.
typedef long long v2i64 __attribute__((vector_size(16)));
void copy_block_nt(char *dst, const char *src) {
    const v2i64 *s = reinterpret_cast<const v2i64 *>(src);
    v2i64 *d = reinterpret_cast<v2i64 *>(dst);
    for (size_t i = 0; i < kBlockBytes / sizeof(v2i64); i += 4) {
        const v2i64 a = s[i], b = s[i + 1], c = s[i + 2], e = s[i + 3];
        __builtin_nontemporal_store(a, d + i);
        __builtin_nontemporal_store(b, d + i + 1);
        __builtin_nontemporal_store(c, d + i + 2);
        __builtin_nontemporal_store(e, d + i + 3);
    }
}

// ------------------------------------------------------------ events

constexpr int kRing = 16;
struct EventRing {
    hipEvent_t ev[kRing] = {};
    int next = 0;
};
thread_local std::vector<EventRing> t_ring;

// Last copy out of each recently used host staging buffer (per thread, each
// entry with an event of its own), so that repacking a buffer waits for the
// copy that still reads it.
struct StageUse {
    const void *buf = nullptr;
    int device = -1;
    hipEvent_t done = nullptr;
    bool pending = false;
};
// enough entries for every staging buffer a thread cycles through (a layer
// pipeline uses two per layer), so that an entry is rarely evicted, which
// waits for its copy
constexpr int kStageUses = 128;
thread_local StageUse t_stage_use[kStageUses];
thread_local int t_stage_next = 0;

int wait_stage_free(const void *buf, int dev) {
    for (auto &u : t_stage_use)
        if (u.pending && u.buf == buf && u.device == dev) {
            OASIS_HIP(hipEventSynchronize(u.done));
            u.pending = false;
        }
    return OASIS_OK;
}

int note_stage_use(const void *buf, int dev, hipStream_t cs) {
    StageUse *slot = nullptr;
    for (auto &u : t_stage_use)
        if (u.buf == buf && u.device == dev) slot = &u;
    if (!slot) {
        slot = &t_stage_use[t_stage_next];
        t_stage_next = (t_stage_next + 1) % kStageUses;
        if (slot->pending) OASIS_HIP(hipEventSynchronize(slot->done));  // evicted entry: settle it
        if (slot->done && slot->device != dev) {
            OASIS_HIP(hipEventDestroy(slot->done));
            slot->done = nullptr;
        }
        slot->buf = buf;
        slot->device = dev;
    }
    if (!slot->done) OASIS_HIP(hipEventCreateWithFlags(&slot->done, hipEventDisableTiming));
    OASIS_HIP(hipEventRecord(slot->done, cs));
    slot->pending = true;
    return OASIS_OK;
}

}  // namespace

void prefault_host(void *p, size_t bytes) {
    constexpr size_t kPage = 4096;
    constexpr size_t kChunk = (size_t)64 << 20;
    char *base = static_cast<char *>(p);
    const size_t chunks = (bytes + kChunk - 1) / kChunk;
    const int threads = (int)std::max(1u, std::min(16u, std::thread::hardware_concurrency()));
    workers().run(threads, (int)chunks, [&](int c) {
        const size_t lo = (size_t)c * kChunk, hi = std::min(bytes, lo + kChunk);
        for (size_t off = lo; off < hi; off += kPage) base[off] = 0;
    });
}

// Per-thread, per-device non-blocking stream for plan read-backs.
thread_local std::vector<hipStream_t> t_readback;

int readback_stream(hipStream_t *out) {
    int dev = 0;
    OASIS_HIP(hipGetDevice(&dev));
    if ((int)t_readback.size() <= dev) t_readback.resize(dev + 1, nullptr);
    if (!t_readback[dev]) OASIS_HIP(hipStreamCreateWithFlags(&t_readback[dev], hipStreamNonBlocking));
    *out = t_readback[dev];
    return OASIS_OK;
}

// A ring, so that an event is not re-recorded while a wait on its previous
// record may still be pending (the ring is much longer than the number of
// events one call keeps alive).
int ring_event(hipEvent_t *ev) {
    int dev = 0;
    OASIS_HIP(hipGetDevice(&dev));
    if ((int)t_ring.size() <= dev) t_ring.resize(dev + 1);
    EventRing &ring = t_ring[dev];
    hipEvent_t &e = ring.ev[ring.next];
    ring.next = (ring.next + 1) % kRing;
    if (!e) OASIS_HIP(hipEventCreateWithFlags(&e, hipEventDisableTiming));
    *ev = e;
    return OASIS_OK;
}

hipError_t stream_wait(hipStream_t s, hipEvent_t e) {
    const hipError_t q = hipEventQuery(e);
    if (q == hipSuccess) return hipSuccess;
    if (q != hipErrorNotReady) return q;
    return hipStreamWaitEvent(s, e, 0);
}

hipError_t record_done(hipEvent_t done, hipStream_t s) { return done ? hipEventRecord(done, s) : hipSuccess; }

int stage_dma(const oasis_dims &d, const oasis_stage_args &a, hipEvent_t plan_ready, hipStream_t cs) {
    const int pairs = d.B * d.H_kv;
    const int row = plan_row(a.C);
    const size_t plan_bytes = plan_ints(pairs, a.C) * sizeof(int32_t);
    int rc;

    // 1. plan to the host, on a stream of its own: the copy stream may still
    //    be busy with an earlier step's copy, the plan's stream with later work
    hipStream_t rb;
    if ((rc = readback_stream(&rb))) return rc;
    hipEvent_t read_done;
    if ((rc = ring_event(&read_done))) return rc;
    OASIS_HIP(hipStreamWaitEvent(rb, plan_ready, 0));
    OASIS_HIP(hipMemcpyAsync(a.host_plan, a.plan, plan_bytes, hipMemcpyDeviceToHost, rb));
    OASIS_HIP(hipEventRecord(read_done, rb));
    OASIS_HIP(hipEventSynchronize(read_done));
    // the copies below are ordered after the plan through the host wait above
    const int32_t *hp = static_cast<const int32_t *>(a.host_plan);
    const int total = hp[(size_t)pairs * row];
    if (total <= 0) return OASIS_OK;

    const int cap_h = (int)std::min<size_t>(a.stage_host_bytes / kBlockBytes, (size_t)INT32_MAX);
    const int cap_d = (int)std::min<size_t>(a.stage_dev_bytes / kBlockBytes, (size_t)INT32_MAX);
    const int cap = std::min(cap_h, cap_d);
    if (cap < 1) {
        set_error("staging buffers hold no block");
        return OASIS_ENOSPACE;
    }
    const char *pool = static_cast<const char *>(a.host_pool);
    char *stage = static_cast<char *>(a.stage_host);
    const int threads = a.host_threads > 0 ? a.host_threads : 8;
    const int C = a.C;

    int dev = 0;
    OASIS_HIP(hipGetDevice(&dev));
    if ((rc = wait_stage_free(a.stage_host, dev))) return rc;
    bool waited = false;
    hipEvent_t round_done = nullptr;
    for (int lo = 0; lo < total; lo += cap) {
        const int hi = std::min(total, lo + cap);
        if (round_done) OASIS_HIP(hipEventSynchronize(round_done));  // the staging buffer is free again
        // 2. pack positions [lo, hi): one work item per group of (r, h)
        const int per_item = 8;
        workers().run(threads, (pairs + per_item - 1) / per_item, [&](int item) {
            for (int rh = item * per_item; rh < std::min(pairs, (item + 1) * per_item); rh++) {
                const int32_t *p = hp + (size_t)rh * row;
                const int n = std::min<int>(p[0], C);
                const int pos = p[2];
                for (int i = 0; i < n; i++) {
                    const int k = pos + i;
                    if (k < lo || k >= hi) continue;
                    const int blk = p[kPlanHead + 2 * i + 1];
                    if (blk < 0 || blk >= d.NB_max) continue;
                    copy_block_nt(stage + (size_t)(k - lo) * kBlockBytes,
                                  pool + ((size_t)rh * d.NB_max + blk) * kBlockBytes);
                }
            }
            // the streaming stores must be visible before the copy engine reads them
            std::atomic_thread_fence(std::memory_order_seq_cst);
        });
        // 3. one copy over PCIe, then the device scatter into the slots
        OASIS_HIP(hipMemcpyAsync(a.stage_dev, a.stage_host, (size_t)(hi - lo) * kBlockBytes,
                                 hipMemcpyHostToDevice, cs));
        if (!waited && a.wait_event) {
            // only the scatter touches working-set slots
            OASIS_HIP(stream_wait(cs, static_cast<hipEvent_t>(a.wait_event)));
            waited = true;
        }
        OASIS_HIP(launch_stage_scatter(d, a, lo, hi, cs));
        if ((rc = ring_event(&round_done))) return rc;
        OASIS_HIP(hipEventRecord(round_done, cs));
    }
    return note_stage_use(a.stage_host, dev, cs);
}

}  // namespace oasis
