// Native scheduler of the per-layer decode chain (oasis_pipeline_*).
//
// OasisKV (arXiv 2608.08097), paperlayer summary, section 4.  Scoring, top-K,
// the staging plan and the block copies of a layer are kept off the attention
// stream, on streams of their own, so that the work of several layers and
// steps overlaps; an attention launch waits only on the copies into its own
// layer's working set.  One call here enqueues one layer-step of that
// schedule through the library's own entry points, so a decode step costs a
// few microseconds of host time per layer instead of a round of interpreter
// calls per launch.  The dependency rules are stated in include/oasis.h.
#include "copy_queue.h"
#include "oasis_internal.h"

#include <algorithm>
#include <chrono>
#include <cstdio>
#include <mutex>
#include <string>
#include <vector>

namespace oasis {
namespace {

enum EvKind { kEvAttn = 0, kEvSel, kEvPlan, kEvStage, kEvKinds };
// Events of (kind, layer, step) are reused every kRing steps.  An event of
// step t is waited on by work issued no later than step t + 2 (and, with the
// DMA worker, before the caller moves on to step t + 2), so a ring of four
// never re-records an event that a wait still has to be issued for.
constexpr int kRing = 4;

// Rates that decide whether a staged step is bound by the link or by HBM:
// the pinned host -> device copy rate and the streaming HBM read rate
// measured on MI355X (PCIe Gen5 x16; HBM3E).
constexpr double kLinkBytesPerS = 57e9;
constexpr double kHbmBytesPerS = 6e12;
constexpr double kSummaryBytes = 2 * kD * 2;  // one block's min and max key, bf16
constexpr int kTimedKinds = 4;

struct Job {
    int layer = 0, step = 0;
    oasis_stage_args args{};
};

// The background half of one layer-step: scores, top-K and staging plan
// from the lookahead queries (and the copies that follow).  attn_prev
// completes with the attention of step - 1.
struct ChainJob {
    int layer = 0, step = 0;
    const uint16_t *q_look = nullptr;
    hipEvent_t attn_prev = nullptr;
};

}  // namespace
}  // namespace oasis

using namespace oasis;

struct oasis_pipeline {
    oasis_dims d{};
    oasis_pipeline_desc desc{};
    std::vector<oasis_layer_buffers> layers;
    std::vector<int> next_step;  // per layer: the step the next call must issue
    int device = 0;
    int S = 0;
    hipStream_t main = nullptr, comp[2] = {nullptr, nullptr}, copy[2] = {nullptr, nullptr};
    bool comp_on_main = false;  // compute_streams = -1: the chain runs on the main stream
    std::vector<hipEvent_t> ev;  // [kind][layer][kRing]
    // per layer: the event that completes with the layer's latest attention
    // (written by the calling thread), and without staging with its latest
    // top-K (written by whichever thread issues the chain, read by the calling
    // thread once that chain job has run); the ring's event, or the timing
    // event bound to the same kernel; nullptr after timing is re-armed
    std::vector<hipEvent_t> attn_last, sel_last;

    // timing
    int t_cap = 0;
    int t_every = 1;       // one launch in every t_every of a kind is timed
    int t_seen[kTimedKinds] = {0, 0, 0, 0};  // launches of each kind since arming
    uint32_t t_kinds = 0;  // bit k: kind k is timed
    std::vector<hipEvent_t> t_ev[kTimedKinds];  // 2 * t_cap each
    int t_n[kTimedKinds] = {0, 0, 0, 0};
    double copy_host_s = 0.0;
    int copy_calls = 0;
    std::mutex t_mu;  // copy-host totals (written by the worker)

    // worker threads, each in submission order: the copy halves (DMA engine,
    // or any engine when `threaded`), and with `threaded` the chain halves
    bool threaded = false;
    CopyQueue<Job> copies;
    CopyQueue<ChainJob> chain;

    hipEvent_t event(int kind, int l, int t) const {
        return ev[((size_t)kind * desc.n_layers + l) * kRing + (t % kRing)];
    }
};

namespace {

#define PFAIL(code, ...)                                  \
    do {                                                  \
        char _buf[512];                                   \
        snprintf(_buf, sizeof _buf, __VA_ARGS__);         \
        set_error(_buf);                                  \
        return (code);                                    \
    } while (0)

// Timing of the next launch of `kind` on stream s: records its start event
// on s (a marker, ~3 us of queue time; binding a start event to the kernel
// would cost the enqueuing thread 9-19 us per launch) and returns its stop
// event, to be bound to the launch's last kernel.  nullptr when the launch is
// not timed (kind not armed, not one in `every`, or capacity used up).
// Kind 0 is taken by the calling thread, kinds 1-3 by whichever thread issues
// the chain.
hipEvent_t timed(oasis_pipeline *p, int kind, hipStream_t s) {
    if (!(p->t_kinds >> kind & 1u) || p->t_n[kind] >= p->t_cap) return nullptr;
    if (p->t_seen[kind]++ % p->t_every != 0) return nullptr;
    const int i = p->t_n[kind]++;
    (void)hipEventRecord(p->t_ev[kind][2 * i], s);
    return p->t_ev[kind][2 * i + 1];
}

// The copy half of staging for one job; called by the calling thread
// (kernel copies) or by the copy worker (DMA copies; any copies with issue
// threads).  On the copy worker a gather waits for its plan on the host, so
// that the copy stream gets no barrier packet (the plan and what it waits
// for are already enqueued): the ragged 32B-class layer runs at 165k against
// 159k tok/s.
int run_copy(oasis_pipeline *p, const Job &j) {
    if (p->threaded && j.args.copy_mode == OASIS_COPY_KERNEL && j.args.plan_event) {
        const hipError_t e = hipEventSynchronize(static_cast<hipEvent_t>(j.args.plan_event));
        if (e != hipSuccess) return hip_check(e, "hipEventSynchronize");
    }
    const auto h0 = std::chrono::steady_clock::now();
    const int rc = oasis_stage_copy(&p->d, &j.args);
    const double dt = std::chrono::duration<double>(std::chrono::steady_clock::now() - h0).count();
    std::lock_guard<std::mutex> lk(p->t_mu);
    p->copy_host_s += dt;
    p->copy_calls++;
    return rc;
}

int worker_error(oasis_pipeline *p) {
    std::string msg;
    int rc = p->chain.error(&msg);
    if (rc == OASIS_OK) rc = p->copies.error(&msg);
    if (rc != OASIS_OK) set_error(msg);
    return rc;
}

// The copy engine of layer l's staging.
int layer_copy_mode(const oasis_pipeline_desc &ds, int l) {
    if (ds.copy_mode == OASIS_COPY_MIXED) return (l & 1) ? OASIS_COPY_KERNEL : OASIS_COPY_DMA;
    return ds.copy_mode;
}

int check_layer(const oasis_pipeline_desc &ds, const oasis_layer_buffers &b, int l, size_t plan_need,
                size_t ws_need) {
#define LNEED(ptr)                                                                   \
    do {                                                                             \
        if ((ptr) == nullptr) PFAIL(OASIS_EINVAL, "layer %d: %s is NULL", l, #ptr);  \
    } while (0)
    LNEED(b.scores);
    for (int k = 0; k < 2; k++) {
        LNEED(b.sel[k]);
        LNEED(b.n_sel[k]);
    }
    if (ws_need > 0) {
        LNEED(b.attn_ws);
        if (b.attn_ws_bytes < ws_need)
            PFAIL(OASIS_ENOSPACE, "layer %d: attention workspace %zu bytes < %zu", l, b.attn_ws_bytes, ws_need);
    }
    if (!ds.staged) return OASIS_OK;
    LNEED(b.ws_pool);
    LNEED(b.slot_block);
    LNEED(b.slot_stamp);
    for (int k = 0; k < 3; k++) {
        LNEED(b.tbl_slot[k]);
        LNEED(b.tbl_block[k]);
        LNEED(b.tbl_n[k]);
    }
    for (int k = 0; k < 2; k++) LNEED(b.plan[k]);
    if (b.plan_bytes < plan_need)
        PFAIL(OASIS_ENOSPACE, "layer %d: plan buffers %zu bytes < %zu", l, b.plan_bytes, plan_need);
    if (layer_copy_mode(ds, l) == OASIS_COPY_DMA) {
        LNEED(b.host_plan);
        LNEED(b.stage_host[0]);
        LNEED(b.stage_host[1]);
        LNEED(b.stage_dev);
        if (b.stage_bytes < kBlockBytes)
            PFAIL(OASIS_ENOSPACE, "layer %d: staging buffers of %zu bytes hold no block", l, b.stage_bytes);
    }
    return OASIS_OK;
#undef LNEED
}

void release(oasis_pipeline *p) {
    p->chain.stop();  // its last jobs may still hand copies on
    p->copies.stop();
    for (hipStream_t c : p->comp)
        if (c) (void)hipStreamSynchronize(c);
    for (hipStream_t c : p->copy)
        if (c) (void)hipStreamSynchronize(c);
    (void)hipStreamSynchronize(p->main);
    for (hipEvent_t e : p->ev)
        if (e) (void)hipEventDestroy(e);
    for (auto &v : p->t_ev)
        for (hipEvent_t e : v)
            if (e) (void)hipEventDestroy(e);
    if (!p->comp_on_main)
        for (hipStream_t c : p->comp)
            if (c) (void)hipStreamDestroy(c);
    for (hipStream_t c : p->copy)
        if (c) (void)hipStreamDestroy(c);
    delete p;
}

}  // namespace

extern "C" {

static int issue_chain(oasis_pipeline *p, int l, int t, const uint16_t *q_look, hipEvent_t attn_prev);

int oasis_pipeline_create(const oasis_dims *dims, const oasis_pipeline_desc *desc, oasis_pipeline **out) {
    clear_error();
    if (!out) PFAIL(OASIS_EINVAL, "out is NULL");
    *out = nullptr;
    if (!dims || !desc) PFAIL(OASIS_EINVAL, "dims or desc is NULL");
    const oasis_pipeline_desc &ds = *desc;
    if (ds.n_layers < 1 || ds.n_layers > 1024) PFAIL(OASIS_EINVAL, "n_layers = %d outside [1, 1024]", ds.n_layers);
    if (ds.K_b < 1) PFAIL(OASIS_EINVAL, "K_b = %d < 1", ds.K_b);
    if (ds.J < 1) PFAIL(OASIS_EINVAL, "J = %d < 1", ds.J);
    if (ds.n_q < 1) PFAIL(OASIS_EINVAL, "n_q = %d < 1", ds.n_q);
    if (ds.staged != 0 && ds.staged != 1) PFAIL(OASIS_EINVAL, "staged = %d", ds.staged);
    if (ds.staged && (ds.C < 0 || ds.C > ds.K_b)) PFAIL(OASIS_EINVAL, "C = %d outside [0, K_b]", ds.C);
    if (ds.copy_mode != OASIS_COPY_KERNEL && ds.copy_mode != OASIS_COPY_DMA && ds.copy_mode != OASIS_COPY_MIXED)
        PFAIL(OASIS_EINVAL, "copy_mode = %d", ds.copy_mode);
    if (!ds.pool || !ds.kminmax || !ds.ctx_len || !ds.layers) PFAIL(OASIS_EINVAL, "pool, kminmax, ctx_len or layers is NULL");
    if (ds.n_split < 0 || ds.n_split > 64) PFAIL(OASIS_EINVAL, "n_split = %d outside [0, 64]", ds.n_split);
    if (ds.issue_threads < -1 || ds.issue_threads > 1)
        PFAIL(OASIS_EINVAL, "issue_threads = %d outside [-1, 1]", ds.issue_threads);
    if (ds.compute_streams < -1 || ds.compute_streams > 2)
        PFAIL(OASIS_EINVAL, "compute_streams = %d outside [-1, 2]", ds.compute_streams);
    int rc0 = check_dims(dims);
    if (rc0) return rc0;
    if ((int64_t)ds.n_q * (dims->H_q / dims->H_kv) > kMaxG)
        PFAIL(OASIS_EUNSUPPORTED, "n_q * H_q / H_kv = %lld (at most %d)",
              (long long)ds.n_q * (dims->H_q / dims->H_kv), kMaxG);
    const size_t plan_need = oasis_stage_plan_bytes(dims, ds.K_b);
    const size_t ws_need = oasis_lookahead_attn_workspace_bytes(dims, ds.n_q, ds.K_b, ds.n_split);
    for (int l = 0; l < ds.n_layers; l++) {
        int rc = check_layer(ds, ds.layers[l], l, plan_need, ws_need);
        if (rc) return rc;
    }
    auto *p = new (std::nothrow) oasis_pipeline();
    if (!p) PFAIL(OASIS_EINVAL, "out of host memory");
    p->d = *dims;
    p->desc = ds;
    p->layers.assign(ds.layers, ds.layers + ds.n_layers);
    p->desc.layers = nullptr;
    p->next_step.assign(ds.n_layers, 0);
    p->attn_last.assign(ds.n_layers, nullptr);
    p->sel_last.assign(ds.n_layers, nullptr);
    p->S = ds.K_b + (ds.staged ? ds.C : 0);
    p->main = static_cast<hipStream_t>(ds.main_stream);
    auto fail = [&](hipError_t e, const char *what) {
        hip_check(e, what);
        release(p);
        return OASIS_EHIP;
    };
    hipError_t e = hipGetDevice(&p->device);
    if (e != hipSuccess) return fail(e, "hipGetDevice");
    // compute streams: with two, even and odd layers alternate, so that one
    // layer's latency-bound top-K and plan overlap the next layer's scores.
    // That pays for a staged step with fewer (request, KV head) pairs than
    // compute units (the 32B-class ragged layer, 128 pairs: 176k against
    // 143k tok/s with one) and for a staged step that HBM binds (the Qwen3-8B
    // layer at batch 128 with a fetch cap of one or two blocks: 393k / 360k
    // against 343k / 320k).  Without staging one compute stream is better:
    // its scores and the attention are the step's HBM traffic, and a second
    // stream only adds a second score kernel taking bandwidth from the
    // attention (Qwen3-8B in HBM at batch 32: 470k against 431k; the
    // reasoning layer: 356k against 351k).  A staged step whose admits can
    // take the link much longer than its HBM kernels take HBM is link-bound:
    // the chain then runs on the main stream behind each attention
    // (compute_streams = -1), so the kernels that read HBM never run beside
    // one another, only beside the copies, and the hardware queues go to two
    // gather streams.  The Qwen3-8B layer at batch 128 (1024 pairs, K_b 128,
    // 1024 blocks of context), fetch cap C blocks per pair per step, tok/s
    // with the chain on the main stream / two compute streams: C = 3: 248k /
    // 271k, C = 4: 216k / 209k, C = 5: 175k / 169k, C = 6: 160k / 156k.  The
    // link time of C blocks per pair over the HBM time of the pair's
    // attention and score bytes is 1.65 at C = 3 and 2.2 at C = 4; the rule
    // below switches at 2.
    int n_comp = ds.compute_streams;
    if (n_comp == 0) {
        const int64_t pairs = (int64_t)dims->B * dims->H_kv;
        const double link_s = (double)ds.C * kBlockBytes / kLinkBytesPerS;
        const double hbm_s = ((double)ds.K_b * kBlockBytes + (double)dims->NB_max * kSummaryBytes) / kHbmBytesPerS;
        const bool link_bound = ds.staged && link_s > 2.0 * hbm_s;
        n_comp = !ds.staged ? 1 : (pairs < device_cu_count() || !link_bound) ? 2 : -1;
    }
    if (n_comp < 0) {
        p->comp_on_main = true;
        p->comp[0] = p->main;
    }
    for (int c = 0; c < n_comp; c++)
        if ((e = hipStreamCreateWithFlags(&p->comp[c], hipStreamNonBlocking)) != hipSuccess)
            return fail(e, "hipStreamCreateWithFlags");
    // copy streams: with one compute stream the zero-copy engine alternates
    // two by layer, so that the tail of one layer's gather overlaps the start
    // of the next one's; otherwise one (at most four streams in all, the
    // process's hardware queues).  The DMA engine's copies all go through
    // one (its packing is serial anyway); the mixed engine has one for the
    // DMA layers and one for the gather layers.
    const int n_copy = !ds.staged                           ? 0
                       : ds.copy_mode == OASIS_COPY_MIXED    ? 2
                       : ds.copy_mode == OASIS_COPY_KERNEL && n_comp <= 1 ? 2
                                                              : 1;
    for (int c = 0; c < n_copy; c++)
        if ((e = hipStreamCreateWithFlags(&p->copy[c], hipStreamNonBlocking)) != hipSuccess)
            return fail(e, "hipStreamCreateWithFlags");
    p->ev.assign((size_t)kEvKinds * ds.n_layers * kRing, nullptr);
    for (auto &x : p->ev)
        if ((e = hipEventCreateWithFlags(&x, hipEventDisableTiming)) != hipSuccess)
            return fail(e, "hipEventCreateWithFlags");
    // issue threads: the chain and the copies are enqueued by two worker
    // threads of their own, so that the calling thread enqueues only the
    // attention, and the cross-stream waits of the chain (the top-K's on the
    // attention of step t - 1, a gather's on its plan) and, without staging,
    // the attention's on the selection of step t - 1 are made on the host by
    // the thread that enqueues the waiting work, after the work it waits for
    // was enqueued.  Those queues then carry no barrier packets, each of
    // which holds its queue ~3 us even when its event has completed, and a
    // stream wait on a pending event costs the enqueuing thread 8 to 24 us
    // (MI355X, ROCm 7.2).  Measured against issue_threads = -1: the ragged
    // 32B-class staged layer 155k -> 176k tok/s (with the events bound to the
    // kernels), Qwen3-8B in HBM at batch 32 420k -> 472k, the B = 1 parity
    // layer 50k -> 52.7k.
    p->threaded = !p->comp_on_main && ds.issue_threads >= 0;
    if (p->threaded) {
        p->chain.start(
            ds.n_layers,
            [p](const ChainJob &j, std::string *msg) {
                const int rc = issue_chain(p, j.layer, j.step, j.q_look, j.attn_prev);
                if (rc != OASIS_OK) {
                    *msg = "scores, top-K or plan of layer " + std::to_string(j.layer) + " step " +
                           std::to_string(j.step) + ": " + oasis_last_error();
                    p->copies.fail(rc, *msg);  // its copies never come: release whoever waits for them
                }
                return rc;
            },
            [p] { (void)hipSetDevice(p->device); });
    }
    if (ds.staged && (ds.copy_mode != OASIS_COPY_KERNEL || p->threaded)) {
        p->copies.start(
            ds.n_layers,
            [p](const Job &j, std::string *msg) {
                const int rc = run_copy(p, j);
                if (rc != OASIS_OK)
                    *msg = "staging copy of layer " + std::to_string(j.layer) + " step " + std::to_string(j.step) +
                           ": " + oasis_last_error();
                return rc;
            },
            [p] { (void)hipSetDevice(p->device); });
    }
    *out = p;
    return OASIS_OK;
}

// The background half of layer-step (l, t): scores, top-K and (staged) the
// staging plan for step t + 1 from the lookahead queries, then the copies
// (handed to the copy worker when there is one).  Runs on the calling thread,
// or on the chain worker in submission order.
static int issue_chain(oasis_pipeline *p, int l, int t, const uint16_t *q_look, hipEvent_t attn_prev) {
    const oasis_pipeline_desc &ds = p->desc;
    const oasis_layer_buffers &b = p->layers[l];
    const oasis_dims *d = &p->d;
    const int K_b = ds.K_b;
    const int j = t % 2;
    const int mode = layer_copy_mode(ds, l);
    int rc;
    hipStream_t cs = p->comp[p->comp[1] ? (l & 1) : 0];
    const hipEvent_t sc = timed(p, 1, cs);
    if ((rc = score_blocks(d, q_look, ds.J, ds.kminmax, ds.ctx_len, b.scores, cs, sc))) return rc;
    if (t >= 2) {
        // unstaged: sel[j], read by the attention of step t - 1.  Staged: the
        // attention of step t - 1 covers every later reuse: table
        // (t + 1) % 3 (read by the attention of step t - 2, earlier on the
        // main stream), plan[j] (read by the copies of step t - 2, which
        // that attention waited for) and the slots this step's copies may
        // refill (read by that attention itself)
        // On the chain worker the wait is made on the host: the attention of
        // step t - 1 and everything it waits for are already enqueued, so the
        // worker cannot block anything it would have to enqueue itself, and
        // the compute stream gets no barrier packet, each of which holds its
        // queue ~3 us even when its event has completed (the ragged 32B-class
        // layer: 159k against 155k tok/s).  No event: timing was re-armed
        // since, after everything enqueued had finished.
        if (attn_prev) {
            if (p->threaded) OASIS_HIP(hipEventSynchronize(attn_prev));
            else OASIS_HIP(stream_wait(cs, attn_prev));
        }
    }
    hipEvent_t tk = timed(p, 2, cs);
    if (!ds.staged && !tk) tk = p->event(kEvSel, l, t);
    if ((rc = select_topk(d, b.scores, ds.ctx_len, K_b, b.sel[j], b.n_sel[j], cs, tk))) return rc;
    if (!ds.staged) {
        // read by the calling thread at step t + 1 (after the chain worker has
        // run this job, when there is one)
        p->sel_last[l] = tk;
        return OASIS_OK;
    }

    Job job;
    job.layer = l;
    job.step = t;
    oasis_stage_args &a = job.args;
    const int k1 = (t + 1) % 3;
    a.sel = b.sel[j];
    a.n_sel = b.n_sel[j];
    a.K_sel = K_b;
    a.scores = b.scores;
    a.K_b = K_b;
    a.C = t == 0 ? K_b : ds.C;
    a.S = p->S;
    a.step = t;
    a.slot_block = b.slot_block;
    a.slot_stamp = b.slot_stamp;
    a.ctx_len = ds.ctx_len;
    a.host_pool = ds.pool;
    a.ws_pool = b.ws_pool;
    a.tbl_slot = b.tbl_slot[k1];
    a.tbl_block = b.tbl_block[k1];
    a.tbl_n = b.tbl_n[k1];
    a.plan = b.plan[j];
    a.plan_bytes = b.plan_bytes;
    a.host_plan = b.host_plan;
    a.host_plan_bytes = b.plan_bytes;
    a.stage_host = b.stage_host[j];
    a.stage_host_bytes = b.stage_bytes;
    a.stage_dev = b.stage_dev;
    a.stage_dev_bytes = b.stage_bytes;
    a.host_threads = ds.host_threads;
    a.copy_mode = mode;
    a.stream = cs;
    // mixed: copy[0] carries the DMA (even) layers, copy[1] the gathers (odd);
    // otherwise the layers alternate over the copy streams there are
    a.copy_stream = p->copy[p->copy[1] ? (l & 1) : 0];
    // the copies follow the plan, which followed the attention of step t - 1
    a.wait_event = nullptr;
    a.done_event = p->event(kEvStage, l, t);
    const hipEvent_t pe = timed(p, 3, cs);
    a.plan_event = pe ? pe : p->event(kEvPlan, l, t);
    a.stats_accum = ds.stage_stats;
    if ((rc = oasis_stage_plan(d, &a))) return rc;
    if (mode == OASIS_COPY_DMA || p->threaded) {
        p->copies.push(job);
    } else if ((rc = run_copy(p, job))) {
        return rc;
    }
    return OASIS_OK;
}

int oasis_pipeline_layer_step(oasis_pipeline *p, int32_t l, int32_t t, const uint16_t *q_look,
                              const uint16_t *q_attn, uint16_t *out, float *lse) {
    clear_error();
    if (!p) PFAIL(OASIS_EINVAL, "pipeline is NULL");
    const oasis_pipeline_desc &ds = p->desc;
    if (l < 0 || l >= ds.n_layers) PFAIL(OASIS_EINVAL, "layer = %d outside [0, %d)", l, ds.n_layers);
    if (t != p->next_step[l]) PFAIL(OASIS_EINVAL, "layer %d: step %d issued, step %d expected", l, t, p->next_step[l]);
    if (!q_look) PFAIL(OASIS_EINVAL, "q_look is NULL");
    if (t >= 1 && (!q_attn || !out)) PFAIL(OASIS_EINVAL, "q_attn or out is NULL at step %d", t);
    int rc;
    if ((rc = worker_error(p))) return rc;
    const oasis_layer_buffers &b = p->layers[l];
    const oasis_dims *d = &p->d;
    const int K_b = ds.K_b;
    const int mode = layer_copy_mode(ds, l);

    // foreground: attention of step t
    const hipEvent_t attn_prev = p->attn_last[l];
    if (t >= 1) {
        hipEvent_t done = nullptr;
        if (ds.staged) {
            // the copy worker has recorded the copies of step t - 1
            if (mode == OASIS_COPY_DMA || p->threaded) (void)p->copies.wait_done(l, t - 1);
            if ((rc = worker_error(p))) return rc;
            OASIS_HIP(stream_wait(p->main, p->event(kEvStage, l, t - 1)));
            const int k = t % 3;
            done = timed(p, 0, p->main);
            if (!done) done = p->event(kEvAttn, l, t);
            rc = lookahead_attn(d, ds.n_q, q_attn, b.ws_pool, p->S, b.tbl_slot[k], b.tbl_block[k], b.tbl_n[k], K_b,
                                ds.ctx_len, ds.sm_scale, out, lse, b.attn_ws, b.attn_ws_bytes, ds.n_split, p->main,
                                done);
        } else {
            const int jp = (t - 1) % 2;
            if (p->threaded) {
                // the chain worker has bound the selection event of step t - 1;
                // the wait itself is made on the host, so that the main stream
                // carries only attention launches (a barrier packet holds a
                // queue ~3 us even when its event has completed)
                (void)p->chain.wait_done(l, t - 1);
                if ((rc = worker_error(p))) return rc;
                if (p->sel_last[l]) OASIS_HIP(hipEventSynchronize(p->sel_last[l]));
            } else if (p->sel_last[l]) {
                OASIS_HIP(stream_wait(p->main, p->sel_last[l]));
            }
            done = timed(p, 0, p->main);
            if (!done) done = p->event(kEvAttn, l, t);
            rc = lookahead_attn(d, ds.n_q, q_attn, ds.pool, d->NB_max, b.sel[jp], b.sel[jp], b.n_sel[jp], K_b,
                                ds.ctx_len, ds.sm_scale, out, lse, b.attn_ws, b.attn_ws_bytes, ds.n_split, p->main,
                                done);
        }
        if (rc) return rc;
        p->attn_last[l] = done;
    }

    p->next_step[l] = t + 1;
    if (p->threaded) {
        p->chain.push(ChainJob{l, t, q_look, attn_prev});
        return OASIS_OK;
    }
    return issue_chain(p, l, t, q_look, attn_prev);
}

int oasis_pipeline_drain(oasis_pipeline *p) {
    clear_error();
    if (!p) PFAIL(OASIS_EINVAL, "pipeline is NULL");
    (void)p->chain.drain();  // before the copies: its jobs hand copies on
    (void)p->copies.drain();
    return worker_error(p);
}

int oasis_pipeline_stream(oasis_pipeline *p, int32_t which, void **stream) {
    clear_error();
    if (!p || !stream) PFAIL(OASIS_EINVAL, "pipeline or stream is NULL");
    if (which < 0 || which > 4) PFAIL(OASIS_EINVAL, "which = %d outside [0, 4]", which);
    *stream = which == 0   ? (void *)p->main
              : which == 1 ? (void *)p->comp[0]
              : which == 4 ? (void *)p->comp[1]
                           : (void *)p->copy[which - 2];
    return OASIS_OK;
}

int oasis_pipeline_issue_threads(oasis_pipeline *p, int32_t *on) {
    clear_error();
    if (!p || !on) PFAIL(OASIS_EINVAL, "pipeline or on is NULL");
    *on = p->threaded ? 1 : 0;
    return OASIS_OK;
}

int oasis_pipeline_timing(oasis_pipeline *p, int32_t capacity, uint32_t kinds, int32_t every) {
    clear_error();
    if (!p) PFAIL(OASIS_EINVAL, "pipeline is NULL");
    if (capacity < 0 || capacity > (1 << 20)) PFAIL(OASIS_EINVAL, "capacity = %d", capacity);
    if (every < 1) PFAIL(OASIS_EINVAL, "every = %d < 1", every);
    if (kinds >> kTimedKinds) PFAIL(OASIS_EINVAL, "kinds = 0x%x (bits 0 .. %d)", kinds, kTimedKinds - 1);
    int rc = oasis_pipeline_drain(p);
    if (rc) return rc;
    // The timing events are bound to launches again from the first one on, so
    // no wait still to be issued may name one: let everything enqueued
    // finish, after which the next steps need no wait on earlier launches.
    OASIS_HIP(hipStreamSynchronize(p->main));  // NULL: the default stream
    for (hipStream_t c : {p->comp[0], p->comp[1], p->copy[0], p->copy[1]})
        if (c) OASIS_HIP(hipStreamSynchronize(c));
    std::fill(p->attn_last.begin(), p->attn_last.end(), nullptr);
    std::fill(p->sel_last.begin(), p->sel_last.end(), nullptr);
    for (int k = 0; k < kTimedKinds; k++) {
        auto &v = p->t_ev[k];
        while ((int)v.size() < 2 * capacity) {
            hipEvent_t e = nullptr;
            OASIS_HIP(hipEventCreate(&e));
            v.push_back(e);
        }
        p->t_n[k] = 0;
        p->t_seen[k] = 0;
    }
    p->t_cap = capacity;
    p->t_every = every;
    p->t_kinds = kinds;
    std::lock_guard<std::mutex> lk(p->t_mu);
    p->copy_host_s = 0.0;
    p->copy_calls = 0;
    return OASIS_OK;
}

int oasis_pipeline_timing_read(oasis_pipeline *p, int32_t kind, double *total_ms, int32_t *count) {
    clear_error();
    if (!p || !total_ms || !count) PFAIL(OASIS_EINVAL, "pipeline, total_ms or count is NULL");
    if (kind < 0 || kind >= kTimedKinds) PFAIL(OASIS_EINVAL, "kind = %d", kind);
    int rc = oasis_pipeline_drain(p);
    if (rc) return rc;
    double sum = 0.0;
    for (int i = 0; i < p->t_n[kind]; i++) {
        OASIS_HIP(hipEventSynchronize(p->t_ev[kind][2 * i + 1]));
        float ms = 0.f;
        OASIS_HIP(hipEventElapsedTime(&ms, p->t_ev[kind][2 * i], p->t_ev[kind][2 * i + 1]));
        sum += ms;
    }
    *total_ms = sum;
    *count = p->t_n[kind];
    return OASIS_OK;
}

int oasis_pipeline_timing_values(oasis_pipeline *p, int32_t kind, float *ms, int32_t capacity, int32_t *count) {
    clear_error();
    if (!p || !count || (!ms && capacity > 0)) PFAIL(OASIS_EINVAL, "pipeline, ms or count is NULL");
    if (kind < 0 || kind >= kTimedKinds) PFAIL(OASIS_EINVAL, "kind = %d", kind);
    if (capacity < 0) PFAIL(OASIS_EINVAL, "capacity = %d", capacity);
    int rc = oasis_pipeline_drain(p);
    if (rc) return rc;
    const int n = p->t_n[kind] < capacity ? p->t_n[kind] : capacity;
    for (int i = 0; i < n; i++) {
        OASIS_HIP(hipEventSynchronize(p->t_ev[kind][2 * i + 1]));
        OASIS_HIP(hipEventElapsedTime(&ms[i], p->t_ev[kind][2 * i], p->t_ev[kind][2 * i + 1]));
    }
    *count = p->t_n[kind];
    return OASIS_OK;
}

int oasis_pipeline_copy_host_seconds(oasis_pipeline *p, double *seconds, int32_t *calls) {
    clear_error();
    if (!p || !seconds || !calls) PFAIL(OASIS_EINVAL, "pipeline, seconds or calls is NULL");
    std::lock_guard<std::mutex> lk(p->t_mu);
    *seconds = p->copy_host_s;
    *calls = p->copy_calls;
    return OASIS_OK;
}

int oasis_pipeline_destroy(oasis_pipeline *p) {
    clear_error();
    if (!p) return OASIS_OK;
    release(p);
    return OASIS_OK;
}

}  // extern "C"
