/*
 * oasis.h -- C ABI of liboasis.so, the decode hot path of lookahead block
 * scoring with sparse KV staging, for AMD Instinct MI355X (gfx950).
 *
 * The method is OasisKV (arXiv 2608.08097, "OasisKV: Scaling In-Decode KV
 * Cache Beyond HBM with Lookahead Sparse Prefetching"); the paperlayer
 * summary's section 4 ("System Design") describes the per-layer decode chain
 * that these calls implement, one entry point per step: block scores from the
 * draft queries against two summary vectors per block (coordinate-wise key
 * minimum and maximum); the best blocks that fit a token budget; an update of
 * the HBM working set that brings in at most C missing blocks per KV head and
 * layer in place of the blocks predicted longest ago, copying them from the
 * host copy of the cache; attention over the working set alone.
 *
 * Conventions shared by every call
 * --------------------------------
 *  - bf16 tensors are passed as uint16_t bit patterns; every array is dense
 *    row-major with the layout written next to it.
 *  - Query head g belongs to KV head g / (H_q / H_kv).
 *  - Request r has n_b(r) = ceil(ctx_len[r] / bs) blocks; token i of block b
 *    is position b * bs + i and is valid iff that is < ctx_len[r].
 *  - K/V pools are [B][H_kv][P][2][bs][D]: one block of one KV head is K
 *    (bs x D) followed by V (bs x D), 2 * bs * D * 2 bytes contiguous.
 *  - "device" pointers are HBM allocations of the current HIP device;
 *    "pinned host" pointers come from hipHostMalloc (e.g. torch pin_memory).
 *    The caller owns every buffer; no call allocates device memory.
 *  - `stream` arguments are hipStream_t values passed as void* (NULL = the
 *    null stream); events are hipEvent_t values passed as void*.  Calls only
 *    enqueue work and return without synchronising the device, except where
 *    a call says otherwise.
 *  - Every call returns OASIS_OK or a negative error code; argument errors
 *    are detected on the host before any work is enqueued, so a failed call
 *    has no effect.  oasis_last_error() returns a per-thread message for the
 *    last failure.  No C++ exception crosses this interface.
 *  - Supported shapes: D = 128, bs = 16, 1 <= H_q / H_kv <= 16,
 *    NB_max <= 16384; staging: S <= 2048 slots, K_sel <= 1024.  Others
 *    return OASIS_EUNSUPPORTED.
 *  - Device-resident indices (selections, slot tables, attention tables) are
 *    range-checked by the kernels: an index outside its documented range is
 *    skipped, never dereferenced.
 */
#ifndef OASIS_H
#define OASIS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define OASIS_OK 0
#define OASIS_EINVAL (-1)        /* null pointer, bad shape or bad value */
#define OASIS_EUNSUPPORTED (-2)  /* valid but unsupported shape */
#define OASIS_EHIP (-3)          /* the HIP runtime reported an error */
#define OASIS_ENOSPACE (-4)      /* workspace or plan buffer too small */

/* Copy engines for oasis_stage_blocks. */
#define OASIS_COPY_KERNEL 0      /* device kernel reads the mapped pinned pool */
#define OASIS_COPY_DMA 1         /* host packs, DMA engine copies, device scatters */
#define OASIS_COPY_MIXED 2       /* layer pipeline only: even layers OASIS_COPY_DMA,
                                    odd layers OASIS_COPY_KERNEL */

typedef struct oasis_dims {
    int32_t B;       /* requests in the batch (0 = nothing to do) */
    int32_t H_q;     /* query heads */
    int32_t H_kv;    /* KV heads; H_q % H_kv == 0 */
    int32_t D;       /* head dimension (128) */
    int32_t bs;      /* tokens per block (16) */
    int32_t NB_max;  /* block capacity per (request, KV head) of the summary
                        and score arrays and of a full pool */
} oasis_dims;

/* Library version string, e.g. "oasis 0.1.0 gfx950". */
const char *oasis_version(void);

/* Message for the calling thread's last failed call ("" if none). */
const char *oasis_last_error(void);

/* Pinned host memory for the KV pool and the staging buffers (hipHostMalloc,
 * default flags), with every page mapped into the process before the call
 * returns.  Pinned pages that only a device has written are otherwise
 * mapped for the CPU on first touch, one fault per 4 KiB page; the DMA
 * engine's packing threads visit fresh pages of the pool every step and would
 * pay that each time.  On success *ptr holds `bytes` bytes (contents
 * unspecified); release with oasis_host_free.  Returns OASIS_EINVAL for a
 * NULL ptr or zero bytes, OASIS_EHIP if the runtime cannot pin the memory. */
int oasis_host_alloc(size_t bytes, void **ptr);
int oasis_host_free(void *ptr);

/* Blocks per KV head per layer per step admitted under a fetch-cap fraction
 * (section 4 bounds the transfer to C blocks per KV head per layer; sections
 * 5 and the agihunt summary give the cap as a fraction, default 0.05):
 * C = max(1, floor(cap * K_b)) for 0 < cap < 1, K_b for cap >= 1 (fetch-all),
 * 0 for cap <= 0 or NaN.  Returns -1 if K_b < 1. */
int32_t oasis_fetch_cap_blocks(double cap, int32_t K_b);

/* Per-block key summaries (section 4: coordinate-wise minimum and maximum of
 * the block's keys, two vectors per block).
 *   kv       [B][H_kv][NB_max][2][bs][D] bf16, device or pinned host
 *   ctx_len  [B] int32, device
 *   kminmax  [B][H_kv][NB_max][2][D] bf16, device; index 0 = min, 1 = max,
 *            over the block's valid tokens only.  Entries of blocks
 *            b >= n_b(r) are not written.
 * Setup work, not part of a decode step. */
int oasis_build_summaries(const oasis_dims *dims, const uint16_t *kv,
                          const int32_t *ctx_len, uint16_t *kminmax,
                          void *stream);

/* Lookahead block scores (section 4: the draft queries scan the compressed
 * per-block key summaries to rank blocks).  For KV head h of request r and
 * block b < n_b(r):
 *     s = sum_{j < J} sum_{g in group(h)} sum_d max(q[j,g,d] kmax[d], q[j,g,d] kmin[d])
 * (the largest value q . k can take over the block's bounding box, summed
 * over drafts and the group's query heads), accumulated in fp64 and rounded
 * once to fp32.  Blocks b >= n_b(r) get -inf.
 *   q_look   [B][J][H_q][D] bf16, device
 *   kminmax  [B][H_kv][NB_max][2][D] bf16, device (from oasis_build_summaries)
 *   ctx_len  [B] int32, device
 *   scores   [B][H_kv][NB_max] fp32, device, written
 * Requires J >= 1 and ctx_len[r] <= NB_max * bs (larger values are clamped to
 * NB_max blocks).  J > 64, or B * H_kv * ceil(NB_max / 64) above 2^31 - 1,
 * returns OASIS_EUNSUPPORTED. */
int oasis_score_blocks(const oasis_dims *dims, const uint16_t *q_look,
                       int32_t J, const uint16_t *kminmax,
                       const int32_t *ctx_len, float *scores, void *stream);

/* Top-K block selection under the token budget (sections 4 and 5: per KV
 * head and layer, the K_b = budget / bs best-scoring blocks are predicted for
 * the next step; default budget 2048 tokens).  Order: fp32 score descending,
 * equal scores by lower block id, NaN below -inf (+0 and -0 equal).  When
 * n_b(r) <= K_b every block is taken.
 *   scores   [B][H_kv][NB_max] fp32, device; entries b >= n_b(r) ignored
 *   ctx_len  [B] int32, device
 *   sel      [B][H_kv][K_b] int32, device, written: chosen ids ascending,
 *            then -1
 *   n_sel    [B][H_kv] int32, device, written: min(n_b(r), K_b) */
int oasis_select_topk(const oasis_dims *dims, const float *scores,
                      const int32_t *ctx_len, int32_t K_b, int32_t *sel,
                      int32_t *n_sel, void *stream);

/* Staging of the predicted set into the HBM working set (section 4: the
 * predicted blocks already resident stay; at most C missing ones per KV head
 * and layer are brought in, each displacing the resident block whose last
 * prediction is oldest; the copies come from the off-GPU pool and must land
 * before the next step's attention). *
 * State per (request r, KV head h) lives in a slot table of S slots:
 * slot_block[s] is the block held by slot s (-1 = free) and slot_stamp[s] the
 * last step at which that block was predicted or admitted.  The resident set
 * R is the set of held blocks.  Initialise slot_block to -1 before step 0.
 * Given the predicted set P (sel / n_sel) of step `step`:
 *   1. blocks of P that are resident get stamp = step;
 *   2. the admitted list A is the first min(C, |P \ R|) blocks of P \ R in
 *      order of fp32 score descending, then block id ascending;
 *   3. free capacity K_b - |R| is used first; each further admit evicts one
 *      block of R \ P, taking them by stamp ascending, then block id
 *      ascending;
 *   4. admitted blocks are placed into slots that were free before this step
 *      (ascending slot index in admission order), so a slot evicted now is
 *      not overwritten until the next step: the attention still reading the
 *      previous table is never raced.  S >= K_b + C guarantees such a slot
 *      for every admit; with fewer slots, admits beyond the free slots are
 *      dropped this step (an empty table, as at step 0, always has room);
 *   5. each admitted block (8 KiB for bs = 16, D = 128) is copied from
 *      host_pool[r][h][block] to ws_pool[r][h][slot].
 * Step 0 with C = K_b is the uncapped initial fill.  Resident blocks that are
 * no longer predicted stay resident (and attended) until evicted.
 *
 * The table for the next attention (tbl_slot / tbl_block / tbl_n, capacity
 * K_b entries per (r, h)) lists every resident slot after the step, in
 * ascending slot order.  It must not be a table that an attention still in
 * flight reads: rotate two tables when each stage call waits for the
 * previous attention, three when stage calls may run one attention ahead.
 *
 * Ordering: the slot-table update and plan run on `stream`.  Copies run on
 * `copy_stream` (NULL = `stream`) after the plan and after `wait_event` (if
 * not NULL).  The copies of this call never touch a slot listed in the table
 * written by the previous call, but may refill slots listed in the table
 * written two calls earlier (blocks the previous call evicted): `wait_event`
 * must mark the end of every attention that read that older table.
 * `done_event` (if not NULL) completes on `copy_stream` with the last copy
 * (with OASIS_COPY_KERNEL it is bound to the gather kernel itself, so it adds
 * no marker to the queue): make the next attention wait on it.
 *
 * Copy engines:
 *  - OASIS_COPY_DMA reads the plan back into `host_plan` (pinned host, at
 *    least oasis_stage_plan_bytes()), BLOCKING THE CALLING THREAD until the
 *    plan kernel has finished; `host_threads` worker threads (0 = 8) then pack
 *    the admitted blocks into `stage_host` (pinned host), one hipMemcpyAsync on
 *    copy_stream moves them into `stage_dev` (device), and a scatter kernel on
 *    copy_stream places them into their slots.  The staging buffers hold
 *    floor(bytes / 8 KiB) blocks each; more admits than that are moved in
 *    rounds, the call waiting on the host for each round's copy before it
 *    repacks.  The call returns once the last copy is enqueued.  A later call
 *    that packs into the same `stage_host` first waits for this call's copy
 *    (the library remembers the last few buffers per thread), so alternating
 *    two staging buffers lets packing overlap the previous step's copy.  The
 *    DMA engines leave the compute units and their memory path to the
 *    HBM-bound kernels running meanwhile.
 *  - OASIS_COPY_KERNEL enqueues a gather kernel on copy_stream that reads the
 *    pinned pool through its device mapping; it never blocks the caller,
 *    needs no staging buffers and no host CPU time.  It runs on a small
 *    fixed grid: its PCIe reads slow concurrent HBM-bound kernels down, and a
 *    small grid still keeps the link near its memcpy rate.
 *
 * The copies read the plan workspace after the call returns: the next
 * step must use another plan buffer, or wait for `done_event` first.  Calls
 * that overlap on the same slot table race; keep them ordered. */
typedef struct oasis_stage_args {
    const int32_t *sel;     /* [B][H_kv][K_sel] device, ascending, -1 padded */
    const int32_t *n_sel;   /* [B][H_kv] device */
    int32_t K_sel;          /* row stride of sel (normally K_b) */
    const float *scores;    /* [B][H_kv][NB_max] fp32 device (admission order) */
    int32_t K_b;            /* budget in blocks per (r, h) */
    int32_t C;              /* fetch cap in blocks per (r, h) per step, 0..K_b */
    int32_t S;              /* slots per (r, h); S >= K_b (see below) */
    int32_t step;           /* step number, >= 0, increasing */
    int32_t *slot_block;    /* [B][H_kv][S] device, in/out */
    int32_t *slot_stamp;    /* [B][H_kv][S] device, in/out */
    const int32_t *ctx_len; /* [B] device */
    const void *host_pool;  /* [B][H_kv][NB_max][2][bs][D] bf16, pinned host */
    void *ws_pool;          /* [B][H_kv][S][2][bs][D] bf16, device */
    int32_t *tbl_slot;      /* [B][H_kv][K_b] device, written */
    int32_t *tbl_block;     /* [B][H_kv][K_b] device, written */
    int32_t *tbl_n;         /* [B][H_kv] device, written */
    int32_t *plan;          /* device workspace, oasis_stage_plan_bytes() */
    size_t plan_bytes;
    void *host_plan;        /* pinned host, oasis_stage_plan_bytes(); DMA only */
    size_t host_plan_bytes;
    void *stage_host;       /* pinned host staging buffer; DMA only */
    size_t stage_host_bytes;
    void *stage_dev;        /* device staging buffer; DMA only */
    size_t stage_dev_bytes;
    int32_t host_threads;   /* packing threads, DMA only (0 = 8) */
    int32_t copy_mode;      /* OASIS_COPY_DMA or OASIS_COPY_KERNEL */
    void *stream;
    void *copy_stream;
    void *wait_event;
    void *done_event;
    void *plan_event;       /* optional: completes with the plan kernels
                               (bound to the last one) */
    int64_t *stats_accum;   /* optional, device int64[4]: the plan kernels add
                               this step's admits, evictions and deferred
                               admits (oasis_stage_stats) to [0], [1], [2] and
                               1 to [3], with device atomics, so a caller can
                               count any run of steps without reading back
                               each plan; the caller clears it */
} oasis_stage_args;

/* Counts of one staging step, summed over the (request, KV head) pairs.
 * Deferred admits are the predicted blocks that were neither resident nor
 * admitted, |P \ R| - |A| per pair: the blocks the fetch cap C (section 4:
 * at most C blocks per KV head and layer) held back this step.  A later
 * prediction may bring them in; until then attention runs without them. */
typedef struct oasis_stage_stats {
    int64_t admits;        /* blocks admitted, each copied host -> HBM */
    int64_t evictions;     /* resident blocks evicted to make room */
    int64_t deferred;      /* predicted blocks neither resident nor admitted */
    int64_t capped_pairs;  /* pairs with at least one deferred admit */
    int64_t bytes;         /* admits * 2 * bs * D * 2: bytes copied */
} oasis_stage_stats;

/* Appending one decoded token per request (section 4: the full KV lives
 * off-GPU while HBM keeps the per-block key summaries and the working set).
 * For request r with c = ctx_len[r] in [0, NB_max * bs):
 *   - K and V of the token (k_new, v_new [B][H_kv][D] bf16, device) are
 *     written at block c / bs, row c % bs of every KV head of `pool`
 *     ([B][H_kv][NB_max][2][bs][D] bf16, pinned host or device);
 *   - that block's summary in kminmax ([B][H_kv][NB_max][2][D] bf16,
 *     device) becomes the coordinate-wise min / max of its valid keys
 *     including the new one: a block's first token sets both bounds, later
 *     ones replace a bound only when strictly beyond it (the first of equal
 *     values is kept, as oasis_build_summaries does), so appending token by
 *     token equals building afresh;
 *   - when ws_pool ([B][H_kv][S][2][bs][D] bf16, device) is not NULL and the
 *     block is resident (slot_block[r][h][s] == c / bs, slot_block
 *     [B][H_kv][S] int32, device, holding each block at most once), the
 *     token is written into that slot too, so the next attention over the
 *     working set sees it;
 *   - then ctx_len[r] ([B] int32, device, in / out) becomes c + 1.
 * Requests with c outside that range are left unchanged.  Enqueued on
 * `stream`; the caller orders it after the work that reads the previous
 * context and before the work that reads the new one.  Errors: EINVAL for
 * NULL arguments or S < 1 with a working set, EUNSUPPORTED for S > 2048. */
int oasis_append_kv(const oasis_dims *dims, const uint16_t *k_new,
                    const uint16_t *v_new, int32_t *ctx_len,
                    uint16_t *kminmax, void *pool, uint16_t *ws_pool,
                    const int32_t *slot_block, int32_t S, void *stream);

/* Lookahead-agreement analogue.  Section 4 reports how often the top-K set
 * predicted from the draft queries agrees with the true next token's top-K
 * set.  oasis_block_attention_mass gives the true side: for each (request
 * r, KV head h) and block b, the exact attention mass of query q over the
 * request's whole context, summed over the query heads g of h's group,
 *     mass[r][h][b] = sum_g sum_{t in b, t < ctx} exp(l_gt - M_g) / L_g,
 *     l_gt = sm_scale * q[r][g] . k_t,  M_g = max_t l_gt,
 *     L_g = sum_t exp(l_gt - M_g),
 * fp32, 0 for blocks at or past the last block.  oasis_select_topk on it
 * gives the true set.
 *   q        [B][H_q][D] bf16, device (the next token's query)
 *   kv_pool  [B][H_kv][NB_max][2][bs][D] bf16, device or pinned host (every
 *            valid key is read once)
 *   ctx_len  [B] int32, device
 *   mass     [B][H_kv][NB_max] fp32, device, written
 *   ws       device workspace of oasis_block_mass_workspace_bytes(dims) */
size_t oasis_block_mass_workspace_bytes(const oasis_dims *dims);
int oasis_block_attention_mass(const oasis_dims *dims, const uint16_t *q,
                               const uint16_t *kv_pool, const int32_t *ctx_len,
                               float sm_scale, float *mass, void *ws,
                               size_t ws_bytes, void *stream);

/* |A & B| per (request, KV head) of two top-K lists as oasis_select_topk
 * writes them (ascending ids, -1 padded, rows of K entries, counts n_a /
 * n_b [B][H_kv] clamped to [0, K]): overlap [B][H_kv] int32, device.  The
 * agreement of a prediction A with the true set B is overlap / n_b. */
int oasis_topk_overlap(const oasis_dims *dims, const int32_t *sel_a,
                       const int32_t *n_a, const int32_t *sel_b,
                       const int32_t *n_b, int32_t K, int32_t *overlap,
                       void *stream);

/* Bytes of the device plan workspace (and of the pinned host plan buffer):
 * 4 * (B * H_kv * (4 + 2 * max(C, 1)) + 4). */
size_t oasis_stage_plan_bytes(const oasis_dims *dims, int32_t C);

/* Bytes of a staging buffer (host or device) that holds n_blocks blocks. */
size_t oasis_stage_buffer_bytes(const oasis_dims *dims, int32_t n_blocks);

/* One staging step.  Once the plan kernels have run, the plan workspace holds
 * int32 [B * H_kv][4 + 2 * max(C, 1)] followed by 4 int32: per (r, h) the
 * admit count, the evict count, the packed position of its first admit (the
 * running total of admits over the (r, h) before it), the deferred admits,
 * then the admitted (slot, block) pairs in admission order; after the rows
 * the step's total admits, evictions and deferred admits, and the number of
 * pairs with deferred admits.  The host plan (OASIS_COPY_DMA) receives a
 * copy.  `stats` may be NULL; otherwise the call also waits (blocking the
 * calling thread) until the plan kernels have run and fills it in for this
 * step. */
int oasis_stage_blocks(const oasis_dims *dims, const oasis_stage_args *args,
                       oasis_stage_stats *stats);

/* The counts of the step whose plan is in `plan` (a plan workspace for
 * `dims` and fetch cap C, as oasis_stage_plan or oasis_stage_blocks wrote
 * it): waits for `stream` (blocking the calling thread), then reads the
 * plan's totals.  Errors: EINVAL for NULL arguments or C < 0. */
int oasis_stage_read_stats(const oasis_dims *dims, int32_t C,
                           const int32_t *plan, oasis_stage_stats *stats,
                           void *stream);

/* The two halves of oasis_stage_blocks, for callers that overlap staging
 * across layers: oasis_stage_plan enqueues the plan kernels (steps 1-4 and
 * the table) on `stream`, binds `plan_event` if given to the last of them,
 * and never blocks.
 * oasis_stage_copy performs step 5 for the plan in `plan`: it orders the
 * copies after `plan_event` if given, else after everything enqueued on
 * `stream` so far, and otherwise behaves as the copy part of
 * oasis_stage_blocks (it blocks the calling thread with OASIS_COPY_DMA).  It
 * may run on another thread than the plan, as long as it is called after
 * oasis_stage_plan of the same step has returned.  oasis_stage_copy reads only
 * copy_mode, C, S, plan, host_pool, ws_pool, the staging buffers, the streams
 * and the events; oasis_stage_plan reads everything else. */
int oasis_stage_plan(const oasis_dims *dims, const oasis_stage_args *args);
int oasis_stage_copy(const oasis_dims *dims, const oasis_stage_args *args);

/* Sparse GQA decode attention over the listed blocks (sections 4 and 7:
 * attention runs over the HBM working set only).  For query head g of
 * request r, KV head h = g / G, the token set is every valid token of the
 * blocks tbl[r][h][0 .. tbl_n[r][h]); with l_t = sm_scale * q . k_t:
 *     out = sum_t exp(l_t - m) v_t / sum_t exp(l_t - m),  m = max_t l_t
 *     lse = m + ln(sum_t exp(l_t - m))       (natural log)
 * bf16 inputs, fp32 accumulation and online softmax, bf16 (round to nearest
 * even) output.  An empty token set gives out = 0 and lse = -inf.
 *   q          [B][H_q][D] bf16, device
 *   kv_pool    [B][H_kv][P][2][bs][D] bf16, device (P = NB_max for a full
 *              pool read through the selection; P = S for a working set)
 *   tbl_slot   [B][H_kv][T] int32, device: pool slot of each entry
 *   tbl_block  [B][H_kv][T] int32, device: logical block id of each entry
 *              (masks the request's partial last block)
 *   tbl_n      [B][H_kv] int32, device: entries used, clamped to [0, T]
 *              Entries with slot outside [0, P) or block outside [0, n_b(r))
 *              are skipped.
 *   ctx_len    [B] int32, device
 *   out        [B][H_q][D] bf16, device, written
 *   lse        [B][H_q] fp32, device, written; may be NULL
 *   ws         device workspace of oasis_attn_workspace_bytes(dims, T,
 *              n_split) bytes (may be NULL when that is 0)
 *   n_split    number of partitions of each table row (0 = chosen by the
 *              library from the shape and the device's compute-unit count;
 *              otherwise 1..64) */
size_t oasis_attn_workspace_bytes(const oasis_dims *dims, int32_t T,
                                  int32_t n_split);
int32_t oasis_attn_num_splits(const oasis_dims *dims, int32_t T,
                              int32_t n_split);
/* The launch shape the attention entry points use for n_q queries per
 * request: *splits partitions of each table row and *waves waves (4 or 8)
 * per workgroup.  The library aims at two waves per SIMD: one split of
 * four-wave workgroups when there are enough (request, KV head) pairs, else
 * one split of eight-wave workgroups, else more splits as long as each
 * keeps at least four table entries per wave (two past eight query columns,
 * where the workgroups have four waves); an explicit n_split fixes the
 * splits and the waves follow.  OASIS_EINVAL for bad arguments,
 * OASIS_EUNSUPPORTED past 16 query columns (n_q * H_q / H_kv). */
int oasis_attn_launch_shape(const oasis_dims *dims, int32_t n_q, int32_t T,
                            int32_t n_split, int32_t *splits,
                            int32_t *waves);
int oasis_sparse_decode_attn(const oasis_dims *dims, const uint16_t *q,
                             const uint16_t *kv_pool, int32_t P,
                             const int32_t *tbl_slot,
                             const int32_t *tbl_block, const int32_t *tbl_n,
                             int32_t T, const int32_t *ctx_len,
                             float sm_scale, uint16_t *out, float *lse,
                             void *ws, size_t ws_bytes, int32_t n_split,
                             void *stream);

/* oasis_sparse_decode_attn for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same computation with the same arguments except the
 * workspace, whose split-K partials go to a fixed array in device memory
 * that the library holds, oasis_sparse_decode_attn_static_bytes() bytes
 * (8 MiB) on each device it runs on, until the process ends.  The call
 * allocates nothing.  It fails with OASIS_ENOSPACE when the partials
 * (B * H_q * splits * (D + 2) * 4 bytes, 0 without splitting) exceed the
 * array.  Every call on a device uses that device's one array: calls that
 * overlap on one device (on different streams, or from different threads)
 * race and must be ordered by the caller.  Each call writes every partial it
 * reads, so nothing needs clearing between calls. */
size_t oasis_sparse_decode_attn_static_bytes(void);
int oasis_sparse_decode_attn_static(const oasis_dims *dims, const uint16_t *q,
                                    const uint16_t *kv_pool, int32_t P,
                                    const int32_t *tbl_slot,
                                    const int32_t *tbl_block,
                                    const int32_t *tbl_n, int32_t T,
                                    const int32_t *ctx_len, float sm_scale,
                                    uint16_t *out, float *lse,
                                    int32_t n_split, void *stream);

/* Look-ahead attention (section 4: the normal query and the draft queries
 * are computed together over the resident KV).  Exactly
 * oasis_sparse_decode_attn applied to each of n_q query vectors per request
 * over the same blocks, in one pass that reads each K / V block once for all
 * of them:
 *   q    [B][n_q][H_q][D] bf16, device (e.g. the normal query, then the J
 *        draft queries)
 *   out  [B][n_q][H_q][D] bf16, device, written
 *   lse  [B][n_q][H_q] fp32, device, written; may be NULL
 *   ws   oasis_lookahead_attn_workspace_bytes(dims, n_q, T, n_split) bytes
 * The other arguments are those of oasis_sparse_decode_attn; n_q = 1 is that
 * call.  Requires 1 <= n_q and n_q * H_q / H_kv <= 16 (the query rows of a KV
 * group fill the 16 columns of one matrix-core tile); more return
 * OASIS_EUNSUPPORTED. */
size_t oasis_lookahead_attn_workspace_bytes(const oasis_dims *dims, int32_t n_q,
                                            int32_t T, int32_t n_split);
int oasis_lookahead_attn(const oasis_dims *dims, int32_t n_q, const uint16_t *q,
                         const uint16_t *kv_pool, int32_t P,
                         const int32_t *tbl_slot, const int32_t *tbl_block,
                         const int32_t *tbl_n, int32_t T,
                         const int32_t *ctx_len, float sm_scale,
                         uint16_t *out, float *lse, void *ws, size_t ws_bytes,
                         int32_t n_split, void *stream);

/* ---------------------------------------------------------------------------
 * Layer pipeline: the per-layer decode chain, scheduled in native code.
 *
 * Section 4 of the paperlayer summary keeps prediction, selection and copies
 * off the attention's critical path, with several layers and decode steps in
 * flight, and holds a layer's attention back only until its own copies are
 * in.  A pipeline enqueues one layer-step of that schedule per call, every
 * launch, event record and stream wait made from native code: *
 *   main stream (the caller's)   attention of (l, t) over the working set
 *                                staged at (l, t - 1)
 *   compute streams (owned)      scores and top-K of (l, t), staging plan:
 *                                one without staging; two for a staged
 *                                step that the link does not bind (even
 *                                and odd layers alternate, so one layer's
 *                                top-K overlaps the next layer's scores);
 *                                or none: the main stream runs them after
 *                                the layer's attention (compute_streams)
 *   copy streams (owned)         the copies of (l, t); the zero-copy engine
 *                                alternates two by layer so that one
 *                                layer's gather tail overlaps the next
 *                                gather, the DMA engine uses one
 *
 * Per layer the buffers rotate: the attention of step t reads table t % 3,
 * the plan of step t writes table (t + 1) % 3 and uses selection and plan
 * buffer t % 2, and the copies of step t may refill slots that the
 * attention of step t - 1 still reads.  So the top-K of step t waits for the
 * attention of step t - 1, which itself waited for the copies of step t - 2
 * (the last readers of plan buffer t % 2); the plan and the copies of step t
 * follow that top-K, and the attention of step t waits for the copies of
 * step t - 1.  Unstaged pipelines (K/V in HBM) attend at step t over the
 * selection of step t - 1 in the full pool.  With
 * OASIS_COPY_DMA the copy half, which blocks on host packing, runs on one
 * worker thread owned by the pipeline, in submission order; with
 * OASIS_COPY_KERNEL it is enqueued by the calling thread.  Streams are
 * created at default priority; the pipeline allocates no device memory.
 * --------------------------------------------------------------------------- */

/* Caller-owned buffers of one layer; they must outlive the pipeline. */
typedef struct oasis_layer_buffers {
    float *scores;            /* [B][H_kv][NB_max] fp32, device */
    int32_t *sel[2];          /* [B][H_kv][K_b] int32, device */
    int32_t *n_sel[2];        /* [B][H_kv] int32, device */
    void *attn_ws;            /* oasis_lookahead_attn_workspace_bytes(dims,
                                 n_q, K_b, n_split) bytes */
    size_t attn_ws_bytes;
    /* staged pipelines only (ignored otherwise) */
    uint16_t *ws_pool;        /* [B][H_kv][K_b + C][2][bs][D] bf16, device */
    int32_t *slot_block;      /* [B][H_kv][K_b + C] int32, device, all -1 */
    int32_t *slot_stamp;      /* [B][H_kv][K_b + C] int32, device, all -1 */
    int32_t *tbl_slot[3];     /* [B][H_kv][K_b] int32, device */
    int32_t *tbl_block[3];    /* [B][H_kv][K_b] int32, device */
    int32_t *tbl_n[3];        /* [B][H_kv] int32, device */
    int32_t *plan[2];         /* device, plan_bytes each */
    size_t plan_bytes;        /* >= oasis_stage_plan_bytes(dims, K_b) */
    void *host_plan;          /* pinned host, plan_bytes; DMA only */
    void *stage_host[2];      /* pinned host staging buffers; DMA only */
    void *stage_dev;          /* device staging buffer; DMA only */
    size_t stage_bytes;       /* bytes of each staging buffer; DMA only */
} oasis_layer_buffers;

typedef struct oasis_pipeline_desc {
    int32_t n_layers;         /* 1 .. 1024 */
    int32_t K_b;              /* budget in blocks per (r, h) */
    int32_t C;                /* fetch cap in blocks per (r, h) per step
                                 (staged; step 0 fills uncapped) */
    int32_t J;                /* lookahead queries per request */
    int32_t n_q;              /* attention queries per request: 1 = decode
                                 attention; 1 + J = look-ahead attention of
                                 the normal and the draft queries
                                 (oasis_lookahead_attn; n_q * H_q / H_kv
                                 <= 16) */
    int32_t staged;           /* 1: pool is pinned host memory staged into
                                 per-layer working sets; 0: pool in HBM */
    int32_t copy_mode;        /* OASIS_COPY_KERNEL, OASIS_COPY_DMA or
                                 OASIS_COPY_MIXED (the DMA engine for even
                                 layers, on one copy stream and the worker
                                 thread, and the gather kernel for odd
                                 layers, on a second copy stream: the link
                                 carries both at once) */
    int32_t host_threads;     /* DMA packing threads (0 = 8) */
    int32_t n_split;          /* attention split count (0 = automatic) */
    float sm_scale;           /* attention scale, e.g. 1 / sqrt(D) */
    const uint16_t *pool;     /* [B][H_kv][NB_max][2][bs][D] bf16 */
    const uint16_t *kminmax;  /* [B][H_kv][NB_max][2][D] summaries, device */
    const int32_t *ctx_len;   /* [B] int32, device */
    void *main_stream;        /* attention stream (hipStream_t; NULL = null
                                 stream) */
    const oasis_layer_buffers *layers;  /* n_layers entries, copied */
    int32_t compute_streams;  /* streams for scores, top-K and the plan: 1,
                                 or 2 (even and odd layers alternate, so one
                                 layer's top-K overlaps the next layer's
                                 scores); -1: none, the chain runs on the
                                 main stream after each layer's attention
                                 (the kernels that read HBM never overlap
                                 each other, only the copies); 0 =
                                 automatic: 1 without staging (a second
                                 stream only adds a second score kernel
                                 beside the attention on HBM); staged, -1
                                 for a step that is bound by the link (C
                                 blocks of 8 KiB at 57 GB/s take over
                                 twice as long as the pair's K_b blocks
                                 and NB_max summaries of 512 B at 6 TB/s)
                                 and has at least as many (request, KV
                                 head) pairs as the device has compute
                                 units; else 2 (top-K and the plan run one
                                 workgroup per pair and, with few pairs,
                                 leave compute units idle).
                                 Copy streams: OASIS_COPY_KERNEL with at
                                 most one compute stream, two (even and odd
                                 layers), so one gather's tail overlaps the
                                 next one's start; OASIS_COPY_MIXED, two
                                 (the DMA layers and the gather layers);
                                 otherwise one.  That keeps to four streams,
                                 the hardware queues of a process, except
                                 two compute streams with the mixed engine
                                 (five). */
    int64_t *stage_stats;     /* optional, device int64[4]: every staging
                                 step of every layer adds its admits,
                                 evictions, deferred admits and 1 (see
                                 oasis_stage_args.stats_accum); the caller
                                 clears it */
    int32_t issue_threads;    /* pipelines whose chain has compute streams
                                 of its own: with issue threads one worker
                                 thread enqueues each layer-step's scores,
                                 top-K and plan, another (staged) its
                                 copies, both in submission order, and the
                                 calling thread only the attention.  The
                                 chain's cross-stream waits (the top-K's on
                                 the attention of step t - 1, a gather's on
                                 its plan) and, without staging, the
                                 attention's on the selection of step t - 1
                                 are then made on the host by the thread
                                 that enqueues the waiting work, once what
                                 it waits for is enqueued, so those queues
                                 carry no barrier packets; without staging
                                 THE CALLING THREAD MAY BLOCK in
                                 oasis_pipeline_layer_step until the
                                 selection of (layer, step - 1) is done.
                                 0 (automatic) or 1 = on; -1 = off, the
                                 calling thread enqueues everything, with
                                 stream waits.  A chain on
                                 the main stream (compute_streams = -1)
                                 always uses the calling thread
                                 (oasis_pipeline_issue_threads tells). */
} oasis_pipeline_desc;

typedef struct oasis_pipeline oasis_pipeline;

/* Checks the description, creates the compute and copy streams, the events
 * and the worker threads (DMA copies; issue threads); *out receives the
 * handle. */
int oasis_pipeline_create(const oasis_dims *dims,
                          const oasis_pipeline_desc *desc,
                          oasis_pipeline **out);

/* Enqueues layer `layer`'s work of decode step `step`: the attention of
 * step t (queries q_attn [B][n_q][H_q][D] bf16, device; output out
 * [B][n_q][H_q][D] bf16 and lse [B][n_q][H_q] fp32 (may be NULL), device;
 * skipped at t = 0 where q_attn and out may be NULL) and the prediction and
 * staging for step t + 1 from q_look [B][J][H_q][D] bf16, device.  Steps of one layer must be
 * issued in order 0, 1, 2, ... (OASIS_EINVAL otherwise); layers may
 * interleave freely.  Inputs must stay valid until the work completes.
 * It blocks the caller while a worker thread has not yet enqueued the
 * copies (DMA engine; issue threads) or the selection (issue threads) of
 * (layer, step - 1), and with issue threads and no staging until that
 * selection has run on the GPU.  An error of a worker thread is returned by
 * the next call. */
int oasis_pipeline_layer_step(oasis_pipeline *p, int32_t layer, int32_t step,
                              const uint16_t *q_look, const uint16_t *q_attn,
                              uint16_t *out, float *lse);

/* Waits until the worker threads (DMA copies, issue threads) have enqueued
 * everything submitted so far (no device synchronisation): after it, work
 * the caller enqueues on a pipeline stream follows every earlier
 * layer-step's work on that stream. */
int oasis_pipeline_drain(oasis_pipeline *p);

/* The pipeline's streams: which = 0 main, 1 compute (of even layers with
 * two compute streams, else of every layer), 2 and 3 the copy streams (of
 * even and odd layers with two, else 2 for every layer), 4 the compute
 * stream of odd layers (NULL where not used). */
int oasis_pipeline_stream(oasis_pipeline *p, int32_t which, void **stream);

/* *on = 1 if the pipeline's chain and copies are enqueued by issue threads,
 * else 0 (issue_threads = -1, or the chain on the main stream). */
int oasis_pipeline_issue_threads(oasis_pipeline *p, int32_t *on);

/* Event timing of the steps: capacity > 0 (re)arms timing of up to
 * `capacity` launches of each kind whose bit is set in `kinds` and clears
 * the totals; capacity 0 or kinds 0 disables it.  Of each kind, one launch
 * in every `every` (>= 1) is timed, the first launch after arming
 * included.  Kinds: 0 attention (main stream), 1 scores, 2 top-K, 3 staging
 * plan (compute stream); each interval starts once the stream's earlier
 * work and waits are done (a start event recorded on the stream, which
 * holds it ~3 us) and ends with the launch's last kernel (a stop event
 * bound to that kernel, which costs the queue nothing).  Re-arming first
 * waits for everything the pipeline has enqueued to finish.  timing_read
 * synchronises on the events and returns their total milliseconds and
 * count. */
int oasis_pipeline_timing(oasis_pipeline *p, int32_t capacity,
                          uint32_t kinds, int32_t every);
int oasis_pipeline_timing_read(oasis_pipeline *p, int32_t kind,
                               double *total_ms, int32_t *count);

/* The same timed launches one by one: ms[i] = milliseconds of the i-th timed
 * launch of `kind` in launch order, for i < min(*count, capacity) (ms
 * caller-owned host memory, may be NULL when capacity is 0); *count
 * receives the number of timed launches.  Synchronises like timing_read. */
int oasis_pipeline_timing_values(oasis_pipeline *p, int32_t kind, float *ms,
                                 int32_t capacity, int32_t *count);

/* Host seconds spent in the copy half of staging (plan read-back and packing
 * with OASIS_COPY_DMA, the enqueue with OASIS_COPY_KERNEL) since timing was
 * last armed, and the number of calls. */
int oasis_pipeline_copy_host_seconds(oasis_pipeline *p, double *seconds,
                                     int32_t *calls);

/* Drains, synchronises the pipeline's streams and the main stream, and
 * frees the streams, events and worker.  NULL is accepted. */
int oasis_pipeline_destroy(oasis_pipeline *p);

#ifdef __cplusplus
}
#endif

#endif /* OASIS_H */
