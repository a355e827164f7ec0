// Internal declarations shared by the liboasis sources (not installed).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>
#include <string>

#include "oasis.h"

namespace oasis {

// ---------------------------------------------------------------- errors

void set_error(const std::string &msg);
void clear_error();

// Returns OASIS_EHIP and records `what` with the runtime's message when `e`
// is not hipSuccess.
int hip_check(hipError_t e, const char *what);

// Shape checks shared by every entry point (sets the error message).
int check_dims(const oasis_dims *d);

#define OASIS_HIP(call)                                   \
    do {                                                  \
        int _rc = ::oasis::hip_check((call), #call);      \
        if (_rc != OASIS_OK) return _rc;                  \
    } while (0)

// ---------------------------------------------------------------- shapes

constexpr int kD = 128;        // head dimension the kernels are written for
constexpr int kBs = 16;        // tokens per block
constexpr int kMaxG = 16;      // query heads per KV head (MFMA N tile)
constexpr int kMaxNB = 16384;  // blocks per (request, KV head)
constexpr int kBlockElems = 2 * kBs * kD;          // bf16 elements per K+V block
constexpr size_t kBlockBytes = kBlockElems * 2;    // 8 KiB

// Number of compute units of the current device (cached per device).
int device_cu_count();

// Resolve a pointer that may be pinned host memory into an address kernels
// can dereference.  Fails (OASIS_EINVAL) for pageable host memory.
int device_view(const void *p, const void **out, const char *name);

// ---------------------------------------------------------------- launchers
// Each launcher assumes its arguments were validated by the C entry point.

// `done` (optional): an event bound to a launcher's last kernel dispatch
// (hipExtLaunchKernelGGL stop event), completing as that kernel ends, with
// its timestamp.  A bound event costs the queue nothing, where a
// hipEventRecord after the kernel adds a marker packet that holds the queue
// ~3 us on MI355X (ROCm 7.2; 24.1 against 21.0 us per 20 us kernel back to
// back).  (Binding a start event as well would cost the enqueuing thread
// 9-19 us per launch.)  A launcher that launches nothing records `done` on
// the stream instead (record_done), so it still completes in stream order.
hipError_t record_done(hipEvent_t done, hipStream_t s);

// The entry points of the same names with `done` bound to their last kernel
// (the layer pipeline's completion and timing events).
int score_blocks(const oasis_dims *dims, const uint16_t *q_look, int32_t J, const uint16_t *kminmax,
                 const int32_t *ctx_len, float *scores, void *stream, hipEvent_t done);
int select_topk(const oasis_dims *dims, const float *scores, const int32_t *ctx_len, int32_t K_b, int32_t *sel,
                int32_t *n_sel, void *stream, hipEvent_t done);
int lookahead_attn(const oasis_dims *dims, int32_t n_q, const uint16_t *q, const uint16_t *kv_pool, int32_t P,
                   const int32_t *tbl_slot, const int32_t *tbl_block, const int32_t *tbl_n, int32_t T,
                   const int32_t *ctx_len, float sm_scale, uint16_t *out, float *lse, void *ws, size_t ws_bytes,
                   int32_t n_split, void *stream, hipEvent_t done);

hipError_t launch_build_summaries(const oasis_dims &d, const uint16_t *kv,
                                  const int32_t *ctx_len, uint16_t *kminmax,
                                  hipStream_t s);

hipError_t launch_score(const oasis_dims &d, const uint16_t *q_look, int J,
                        const uint16_t *kminmax, const int32_t *ctx_len,
                        float *scores, hipStream_t s, hipEvent_t done = nullptr);

hipError_t launch_topk(const oasis_dims &d, const float *scores,
                       const int32_t *ctx_len, int K_b, int32_t *sel,
                       int32_t *n_sel, hipStream_t s, hipEvent_t done = nullptr);

hipError_t launch_stage_plan(const oasis_dims &d, const oasis_stage_args &a,
                             hipStream_t s);

hipError_t launch_stage_gather(const oasis_dims &d, const oasis_stage_args &a,
                               const void *host_pool_dev, hipStream_t s,
                               hipEvent_t done = nullptr);

hipError_t launch_append(const oasis_dims &d, const uint16_t *k_new,
                         const uint16_t *v_new, int32_t *ctx_len,
                         uint16_t *kminmax, void *pool_dev, uint16_t *ws_pool,
                         const int32_t *slot_block, int S, hipStream_t s);

size_t block_mass_ws_bytes(const oasis_dims &d);
hipError_t launch_block_mass(const oasis_dims &d, const uint16_t *q,
                             const void *kv_dev, const int32_t *ctx_len,
                             float sm_scale, float *mass, void *ws,
                             hipStream_t s);
hipError_t launch_topk_overlap(int pairs, const int32_t *a, const int32_t *na,
                               const int32_t *b, const int32_t *nb, int K,
                               int32_t *out, hipStream_t s);

// split count of an attention launch with n_q queries per request
int attn_splits(const oasis_dims &d, int n_q, int T, int n_split);
// waves per workgroup of an attention launch with `splits` splits
int attn_waves(const oasis_dims &d, int n_q, int T, int splits);
// split-K workspace for n_q queries per request
size_t attn_ws_bytes(const oasis_dims &d, int n_q, int T, int n_split);

// The fixed split-K scratch of oasis_sparse_decode_attn_static: its size, and
// its address on the current device (looked up once per device).
constexpr int kMaxDevices = 64;
size_t attn_static_scratch_bytes();
hipError_t attn_static_scratch(void **ptr);

// n_q queries per request, q / out [B][n_q][H_q][D]; n_q * G <= kMaxG
hipError_t launch_attn(const oasis_dims &d, int n_q, const uint16_t *q,
                       const uint16_t *kv_pool, int P, const int32_t *tbl_slot,
                       const int32_t *tbl_block, const int32_t *tbl_n, int T,
                       const int32_t *ctx_len, float sm_scale, uint16_t *out,
                       float *lse, float *ws, int n_split, hipStream_t s,
                       hipEvent_t done = nullptr);

// Plan workspace: per (r, h) a row of int32
//   [0] admits, [1] evictions, [2] packed position of the first admit (the
//   exclusive prefix of admits over (r, h)), [3] deferred admits (predicted
//   blocks neither resident nor admitted), then one (slot, block) pair per
//   admit;
// after the rows, kPlanTail int32: [0] total admits, [1] total evictions,
// [2] total deferred admits, [3] pairs with deferred admits.
constexpr int kPlanHead = 4;
constexpr int kPlanTail = 4;
__host__ __device__ inline int plan_row(int C) { return kPlanHead + 2 * (C > 0 ? C : 1); }
inline size_t plan_ints(int pairs, int C) { return (size_t)pairs * plan_row(C) + kPlanTail; }

hipError_t launch_stage_prefix(const oasis_dims &d, const oasis_stage_args &a, hipStream_t s,
                               hipEvent_t done = nullptr);

// Copy the admitted blocks of packed positions [lo, hi) from the device
// staging buffer (position lo at its start) into their working-set slots.
hipError_t launch_stage_scatter(const oasis_dims &d, const oasis_stage_args &a, int lo, int hi,
                                hipStream_t s);

// Host side of the DMA copy engine: read back the plan, pack the admitted
// blocks on worker threads, one H2D copy per round, scatter on the device.
int stage_dma(const oasis_dims &d, const oasis_stage_args &a, hipEvent_t plan_ready, hipStream_t cs);

// per-thread ring of ordering events on the current device
int ring_event(hipEvent_t *ev);

// Make stream s wait for event e unless e has already completed (or was never
// recorded).  A wait on a pending event costs the calling thread 8-24 us, and
// its barrier packet delays the stream even when the event is done by then.
hipError_t stream_wait(hipStream_t s, hipEvent_t e);

// Map every page of a fresh pinned host allocation into the process (one
// write per page, on the worker threads) so that later CPU accesses, such as
// the DMA engine's packing, do not take a page fault per new page.
void prefault_host(void *p, size_t bytes);

}  // namespace oasis

// ---------------------------------------------------------------- device helpers

namespace oasis {

__device__ __forceinline__ float bf16_lo(uint32_t pair) { return __uint_as_float(pair << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t pair) { return __uint_as_float(pair & 0xffff0000u); }

// Round to nearest even; NaN stays NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// Order-preserving key: a ranks before b (higher score) iff key(a) > key(b).
// NaN maps below -inf; -0 maps to +0.
__device__ __forceinline__ uint32_t rank_key(float s) {
    uint32_t u = __float_as_uint(s);
    if ((u & 0x7fffffffu) > 0x7f800000u) return 0u;
    if (u == 0x80000000u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ int n_blocks_of(int ctx, int nb_max) {
    int nb = ctx <= 0 ? 0 : (ctx + kBs - 1) / kBs;
    return nb < nb_max ? nb : nb_max;
}

}  // namespace oasis
