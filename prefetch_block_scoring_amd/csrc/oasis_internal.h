// Internal declarations shared by the liboasis sources (not installed).
#pragma once

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

hipError_t launch_build_summaries(const oasis_dims &d, const uint16_t *kv,
                                  const int32_t *ctx_len, uint16_t *kminmax,
                                  hipStream_t s);

hipError_t launch_score(const oasis_dims &d, const uint16_t *q_look, int J,
                        const uint16_t *kminmax, const int32_t *ctx_len,
                        float *scores, hipStream_t s);

hipError_t launch_topk(const oasis_dims &d, const float *scores,
                       const int32_t *ctx_len, int K_b, int32_t *sel,
                       int32_t *n_sel, hipStream_t s);

hipError_t launch_stage_plan(const oasis_dims &d, const oasis_stage_args &a,
                             hipStream_t s);

hipError_t launch_stage_gather(const oasis_dims &d, const oasis_stage_args &a,
                               const void *host_pool_dev, hipStream_t s);

int attn_splits(const oasis_dims &d, int T, int n_split);
size_t attn_ws_bytes(const oasis_dims &d, int T, int n_split);

hipError_t launch_attn(const oasis_dims &d, const uint16_t *q,
                       const uint16_t *kv_pool, int P, const int32_t *tbl_slot,
                       const int32_t *tbl_block, const int32_t *tbl_n, int T,
                       const int32_t *ctx_len, float sm_scale, uint16_t *out,
                       float *lse, float *ws, int n_split, hipStream_t s);

// plan workspace row length in int32 per (r, h)
__host__ __device__ inline int plan_row(int C) { return 2 + 2 * (C > 0 ? C : 1); }

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
