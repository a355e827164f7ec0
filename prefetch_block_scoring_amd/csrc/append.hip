// Appending one decoded token per request: pool, block summary, resident slot.
//
// OasisKV (arXiv 2608.08097), paperlayer summary, section 4: the full KV
// lives off-GPU while HBM keeps the compressed per-block key summaries and
// the sparse working set.  Each decode step adds one token per request: its
// K and V go to the pool at the context position, its block's min / max
// summary takes the new key in, and, when that block is resident in the
// working set, its slot gets the token too, so that the next attention over
// the working set sees the whole block.
//
// Mapping: one workgroup per request (the context is advanced once every
// head is written); wave w takes KV heads w, w + 4, ...; lane i moves dims
// 2i and 2i + 1 (one 32-bit word of K and one of V).  The summary keeps the
// first of equal extreme values, like the builder, so appending token by
// token gives the same bits as building the summary afresh.
#include "oasis_internal.h"

namespace oasis {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kWords = kD / 2;  // 32-bit words per key / value row

__device__ __forceinline__ uint32_t pick_half(uint32_t cur, uint32_t x, bool lower, int half) {
    const uint32_t sh = 16u * (uint32_t)half;
    const float fc = __uint_as_float(((cur >> sh) & 0xffffu) << 16);
    const float fx = __uint_as_float(((x >> sh) & 0xffffu) << 16);
    const bool take = lower ? (fx < fc) : (fx > fc);
    return take ? ((cur & ~(0xffffu << sh)) | (x & (0xffffu << sh))) : cur;
}

__global__ __launch_bounds__(kThreads) void append_kernel(
    const uint32_t *__restrict__ k_new, const uint32_t *__restrict__ v_new, int32_t *__restrict__ ctx_len,
    uint32_t *__restrict__ kminmax, uint32_t *__restrict__ pool, uint32_t *__restrict__ ws,
    const int32_t *__restrict__ slot_block, int S, int H_kv, int NB_max) {
    const int r = blockIdx.x;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int c = ctx_len[r];
    const bool ok = c >= 0 && (long)c < (long)NB_max * kBs;
    if (ok) {
        const int b = c / kBs, row = c - b * kBs;
        for (int h = wave; h < H_kv; h += kWaves) {
            const size_t rh = (size_t)r * H_kv + h;
            const uint32_t k = k_new[rh * kWords + lane];
            const uint32_t v = v_new[rh * kWords + lane];
            uint32_t *blk = pool + (rh * NB_max + b) * (2 * kBs * kWords);
            blk[row * kWords + lane] = k;
            blk[(kBs + row) * kWords + lane] = v;
            uint32_t *sm = kminmax + (rh * NB_max + b) * (2 * kWords);
            uint32_t lo = k, hi = k;
            if (row > 0) {
                lo = pick_half(pick_half(sm[lane], k, true, 0), k, true, 1);
                hi = pick_half(pick_half(sm[kWords + lane], k, false, 0), k, false, 1);
            }
            sm[lane] = lo;
            sm[kWords + lane] = hi;
            if (ws) {
                // the slot that holds block b, if any (slot tables hold a
                // block at most once)
                int slot = -1;
                for (int s = lane; s < S; s += 64)
                    if (slot_block[rh * S + s] == b) slot = s;
#pragma unroll
                for (int o = 32; o > 0; o >>= 1) slot = max(slot, __shfl_xor(slot, o, 64));
                if (slot >= 0) {
                    uint32_t *dst = ws + (rh * S + slot) * (2 * kBs * kWords);
                    dst[row * kWords + lane] = k;
                    dst[(kBs + row) * kWords + lane] = v;
                }
            }
        }
    }
    __syncthreads();  // every thread has read ctx_len[r]
    if (ok && threadIdx.x == 0) ctx_len[r] = c + 1;
}

}  // namespace

hipError_t launch_append(const oasis_dims &d, const uint16_t *k_new, const uint16_t *v_new, int32_t *ctx_len,
                         uint16_t *kminmax, void *pool_dev, uint16_t *ws_pool, const int32_t *slot_block, int S,
                         hipStream_t s) {
    hipLaunchKernelGGL(append_kernel, dim3((unsigned)d.B), dim3(kThreads), 0, s,
                       reinterpret_cast<const uint32_t *>(k_new), reinterpret_cast<const uint32_t *>(v_new),
                       ctx_len, reinterpret_cast<uint32_t *>(kminmax), static_cast<uint32_t *>(pool_dev),
                       reinterpret_cast<uint32_t *>(ws_pool), slot_block, S, d.H_kv, d.NB_max);
    return hipGetLastError();
}

}  // namespace oasis
