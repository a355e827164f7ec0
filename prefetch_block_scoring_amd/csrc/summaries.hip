// Per-block coordinate-wise min / max key summaries.
//
// OasisKV (arXiv 2608.08097), paperlayer summary, section 4: the prototype
// keeps two vectors per block, the coordinate-wise minimum and maximum of the
// block's keys, in HBM in place of the keys themselves.  Built once when a
// block's keys are final; not part of a decode step.
//
// One wavefront per block: lane l owns dims 2l and 2l+1 and walks the block's
// valid tokens; each step of the walk is one coalesced 256-byte row read.
#include "oasis_internal.h"

namespace oasis {
namespace {

constexpr int kBlocksPerWg = 4;

__global__ __launch_bounds__(256) void build_summaries_kernel(
    const uint32_t *__restrict__ kv, const int32_t *__restrict__ ctx_len,
    uint32_t *__restrict__ kminmax, int H_kv, int NB_max) {
    const int rh = blockIdx.x;
    const int r = rh / H_kv;
    const int b = blockIdx.y * kBlocksPerWg + threadIdx.x / 64;
    const int ctx = ctx_len[r];
    const int nb = n_blocks_of(ctx, NB_max);
    if (b >= nb) return;
    int valid = ctx - b * kBs;
    valid = valid < kBs ? valid : kBs;
    const int dp = threadIdx.x % 64;  // dim pair
    // K of block b: kBs rows of kD bf16 = 64 uint32 per row
    const uint32_t *K = kv + ((size_t)rh * NB_max + b) * (kBlockElems / 2);
    uint32_t x = K[dp];
    uint32_t lo0 = x & 0xffffu, hi0 = lo0, lo1 = x >> 16, hi1 = lo1;
    float flo0 = bf16_lo(x), fhi0 = flo0, flo1 = bf16_hi(x), fhi1 = flo1;
    for (int t = 1; t < valid; t++) {
        x = K[t * (kD / 2) + dp];
        const float a = bf16_lo(x), c = bf16_hi(x);
        if (a < flo0) { flo0 = a; lo0 = x & 0xffffu; }
        if (a > fhi0) { fhi0 = a; hi0 = x & 0xffffu; }
        if (c < flo1) { flo1 = c; lo1 = x >> 16; }
        if (c > fhi1) { fhi1 = c; hi1 = x >> 16; }
    }
    uint32_t *out = kminmax + ((size_t)rh * NB_max + b) * kD;  // [2][kD] bf16 = kD uint32
    out[dp] = lo0 | (lo1 << 16);
    out[kD / 2 + dp] = hi0 | (hi1 << 16);
}

}  // namespace

hipError_t launch_build_summaries(const oasis_dims &d, const uint16_t *kv,
                                  const int32_t *ctx_len, uint16_t *kminmax,
                                  hipStream_t s) {
    dim3 grid((unsigned)(d.B * d.H_kv), (unsigned)((d.NB_max + kBlocksPerWg - 1) / kBlocksPerWg));
    hipLaunchKernelGGL(build_summaries_kernel, grid, dim3(256), 0, s,
                       reinterpret_cast<const uint32_t *>(kv), ctx_len,
                       reinterpret_cast<uint32_t *>(kminmax), d.H_kv, d.NB_max);
    return hipGetLastError();
}

}  // namespace oasis
