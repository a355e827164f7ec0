// Lookahead block scoring over the min / max key summaries.
//
// OasisKV (arXiv 2608.08097), paperlayer summary, section 4: the draft
// queries scan the compressed per-block key summaries to rank the blocks the
// next step will need.  The score of block b for KV head h is the largest
// value q . k can reach over the block's bounding box [kmin, kmax], summed
// over the drafts j and the query heads g of h's group:
//     s = sum_{j,g,d} max(q[j,g,d] kmax[d], q[j,g,d] kmin[d]).
// Because max(q a, q c) with a >= c is q a for q > 0 and q c for q < 0, the
// sum splits by sign:  s = sum_d Qp[d] kmax[d] + Qm[d] kmin[d]  with
// Qp = sum_{j,g} max(q, 0) and Qm = sum_{j,g} min(q, 0).  That turns J * G
// query vectors into two per (request, KV head), so the scan reads each
// summary byte once and does 0.5 FMA per byte: HBM-bound.
//
// Arithmetic: Qp / Qm are summed in fp64 (exact for bf16 inputs of ordinary
// range), the 2 * D products and their sum in fp64, rounded once to fp32.
//
// Mapping: a workgroup owns one (request, KV head) and a chunk of 256 blocks.
// Eight lanes share a block (512 bytes of summary); lane i of the eight holds
// dims [8i, 8i + 8) and [64 + 8i, 64 + 8i + 8) of kmin and kmax, so each of the
// four 16-byte loads per lane is one fully used 128-byte line per eight lanes.
// The eight partial sums meet through three xor shuffles.
#include "oasis_internal.h"

namespace oasis {
namespace {

constexpr int kChunk = 256;        // blocks per workgroup
constexpr int kLanesPerBlock = 8;  // lanes sharing one block
constexpr int kBlocksPerIter = 256 / kLanesPerBlock;

__device__ __forceinline__ double bf16_d(uint32_t bits16) {
    return (double)__uint_as_float(bits16 << 16);
}

__global__ __launch_bounds__(256) void score_kernel(
    const uint16_t *__restrict__ q_look, int J, int H_q, int H_kv,
    const uint4 *__restrict__ kminmax, const int32_t *__restrict__ ctx_len,
    float *__restrict__ scores, int NB_max) {
    __shared__ double Qsh[2][kD];  // [0] = Qm (pairs with kmin), [1] = Qp (pairs with kmax)
    const int rh = blockIdx.x;
    const int r = rh / H_kv;
    const int h = rh - r * H_kv;
    const int G = H_q / H_kv;
    const int tid = threadIdx.x;
    if (tid < kD) {
        double qp = 0.0, qm = 0.0;
        for (int j = 0; j < J; j++) {
            const uint16_t *qrow = q_look + (((size_t)r * J + j) * H_q + (size_t)h * G) * kD + tid;
            for (int gi = 0; gi < G; gi++) {
                const double v = bf16_d(qrow[(size_t)gi * kD]);
                if (v > 0.0) qp += v; else qm += v;
            }
        }
        Qsh[0][tid] = qm;
        Qsh[1][tid] = qp;
    }
    __syncthreads();

    const int li = tid % kLanesPerBlock;
    double qm[16], qp[16];
#pragma unroll
    for (int e = 0; e < 8; e++) {
        qm[e] = Qsh[0][li * 8 + e];
        qm[8 + e] = Qsh[0][64 + li * 8 + e];
        qp[e] = Qsh[1][li * 8 + e];
        qp[8 + e] = Qsh[1][64 + li * 8 + e];
    }

    const int nb = n_blocks_of(ctx_len[r], NB_max);
    const int b_end = min(NB_max, (int)(blockIdx.y + 1) * kChunk);
    float *out = scores + (size_t)rh * NB_max;
    // summary of block b: [2][kD] bf16 = 32 uint4; kmin at 0..15, kmax at 16..31
    const uint4 *base = kminmax + (size_t)rh * NB_max * 32;
    for (int b0 = blockIdx.y * kChunk; b0 < b_end; b0 += kBlocksPerIter) {
        const int b = b0 + tid / kLanesPerBlock;
        if (b >= b_end) continue;            // whole group of eight skips together
        if (b >= nb) {
            if (li == 0) out[b] = -INFINITY;
            continue;
        }
        const uint4 *sb = base + (size_t)b * 32;
        const uint4 mn0 = sb[li], mn1 = sb[8 + li], mx0 = sb[16 + li], mx1 = sb[24 + li];
        const uint32_t wmn[8] = {mn0.x, mn0.y, mn0.z, mn0.w, mn1.x, mn1.y, mn1.z, mn1.w};
        const uint32_t wmx[8] = {mx0.x, mx0.y, mx0.z, mx0.w, mx1.x, mx1.y, mx1.z, mx1.w};
        double acc = 0.0;
#pragma unroll
        for (int w = 0; w < 8; w++) {
            const int e = (w < 4) ? 2 * w : 8 + 2 * (w - 4);
            acc = fma(qm[e], bf16_d(wmn[w] & 0xffffu), acc);
            acc = fma(qm[e + 1], bf16_d(wmn[w] >> 16), acc);
            acc = fma(qp[e], bf16_d(wmx[w] & 0xffffu), acc);
            acc = fma(qp[e + 1], bf16_d(wmx[w] >> 16), acc);
        }
        acc += __shfl_xor(acc, 1, kLanesPerBlock);
        acc += __shfl_xor(acc, 2, kLanesPerBlock);
        acc += __shfl_xor(acc, 4, kLanesPerBlock);
        if (li == 0) out[b] = (float)acc;
    }
}

}  // namespace

hipError_t launch_score(const oasis_dims &d, const uint16_t *q_look, int J,
                        const uint16_t *kminmax, const int32_t *ctx_len,
                        float *scores, hipStream_t s) {
    dim3 grid((unsigned)(d.B * d.H_kv), (unsigned)((d.NB_max + kChunk - 1) / kChunk));
    hipLaunchKernelGGL(score_kernel, grid, dim3(256), 0, s, q_look, J, d.H_q, d.H_kv,
                       reinterpret_cast<const uint4 *>(kminmax), ctx_len, scores, d.NB_max);
    return hipGetLastError();
}

}  // namespace oasis
