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
// Mapping: the grid is persistent (compute units x resident workgroups).  The
// work items are the (request, KV head, 128-block chunk) triples whose chunk
// holds at least one of the request's blocks; they are split into equal
// contiguous ranges, one per workgroup, so that ragged contexts balance and
// Qp / Qm are rebuilt only when a range crosses into the next (request, KV
// head).  Each workgroup counts the items itself from the context lengths.
// The chunks past a request's last block only get -inf, in a second, strided
// loop.  Eight lanes share a block (512 bytes of
// summary); lane i of the eight holds dims [8i, 8i + 8) and [64 + 8i, 72 + 8i)
// of kmin and kmax, so each 16-byte load fills whole 128-byte lines per eight
// lanes.  Four 32-block groups are loaded before any is used (16 KiB in flight
// per wave).  The eight partial sums meet through three DPP steps.
#include "oasis_internal.h"

namespace oasis {
namespace {

constexpr int kThreads = 256;
constexpr int kLanesPerBlock = 8;                       // lanes sharing one block
constexpr int kBlocksPerGroup = kThreads / kLanesPerBlock;  // 32
constexpr int kUnroll = 4;
constexpr int kItemBlocks = kBlocksPerGroup * kUnroll;  // 128 blocks per item

__device__ __forceinline__ double bf16_d(uint32_t bits16) {
    return (double)__uint_as_float(bits16 << 16);
}

template <int CTRL>
__device__ __forceinline__ double dpp_d(double x) {
    const long long v = __double_as_longlong(x);
    const int lo = __builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, true);
    const int hi = __builtin_amdgcn_update_dpp(0, (int)(v >> 32), CTRL, 0xF, 0xF, true);
    return __longlong_as_double(((long long)hi << 32) | (unsigned)lo);
}

// Sum over the eight lanes of an aligned octet; every lane gets the total.
__device__ __forceinline__ double octet_sum(double x) {
    x += dpp_d<0xB1>(x);   // quad_perm [1,0,3,2]
    x += dpp_d<0x4E>(x);   // quad_perm [2,3,0,1]
    x += dpp_d<0x141>(x);  // row_half_mirror: lane i <- lane 7 - i within 8
    return x;
}

// chunks of request r that hold at least one of its blocks
__device__ __forceinline__ int valid_chunks(const int32_t *ctx_len, int r, int NB_max) {
    return (n_blocks_of(ctx_len[r], NB_max) + kItemBlocks - 1) / kItemBlocks;
}

__global__ __launch_bounds__(kThreads, 3) void score_kernel(
    const uint16_t *__restrict__ q_look, int J, int H_q, int H_kv,
    const uint4 *__restrict__ kminmax, const int32_t *__restrict__ ctx_len,
    float *__restrict__ scores, int NB_max, int B) {
    __shared__ double Qsh[2][kD];  // [0] = Qm (pairs with kmin), [1] = Qp (pairs with kmax)
    const int G = H_q / H_kv;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int li = tid % kLanesPerBlock;

    // the -inf rows this workgroup fills at the end (loads issued now, with
    // the scan's, so that their latency is not paid at the end)
    const int pairs = B * H_kv;
    const int fill_ctx = (int)blockIdx.x < pairs ? ctx_len[blockIdx.x / H_kv] : 0;

    // items before each request, by a scan over the context lengths that
    // every wave does alike (uniform results, no synchronisation); up to 64
    // requests need one load per lane
    int c_lane = lane < B ? H_kv * valid_chunks(ctx_len, lane, NB_max) : 0;
    int total = 0;
    for (int r0 = 0; r0 < B; r0 += 64) {
        int c = r0 == 0 ? c_lane : (r0 + lane < B ? H_kv * valid_chunks(ctx_len, r0 + lane, NB_max) : 0);
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) c += __shfl_xor(c, o, 64);
        total += c;
    }
    total = __builtin_amdgcn_readfirstlane(total);  // uniform: keep the walk in scalar registers
    const int per = (total + (int)gridDim.x - 1) / (int)gridDim.x;
    const int v0 = min(total, (int)blockIdx.x * per), v1 = min(total, v0 + per);
    // the request holding item v0, and the item's place in it
    int r = 0, before = 0;
    if (v0 < v1) {
        for (int r0 = 0; r0 < B; r0 += 64) {
            const int c = r0 == 0 ? c_lane : (r0 + lane < B ? H_kv * valid_chunks(ctx_len, r0 + lane, NB_max) : 0);
            int inc = c;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const int y = __shfl_up(inc, o, 64);
                if (lane >= o) inc += y;
            }
            const int chunk_total = __shfl(inc, 63, 64);
            if (before + chunk_total > v0) {
                // first lane whose running count passes v0
                const unsigned long long m = __ballot(before + inc > v0);
                const int first = __ffsll((long long)m) - 1;
                r = __builtin_amdgcn_readfirstlane(r0 + first);
                before = __builtin_amdgcn_readfirstlane(before + __shfl(inc - c, first, 64));
                break;
            }
            before = __builtin_amdgcn_readfirstlane(before + chunk_total);
        }
    }
    int cr = v0 < v1 ? __builtin_amdgcn_readfirstlane(valid_chunks(ctx_len, r, NB_max)) : 0;  // chunks of r
    const int rem = v0 - before;                               // item index within request r
    int h = cr > 0 ? rem / cr : 0;
    int chunk = cr > 0 ? rem - h * cr : 0;

    int cur = -1, nb = 0;
    double qm[16], qp[16];
    for (int v = v0; v < v1; v++) {
        const int rh = r * H_kv + h;
        if (rh != cur) {  // uniform across the workgroup
            cur = rh;
            __syncthreads();
            if (tid < kD) {
                double sp = 0.0, sm = 0.0;
                for (int j = 0; j < J; j++) {
                    const uint16_t *qrow = q_look + (((size_t)r * J + j) * H_q + (size_t)h * G) * kD + tid;
                    for (int gi = 0; gi < G; gi++) {
                        const double v = bf16_d(qrow[(size_t)gi * kD]);
                        if (v > 0.0) sp += v; else sm += v;
                    }
                }
                Qsh[0][tid] = sm;
                Qsh[1][tid] = sp;
            }
            __syncthreads();
#pragma unroll
            for (int e = 0; e < 8; e++) {
                qm[e] = Qsh[0][li * 8 + e];
                qm[8 + e] = Qsh[0][64 + li * 8 + e];
                qp[e] = Qsh[1][li * 8 + e];
                qp[8 + e] = Qsh[1][64 + li * 8 + e];
            }
            nb = n_blocks_of(ctx_len[r], NB_max);
        }
        float *out = scores + (size_t)rh * NB_max;
        const uint4 *base = kminmax + (size_t)rh * NB_max * 32;  // 32 uint4 per block summary
        const int b0 = chunk * kItemBlocks + tid / kLanesPerBlock;
        uint4 mn0[kUnroll], mn1[kUnroll], mx0[kUnroll], mx1[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; u++) {
            const int b = b0 + u * kBlocksPerGroup;
            if (b < nb) {
                const uint4 *sb = base + (size_t)b * 32;
                mn0[u] = sb[li];
                mn1[u] = sb[8 + li];
                mx0[u] = sb[16 + li];
                mx1[u] = sb[24 + li];
            }
        }
#pragma unroll
        for (int u = 0; u < kUnroll; u++) {
            const int b = b0 + u * kBlocksPerGroup;
            if (b >= NB_max) continue;            // the octet skips together
            if (b >= nb) {
                if (li == 0) out[b] = -INFINITY;
                continue;
            }
            const uint32_t wmn[8] = {mn0[u].x, mn0[u].y, mn0[u].z, mn0[u].w,
                                     mn1[u].x, mn1[u].y, mn1[u].z, mn1[u].w};
            const uint32_t wmx[8] = {mx0[u].x, mx0[u].y, mx0[u].z, mx0[u].w,
                                     mx1[u].x, mx1[u].y, mx1[u].z, mx1[u].w};
            double acc = 0.0;
#pragma unroll
            for (int w = 0; w < 8; w++) {
                const int e = (w < 4) ? 2 * w : 8 + 2 * (w - 4);
                acc = fma(qm[e], bf16_d(wmn[w] & 0xffffu), acc);
                acc = fma(qm[e + 1], bf16_d(wmn[w] >> 16), acc);
                acc = fma(qp[e], bf16_d(wmx[w] & 0xffffu), acc);
                acc = fma(qp[e + 1], bf16_d(wmx[w] >> 16), acc);
            }
            acc = octet_sum(acc);
            if (li == 0) out[b] = (float)acc;
        }
        // next item: the next chunk, then the next KV head, then the next
        // request with any blocks
        if (++chunk == cr) {
            chunk = 0;
            if (++h == H_kv) {
                h = 0;
                do {
                    ++r;
                    cr = r < B ? __builtin_amdgcn_readfirstlane(valid_chunks(ctx_len, r, NB_max)) : 1;
                } while (cr == 0);
            }
        }
    }

    // -inf past each request's last valid chunk
    for (int rh = blockIdx.x; rh < pairs; rh += gridDim.x) {
        const int c = rh == (int)blockIdx.x ? fill_ctx : ctx_len[rh / H_kv];
        const int first = (n_blocks_of(c, NB_max) + kItemBlocks - 1) / kItemBlocks * kItemBlocks;
        float *out = scores + (size_t)rh * NB_max;
        for (int b = first + tid; b < NB_max; b += kThreads) out[b] = -INFINITY;
    }
}

int score_grid(int n_items) {
    static int occ = 0;  // resident workgroups per compute unit
    if (occ == 0) {
        int o = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&o, score_kernel, kThreads, 0) != hipSuccess || o < 1) o = 2;
        occ = o;
    }
    const long g = (long)device_cu_count() * occ;
    return (int)(n_items < g ? n_items : g);
}

}  // namespace

hipError_t launch_score(const oasis_dims &d, const uint16_t *q_look, int J,
                        const uint16_t *kminmax, const int32_t *ctx_len,
                        float *scores, hipStream_t s) {
    const int chunks = (d.NB_max + kItemBlocks - 1) / kItemBlocks;
    const int n_items = d.B * d.H_kv * chunks;  // at most this many items hold blocks
    hipLaunchKernelGGL(score_kernel, dim3((unsigned)score_grid(n_items)), dim3(kThreads), 0, s, q_look, J,
                       d.H_q, d.H_kv, reinterpret_cast<const uint4 *>(kminmax), ctx_len, scores, d.NB_max,
                       d.B);
    return hipGetLastError();
}

}  // namespace oasis
