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
// Mapping: the grid is persistent (two workgroups per compute unit).  The
// work items are the (request, KV head, 64-block chunk) triples whose chunk
// holds at least one of the request's blocks; they are split into equal
// contiguous ranges, one per workgroup, so that ragged contexts balance and
// Qp / Qm are rebuilt only when a range crosses into the next (request, KV
// head).  Each workgroup counts the items itself from the context lengths.
// The chunks past a request's last block only get -inf, in a second, strided
// loop.
//
// Sixteen lanes share a block (512 bytes of summary): lane i of the sixteen
// holds dims [8i, 8i + 8) of kmin and of kmax (two 16-byte loads), so a wave's
// load instruction reads four consecutive blocks' halves, 1 KiB in whole
// 128-byte lines, and a lane keeps only 16 of the 256 Qp / Qm values (32
// registers).  The sixteen partial sums meet through four DPP steps.  A wave
// owns 16 consecutive blocks of each 64-block chunk; their scores go to an
// LDS buffer, and the workgroup writes the scores of all its items once its
// loads are done (a store between the loads of a streaming read turns the
// memory around and cost ~9% alone at batch 128).
//
// Software pipeline: the registers hold two items' load groups (eight groups,
// 16 KiB per wave).  As each group of the current item is used, the same
// registers are refilled with that group of the item two ahead, so a wave
// keeps about 14 KiB of loads in flight while its fp64 arithmetic runs.  When
// a range crosses into another (request, KV head), the first two items' loads
// are issued before the Qp / Qm rebuild, whose query loads then wait with
// them (the load counter is in order): one memory latency per crossing
// instead of two (3-4% alone at batch 32 and on ragged contexts).
#include "oasis_internal.h"

namespace oasis {
namespace {

constexpr int kThreads = 256;
constexpr int kLanesPerBlock = 16;                          // lanes sharing one block
constexpr int kBlocksPerGroup = kThreads / kLanesPerBlock;  // 16: blocks per load instruction of the workgroup
constexpr int kGroups = 4;                                  // load groups per item
constexpr int kItemBlocks = kBlocksPerGroup * kGroups;      // 64 blocks per item
constexpr int kBuf = 2 * kGroups;                           // uint4 per lane per item
constexpr int kMaxItems = 32;                               // items per workgroup, their scores kept in LDS

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Word 3 of a raw buffer resource for dword loads (no swizzle, no format
// conversion): the value gfx9-family raw buffers use.
constexpr int kRsrcWord3 = 0x00020000;
constexpr int kSummaryBytes = 2 * kD * 2;  // one block's kmin and kmax, bf16
// A byte offset past every row (NB_max <= 16384 blocks: at most 8 MiB) that a
// lane's offset within a group cannot carry past 2^31 - 1.
constexpr int kPastRow = 0x7fff0000;

// 16 bytes at byte offset `off` of a raw buffer; zeros when off is at or past
// the buffer's size.  The whole offset goes in the vector operand, which the
// range check always covers.
__device__ __forceinline__ u32x4 load16(__amdgpu_buffer_rsrc_t r, int off) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

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

// Sum over the sixteen lanes of a DPP row; every lane gets the total.
__device__ __forceinline__ double row_sum(double x) {
    x += dpp_d<0xB1>(x);   // quad_perm [1,0,3,2]
    x += dpp_d<0x4E>(x);   // quad_perm [2,3,0,1]
    x += dpp_d<0x141>(x);  // row_half_mirror: lane i <- lane 7 - i within 8
    x += dpp_d<0x140>(x);  // row_mirror: lane i <- lane 15 - i within 16
    return x;
}

// chunks of request r that hold at least one of its blocks
__device__ __forceinline__ int valid_chunks(const int32_t *ctx_len, int r, int NB_max) {
    return (n_blocks_of(ctx_len[r], NB_max) + kItemBlocks - 1) / kItemBlocks;
}

__device__ __forceinline__ int uni(int x) { return __builtin_amdgcn_readfirstlane(x); }

__global__ __launch_bounds__(kThreads, 3) void score_kernel(
    const uint16_t *__restrict__ q_look, int J, int H_q, int H_kv,
    const uint4 *__restrict__ kminmax, const int32_t *__restrict__ ctx_len,
    float *__restrict__ scores, int NB_max, int B) {
    // per half of the workgroup: [half][0] = its part of Qm (pairs with kmin),
    // [half][1] of Qp (pairs with kmax); each lane adds the two halves
    __shared__ double Qpart[2][2][kD];
    // the scores of the workgroup's items (at most kMaxItems, which the grid
    // size guarantees), written out together at the end, with each item's
    // place in the score array and how many of its 64 blocks lie below NB_max
    __shared__ float sbuf[kMaxItems * kItemBlocks];
    __shared__ int sdst[kMaxItems];
    __shared__ int scnt[kMaxItems];
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
    const int ctx_lane = lane < B ? ctx_len[lane] : 0;  // requests 0 .. 63
    int c_lane = lane < B ? H_kv * ((n_blocks_of(ctx_lane, NB_max) + kItemBlocks - 1) / kItemBlocks) : 0;
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
    int r = 0, before = 0, ctx_r = 0;
    if (v0 < v1) {
        for (int r0 = 0; r0 < B; r0 += 64) {
            const int ctx_l = r0 == 0 ? ctx_lane : (r0 + lane < B ? ctx_len[r0 + lane] : 0);
            const int c = H_kv * ((n_blocks_of(ctx_l, NB_max) + kItemBlocks - 1) / kItemBlocks);
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
                ctx_r = __builtin_amdgcn_readfirstlane(__shfl(ctx_l, first, 64));
                break;
            }
            before = __builtin_amdgcn_readfirstlane(before + chunk_total);
        }
    }

    double qm[8], qp[8];

    // Qp / Qm of (request r, KV head h) into the registers
    auto rebuild = [&](int rr, int hh) {
        __syncthreads();  // every wave has read the previous Qp / Qm
        {
            // dim tid % 128 over the J * G query rows of the group; the two
            // halves of the workgroup take alternate rows, four independent
            // loads at a time (rows past the last re-read it, then count as 0)
            const int dim = tid & (kD - 1), half = tid >> 7;
            const int nk = J * G;
            double sp = 0.0, sm = 0.0;
            for (int k0 = half; k0 < nk; k0 += 8) {
                uint32_t raw[4];
#pragma unroll
                for (int t = 0; t < 4; t++) {
                    const int k = min(k0 + 2 * t, nk - 1), j = k / G, gi = k - j * G;
                    raw[t] = q_look[(((size_t)rr * J + j) * H_q + (size_t)hh * G + gi) * kD + dim];
                }
#pragma unroll
                for (int t = 0; t < 4; t++) {
                    const double v = k0 + 2 * t < nk ? bf16_d(raw[t]) : 0.0;
                    if (v > 0.0) sp += v; else sm += v;
                }
            }
            Qpart[half][0][dim] = sm;
            Qpart[half][1][dim] = sp;
        }
        __syncthreads();
#pragma unroll
        for (int e = 0; e < 8; e++) {
            const int d = li * 8 + e;
            qm[e] = Qpart[0][0][d] + Qpart[1][0][d];
            qp[e] = Qpart[0][1][d] + Qpart[1][1][d];
        }
    };

    // Loads go through a raw buffer resource over the valid blocks of one
    // (request, KV head) row (base and size in scalar registers): a lane adds
    // its fixed offset in the group to the chunk's group offset, and a block
    // past the request's last one reads zeros, so no load sits under a branch
    // or needs a clamp.
    // Wave w owns blocks [16 w, 16 w + 16) of each 64-block chunk: group g
    // covers its blocks 4 g + q, q = lane / 16 (a DPP row per block).  After
    // the four groups, lane d < 16 holds the score of the wave's block d.
    // Scores collect in LDS and go out once, after the workgroup's last item:
    // 64-byte writes scattered through the summary stream cost far more than
    // their bytes (the DRAM turns from reads to writes for each), about 9% of
    // the kernel, and the loop then holds no store.
    const int wave = tid >> 6;
    const int row_q = lane >> 4;
    const int lane_voff = (16 * wave + row_q) * kSummaryBytes + li * 16;

    // Segments: the runs of consecutive items of one (request, KV head) in
    // this workgroup's range.  Qp / Qm are rebuilt at the start of each; the
    // chunks of a segment then run through the pipeline, whose loop holds no
    // branch but its exit.
    int v = v0;
    int rr = r, hh = 0, chunk = 0;
    int nb = 0, cr = 0;
    if (v0 < v1) {
        nb = uni(n_blocks_of(ctx_r, NB_max));  // from the scan: no second load
        cr = (nb + kItemBlocks - 1) / kItemBlocks;
        const int rem = v0 - before;  // item index within request r
        hh = uni(rem / cr);
        chunk = uni(rem - hh * cr);
    }
    while (v < v1) {
        const int c1 = uni(min(cr, chunk + (v1 - v)));  // this segment: chunks [chunk, c1)
        const int rh = uni(rr * H_kv + hh);
        const auto in = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<uint4 *>(kminmax + (size_t)rh * NB_max * 32), (short)0, nb * kSummaryBytes, kRsrcWord3);
        const int last = c1 - 1;
        // loads of group g of chunk c (its byte offset in the row is uniform)
        auto load_group = [&](int c, int g, u32x4 &mn, u32x4 &mx) {
            const int o = lane_voff + uni(c <= last ? (c * kItemBlocks + 4 * g) * kSummaryBytes : kPastRow);
            mn = load16(in, o);               // kmin, dims [8 li, 8 li + 8)
            mx = load16(in, o + kD * 2);      // kmax, the same dims
        };
        // group g of chunk c: its scores go to lanes 4 g + q of `sv`; the
        // registers are refilled with group g of chunk c_next
        auto group = [&](int g, u32x4 &mn, u32x4 &mx, int c_next, float &sv) {
            const uint32_t wmn[4] = {mn.x, mn.y, mn.z, mn.w};
            const uint32_t wmx[4] = {mx.x, mx.y, mx.z, mx.w};
            double acc = 0.0;
#pragma unroll
            for (int w = 0; w < 4; w++) {
                acc = fma(qm[2 * w], bf16_d(wmn[w] & 0xffffu), acc);
                acc = fma(qm[2 * w + 1], bf16_d(wmn[w] >> 16), acc);
                acc = fma(qp[2 * w], bf16_d(wmx[w] & 0xffffu), acc);
                acc = fma(qp[2 * w + 1], bf16_d(wmx[w] >> 16), acc);
            }
            load_group(c_next, g, mn, mx);
            acc = row_sum(acc);
            const float got = __shfl((float)acc, 16 * (lane & 3), 64);  // block 4 g + (lane & 3)
            if ((lane >> 2) == g) sv = got;
        };
        // the wave's 16 scores of chunk c (the workgroup's item k), -inf
        // past the request's blocks, into LDS
        auto keep_chunk = [&](int c, int k, float sv) {
            const int b = c * kItemBlocks + 16 * wave + lane;
            if (lane < 16) sbuf[k * kItemBlocks + 16 * wave + lane] = b < nb ? sv : -INFINITY;
        };
        const int k0 = v - v0;  // the segment's first item, in the workgroup's order
        for (int i = tid; i < c1 - chunk; i += kThreads) {
            sdst[k0 + i] = rh * NB_max + (chunk + i) * kItemBlocks;
            scnt[k0 + i] = min(kItemBlocks, NB_max - (chunk + i) * kItemBlocks);
        }
        u32x4 X[kBuf], Y[kBuf];
#pragma unroll
        for (int g = 0; g < kGroups; g++) load_group(chunk, g, X[2 * g], X[2 * g + 1]);
#pragma unroll
        for (int g = 0; g < kGroups; g++) load_group(chunk + 1, g, Y[2 * g], Y[2 * g + 1]);
        // Qp / Qm of the segment while its first loads are in flight
        rebuild(rr, hh);
        // X holds chunk c, Y chunk c + 1; using X refills it with c + 2, using
        // Y with c + 3.  A refill past the segment gets an offset past the
        // buffer's end (a uniform select, not a branch), so the buffer unit
        // returns zeros without a memory request and the loop body stays
        // straight-line code (re-reading the last chunk instead cost 2 of a
        // workgroup's 8 items in L2 reads at batch 32: 461k against 467k
        // tok/s in the pipeline).
        for (int c = chunk;; c += 2) {
            float sv = 0.f;
#pragma unroll
            for (int g = 0; g < kGroups; g++) group(g, X[2 * g], X[2 * g + 1], c + 2, sv);
            keep_chunk(c, k0 + c - chunk, sv);
            if (c + 1 >= c1) break;
#pragma unroll
            for (int g = 0; g < kGroups; g++) group(g, Y[2 * g], Y[2 * g + 1], c + 3, sv);
            keep_chunk(c + 1, k0 + c + 1 - chunk, sv);
            if (c + 2 >= c1) break;
        }
        v += c1 - chunk;
        // next segment: the next KV head, then the next request with blocks
        chunk = 0;
        if (++hh >= H_kv) {
            hh = 0;
            do {
                rr = uni(rr + 1);
                nb = rr < B ? uni(n_blocks_of(ctx_len[rr], NB_max)) : 1;
                cr = (nb + kItemBlocks - 1) / kItemBlocks;
            } while (cr == 0);
        }
    }

    // the workgroup's scores: item i's blocks below NB_max go to sdst[i]
    __syncthreads();
    for (int idx = tid; idx < (v1 - v0) * kItemBlocks; idx += kThreads) {
        const int i = idx / kItemBlocks, j = idx - i * kItemBlocks;
        if (j < scnt[i]) scores[sdst[i] + j] = sbuf[idx];
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
    // a persistent grid of two workgroups per compute unit (four fit, but
    // fewer workgroups with longer item ranges pay the range set-up and the
    // Qp / Qm rebuilds less often: alone over rotated copies at batch 128 /
    // 16K, 96.6 against 98.8 us; in the reasoning pipeline 343k against
    // 326k tok/s; at batch 32, 27.5 us alone and 462k tok/s against 28.3 us
    // and 424k with four, 31.9 us and 420k with three), but at least enough
    // that no workgroup holds more than kMaxItems items
    long g = (long)device_cu_count() * (occ < 2 ? occ : 2);
    const long need = (n_items + kMaxItems - 1) / kMaxItems;
    if (g < need) g = need;
    return (int)(n_items < g ? n_items : g);
}

}  // namespace

hipError_t launch_score(const oasis_dims &d, const uint16_t *q_look, int J,
                        const uint16_t *kminmax, const int32_t *ctx_len,
                        float *scores, hipStream_t s, hipEvent_t done) {
    const int chunks = (d.NB_max + kItemBlocks - 1) / kItemBlocks;
    const int n_items = d.B * d.H_kv * chunks;  // at most this many items hold blocks
    hipExtLaunchKernelGGL(score_kernel, dim3((unsigned)score_grid(n_items)), dim3(kThreads), 0, s, nullptr,
                          done, 0, q_look, J, d.H_q, d.H_kv, reinterpret_cast<const uint4 *>(kminmax), ctx_len,
                          scores, d.NB_max, d.B);
    return hipGetLastError();
}

}  // namespace oasis
