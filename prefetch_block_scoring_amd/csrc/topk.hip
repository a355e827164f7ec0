// Top-K block selection under the token budget.
//
// OasisKV (arXiv 2608.08097), paperlayer summary, sections 4 and 5: per KV
// head and layer, the best-scoring blocks that fit the KV budget (2048 tokens
// by default, K_b = budget / bs blocks) are predicted for the next step.
// Order: fp32 score descending, equal scores by lower block id; ids are
// written ascending.
//
// One workgroup per (request, KV head).  Scores are mapped to order-preserving
// uint32 keys in LDS; a radix select (8-bit digits, most significant first)
// finds the K_b-th largest key T and how many keys equal to T must be taken,
// starting at the first digit where the keys differ (the leading digits all
// keys share, from an AND / OR of the keys, go straight into the prefix); a
// compaction in index order then writes every key > T and the first `need`
// keys == T, which is exactly the (score desc, id asc) prefix.  All work is
// integer, so the result is bit-exact.
#include "oasis_internal.h"

namespace oasis {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;

// Exclusive scan of one uint32 per thread across the workgroup; returns the
// exclusive prefix and writes the total to *total.  `tmp` holds kWaves words.
__device__ __forceinline__ uint32_t wg_exclusive_scan(uint32_t v, uint32_t *tmp, uint32_t *total) {
    const int lane = threadIdx.x % 64, wave = threadIdx.x / 64;
    uint32_t inc = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const uint32_t y = __shfl_up(inc, o, 64);
        if (lane >= o) inc += y;
    }
    if (lane == 63) tmp[wave] = inc;
    __syncthreads();
    uint32_t before = 0, all = 0;
#pragma unroll
    for (int w = 0; w < kWaves; w++) {
        const uint32_t t = tmp[w];
        before += (w < wave) ? t : 0u;
        all += t;
    }
    __syncthreads();
    *total = all;
    return before + inc - v;
}

__global__ __launch_bounds__(kThreads) void topk_kernel(
    const float *__restrict__ scores, const int32_t *__restrict__ ctx_len, int H_kv,
    int NB_max, int K_b, int32_t *__restrict__ sel, int32_t *__restrict__ n_sel) {
    extern __shared__ uint32_t keys[];  // NB_max
    __shared__ uint32_t hist[kWaves][256];
    __shared__ uint32_t tmp[kWaves];
    __shared__ uint32_t s_digit, s_above;
    __shared__ uint32_t s_and[kWaves], s_or[kWaves];

    const int rh = blockIdx.x;
    const int r = rh / H_kv;
    const int tid = threadIdx.x;
    const int wave = tid / 64;
    const float *row = scores + (size_t)rh * NB_max;
    // Scores are read kBatch per thread at a time, every load issued before
    // any is used; the first batch goes out with the context length (the row
    // holds NB_max scores, so the reads stay inside it whatever the length).
    constexpr int kBatch = 8;
    float v[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; u++) v[u] = row[min(tid + u * kThreads, NB_max - 1)];
    const int nb = n_blocks_of(ctx_len[r], NB_max);
    int32_t *out = sel + (size_t)rh * K_b;

    if (nb <= K_b) {
        for (int i = tid; i < K_b; i += kThreads) out[i] = i < nb ? i : -1;
        if (tid == 0) n_sel[rh] = nb;
        return;
    }

    uint32_t k_and = 0xffffffffu, k_or = 0u;
    for (int b0 = tid;; b0 += kBatch * kThreads) {
#pragma unroll
        for (int u = 0; u < kBatch; u++) {
            const int b = b0 + u * kThreads;
            if (b < nb) {
                const uint32_t key = rank_key(v[u]);
                keys[b] = key;
                k_and &= key;
                k_or |= key;
            }
        }
        if (b0 + kBatch * kThreads >= nb) break;
#pragma unroll
        for (int u = 0; u < kBatch; u++) v[u] = row[min(b0 + (kBatch + u) * kThreads, nb - 1)];
    }
    // bits every key shares: the leading digits made of them need no pass
    // (the scores of one row usually share sign and most of the exponent)
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        k_and &= __shfl_xor(k_and, o, 64);
        k_or |= __shfl_xor(k_or, o, 64);
    }
    if ((tid & 63) == 0) {
        s_and[wave] = k_and;
        s_or[wave] = k_or;
    }
    __syncthreads();
#pragma unroll
    for (int w = 0; w < kWaves; w++) {
        k_and &= s_and[w];
        k_or |= s_or[w];
    }
    const uint32_t diff = k_and ^ k_or;  // bits where some keys differ

    // ---- radix select of the K_b-th largest key
    uint32_t prefix = 0, mask = 0;
    uint32_t k = (uint32_t)K_b;  // rank still to find among keys matching prefix
    int first_shift = 24;
    while (first_shift > 0 && ((diff >> first_shift) & 255u) == 0) {
        prefix |= k_and & (255u << first_shift);
        mask |= 255u << first_shift;
        first_shift -= 8;
    }
    for (int shift = first_shift; shift >= 0; shift -= 8) {
        for (int i = tid; i < kWaves * 256; i += kThreads) (&hist[0][0])[i] = 0;
        __syncthreads();
        for (int b = tid; b < nb; b += kThreads) {
            const uint32_t key = keys[b];
            if ((key & mask) == prefix) atomicAdd(&hist[wave][(key >> shift) & 255u], 1u);
        }
        __syncthreads();
        // thread t looks at digit 255 - t: inclusive suffix count from the top
        const uint32_t digit = 255u - (uint32_t)tid;
        uint32_t c = 0;
#pragma unroll
        for (int w = 0; w < kWaves; w++) c += hist[w][digit];
        uint32_t total;
        const uint32_t above = wg_exclusive_scan(c, tmp, &total);  // keys with larger digits
        if (above < k && above + c >= k) {
            s_digit = digit;
            s_above = above;
        }
        __syncthreads();
        prefix |= s_digit << shift;
        mask |= 255u << shift;
        k -= s_above;
        __syncthreads();
    }
    const uint32_t T = prefix;  // K_b-th largest key
    const uint32_t need = k;    // how many keys == T are taken (lowest ids first)

    // ---- compaction in index order: thread t owns a contiguous id range
    const int per = (nb + kThreads - 1) / kThreads;
    const int lo = min(nb, tid * per), hi = min(nb, lo + per);
    uint32_t gt = 0, eq = 0;
    for (int b = lo; b < hi; b++) {
        const uint32_t key = keys[b];
        gt += key > T;
        eq += key == T;
    }
    uint32_t tot;
    const uint32_t eq_before = wg_exclusive_scan(eq, tmp, &tot);
    const uint32_t take_eq = need > eq_before ? min(need - eq_before, eq) : 0u;
    const uint32_t pos0 = wg_exclusive_scan(gt + take_eq, tmp, &tot);
    uint32_t pos = pos0, eq_seen = 0;
    for (int b = lo; b < hi; b++) {
        const uint32_t key = keys[b];
        bool take = key > T;
        if (key == T) {
            take = eq_seen < take_eq;
            eq_seen++;
        }
        if (take && pos < (uint32_t)K_b) out[pos++] = b;
    }
    if (tid == 0) n_sel[rh] = K_b;
}

}  // namespace

hipError_t launch_topk(const oasis_dims &d, const float *scores, const int32_t *ctx_len,
                       int K_b, int32_t *sel, int32_t *n_sel, hipStream_t s, hipEvent_t done) {
    const size_t lds = (size_t)d.NB_max * sizeof(uint32_t);
    hipExtLaunchKernelGGL(topk_kernel, dim3((unsigned)(d.B * d.H_kv)), dim3(kThreads), lds, s, nullptr, done, 0,
                          scores, ctx_len, d.H_kv, d.NB_max, K_b, sel, n_sel);
    return hipGetLastError();
}

}  // namespace oasis
