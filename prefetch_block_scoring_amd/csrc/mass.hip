// Exact attention mass per block, and top-K overlap: the lookahead-agreement
// analogue.
//
// OasisKV (arXiv 2608.08097), paperlayer summary, section 4, reports how
// often the draft-based top-K block prediction agrees with the true next
// token's top-K set.  Here the true set of KV head h is the top-K by the next
// query's exact attention mass over the whole context, summed over the query
// heads g of h's group:
//     mass[b] = sum_g sum_{t in b} exp(l_gt - M_g) / L_g,
//     M_g = max_t l_gt,  L_g = sum_t exp(l_gt - M_g).
// Two kernels: block_stats_kernel reads every valid key once (q . K on the
// matrix cores, as in attention) and writes, per (head g, block b), the
// block's own max m and sum s = sum_{t in b} exp(l_t - m); block_mass_kernel
// then forms M_g = max_b m, L_g = sum_b s exp(m - M_g) and the masses.  The
// logits are kept in base 2 (scaled by log2 e), as in attention.
#include "oasis_internal.h"

#include <cmath>

namespace oasis {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kVecPerBlock = (int)(kBlockBytes / 16);  // uint4 per K+V block

__device__ __forceinline__ float exp2_(float x) { return __builtin_amdgcn_exp2f(x); }

// stats[(rh * G + g) * NB_max + b] = (m, s) of head g of pair rh over block b.
__global__ __launch_bounds__(kThreads, 4) void block_stats_kernel(
    const uint16_t *__restrict__ q, const uint4 *__restrict__ kv, const int32_t *__restrict__ ctx_len,
    float scale_log2, int H_q, int H_kv, int NB_max, int n_split, float2 *__restrict__ stats) {
    __shared__ uint4 q_lds[16][17];
    const int rh = blockIdx.x, split = blockIdx.y;
    const int r = rh / H_kv, h = rh - r * H_kv;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int col = lane & 15, grp = lane >> 4;
    const int G = H_q / H_kv;
    const int ctx = ctx_len[r];
    const int nb = n_blocks_of(ctx, NB_max);
    const int per = (nb + n_split - 1) / n_split;
    const int b0 = split * per, b1 = min(nb, b0 + per);
    {
        const int c = tid >> 4, chunk = tid & 15;
        uint4 v = make_uint4(0, 0, 0, 0);
        if (c < G) v = reinterpret_cast<const uint4 *>(q + ((size_t)r * H_q + (size_t)h * G + c) * kD)[chunk];
        q_lds[c][chunk] = v;
    }
    __syncthreads();
    const uint4 *pool = kv + (size_t)rh * NB_max * kVecPerBlock;
    float2 *out = stats + (size_t)rh * G * NB_max;
    auto load = [&](int b, uint4 (&kr)[4]) {
        const uint4 *src = pool + (size_t)b * kVecPerBlock;
#pragma unroll
        for (int kk = 0; kk < 4; kk++) kr[kk] = src[col * 16 + kk * 4 + grp];
    };
    int b = b0 + wave;
    uint4 kc[4];
    if (b < b1) load(b, kc);
    for (; b < b1; b += kWaves) {
        uint4 kn[4];
        const int bn = b + kWaves;
        if (bn < b1) load(bn, kn);
        f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < 4; kk++)
            c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kc[kk]),
                                                         __builtin_bit_cast(bf16x8, q_lds[col][kk * 4 + grp]), c,
                                                         0, 0, 0);
        const int valid = ctx - b * kBs;
        float l[4];
#pragma unroll
        for (int t = 0; t < 4; t++) l[t] = (4 * grp + t < valid) ? c[t] * scale_log2 : -INFINITY;
        float m = fmaxf(fmaxf(l[0], l[1]), fmaxf(l[2], l[3]));
        m = fmaxf(m, __shfl_xor(m, 16));
        m = fmaxf(m, __shfl_xor(m, 32));
        float s = 0.f;
#pragma unroll
        for (int t = 0; t < 4; t++) s += exp2_(l[t] - m);  // the block holds >= 1 valid token: m finite
        s += __shfl_xor(s, 16);
        s += __shfl_xor(s, 32);
        if (grp == 0 && col < G) out[(size_t)col * NB_max + b] = make_float2(m, s);
#pragma unroll
        for (int x = 0; x < 4; x++) kc[x] = kn[x];
    }
}

__device__ __forceinline__ float wg_reduce(float v, bool is_max, float *tmp) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const float y = __shfl_xor(v, o, 64);
        v = is_max ? fmaxf(v, y) : v + y;
    }
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    __syncthreads();
    if (lane == 0) tmp[wave] = v;
    __syncthreads();
    float all = tmp[0];
#pragma unroll
    for (int w = 1; w < kWaves; w++) all = is_max ? fmaxf(all, tmp[w]) : all + tmp[w];
    return all;
}

// One workgroup per (request, KV head): mass[rh][b] for b < NB_max.
__global__ __launch_bounds__(kThreads) void block_mass_kernel(const float2 *__restrict__ stats,
                                                              const int32_t *__restrict__ ctx_len, int H_q,
                                                              int H_kv, int NB_max, float *__restrict__ mass) {
    __shared__ float tmp[kWaves];
    __shared__ float Mg[16], Lg[16];
    const int rh = blockIdx.x;
    const int r = rh / H_kv;
    const int G = H_q / H_kv;
    const int nb = n_blocks_of(ctx_len[r], NB_max);
    const float2 *st = stats + (size_t)rh * G * NB_max;
    for (int g = 0; g < G; g++) {
        float m = -INFINITY;
        for (int b = threadIdx.x; b < nb; b += kThreads) m = fmaxf(m, st[(size_t)g * NB_max + b].x);
        const float M = wg_reduce(m, true, tmp);
        float l = 0.f;
        for (int b = threadIdx.x; b < nb; b += kThreads) {
            const float2 v = st[(size_t)g * NB_max + b];
            l += v.y * exp2_(v.x - M);
        }
        const float L = wg_reduce(l, false, tmp);
        if (threadIdx.x == 0) {
            Mg[g] = M;
            Lg[g] = L;
        }
    }
    __syncthreads();
    float *out = mass + (size_t)rh * NB_max;
    for (int b = threadIdx.x; b < NB_max; b += kThreads) {
        float x = 0.f;
        if (b < nb)
            for (int g = 0; g < G; g++) {
                const float2 v = st[(size_t)g * NB_max + b];
                x += Lg[g] > 0.f ? v.y * exp2_(v.x - Mg[g]) / Lg[g] : 0.f;
            }
        out[b] = x;
    }
}

// |A & B| per (request, KV head) for two ascending, -1 padded top-K lists.
__global__ __launch_bounds__(64) void topk_overlap_kernel(const int32_t *__restrict__ a, const int32_t *__restrict__ na,
                                                          const int32_t *__restrict__ b, const int32_t *__restrict__ nb,
                                                          int K, int pairs, int32_t *__restrict__ out) {
    const int rh = blockIdx.x * 64 + threadIdx.x;
    if (rh >= pairs) return;
    const int32_t *x = a + (size_t)rh * K, *y = b + (size_t)rh * K;
    const int n = min(max(na[rh], 0), K), m = min(max(nb[rh], 0), K);
    int i = 0, j = 0, c = 0;
    while (i < n && j < m) {
        if (x[i] == y[j]) {
            c++;
            i++;
            j++;
        } else if (x[i] < y[j]) {
            i++;
        } else {
            j++;
        }
    }
    out[rh] = c;
}

}  // namespace

size_t block_mass_ws_bytes(const oasis_dims &d) { return (size_t)d.B * d.H_q * d.NB_max * sizeof(float2); }

hipError_t launch_block_mass(const oasis_dims &d, const uint16_t *q, const void *kv_dev, const int32_t *ctx_len,
                             float sm_scale, float *mass, void *ws, hipStream_t s) {
    // enough workgroups for four per compute unit, at least eight blocks each
    const long pairs = (long)d.B * d.H_kv;
    long sp = (4L * device_cu_count() + pairs - 1) / pairs;
    const long cap = (d.NB_max + 7) / 8;
    sp = sp > cap ? cap : sp;
    const int splits = (int)(sp < 1 ? 1 : (sp > 64 ? 64 : sp));
    hipLaunchKernelGGL(block_stats_kernel, dim3((unsigned)(d.B * d.H_kv), (unsigned)splits), dim3(kThreads), 0, s,
                       q, static_cast<const uint4 *>(kv_dev), ctx_len, sm_scale * 1.4426950408889634f, d.H_q, d.H_kv,
                       d.NB_max, splits, static_cast<float2 *>(ws));
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(block_mass_kernel, dim3((unsigned)(d.B * d.H_kv)), dim3(kThreads), 0, s,
                       static_cast<const float2 *>(ws), ctx_len, d.H_q, d.H_kv, d.NB_max, mass);
    return hipGetLastError();
}

hipError_t launch_topk_overlap(int pairs, const int32_t *a, const int32_t *na, const int32_t *b, const int32_t *nb,
                               int K, int32_t *out, hipStream_t s) {
    hipLaunchKernelGGL(topk_overlap_kernel, dim3((unsigned)((pairs + 63) / 64)), dim3(64), 0, s, a, na, b, nb, K,
                       pairs, out);
    return hipGetLastError();
}

}  // namespace oasis
