// Sparse GQA decode attention over the staged blocks (split-K flash decode).
//
// OasisKV (arXiv 2608.08097), paperlayer summary, sections 4 and 7: decode
// attention runs only over the KV blocks held in the HBM working set.  For each
// query head, softmax attention over the valid tokens of the listed blocks.
//
// Look-ahead attention (section 4: the normal and the draft queries are
// computed together over the resident KV) is the same kernel with n_q query
// vectors per request: the MFMA's 16 columns hold the n_q * G (query, head)
// pairs of the KV group, column c = query (c / G), head (c % G), and every
// K / V load serves all of them.  Plain decode attention is n_q = 1.
//
// Work split: a workgroup of four or eight waves owns one (request, KV head)
// and one of n_split contiguous ranges of its table; the waves take the
// range's entries round-robin and keep private online-softmax states, merged
// in LDS at the end; with n_split > 1 a second kernel merges the ranges by
// their log-sum-exp.  The launch shape (attn_shape) aims at two waves per
// SIMD: one split of four-wave workgroups when there are enough (request,
// KV head) pairs, else one split of eight-wave workgroups, else more splits.
//
// Per 16-token block (8 KiB of K and V) a wave does:
//   q . K   on the matrix cores: one v_mfma_f32_16x16x32_bf16 per 32 dims,
//           A = K (16 tokens x 32 dims), B = Q^T (32 dims x 16 columns, the
//           group's n_q * G query rows, the rest zero).  The columns share
//           every K load, and the MFMA replaces n_q * G * 128 VALU FMAs per
//           token.
//           Each lane loads 16 bytes of one key row per MFMA; since the sum
//           over dims may be taken in any order, A and B only have to agree on
//           which dims a lane brings.
//   softmax fp32, base-2 online max / sum per head on the MFMA output.
//   p . V   up to 8 columns (attn_kernel): on the VALU; lane (c, q) owns
//           dims [8c, 8c + 8) of tokens q, q + 4, q + 8, q + 12, each V load
//           is a fully used 1 KiB row group, and the four token groups are
//           summed once at the end.  VALU work and accumulator registers
//           grow with the columns (8 per column per lane).
//           9 to 16 columns (attn_pv_kernel): on the matrix cores,
//           O^T[dims][columns] += V^T[dims][16 tokens] P[16 tokens][columns]
//           with v_mfma_f32_16x16x16_bf16.  The logits' MFMA output already
//           is P in the B-operand layout; V is transposed through a 5 KiB
//           LDS tile per wave; p enters as two bf16 parts (hi + lo).  The
//           accumulator is 32 registers for any column count, so 16 columns
//           run at four waves per SIMD, at the cost of one column.
// Loads of the next block are issued before the current block is computed.
#include "oasis_internal.h"

#include <cmath>
#include <mutex>

namespace oasis {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;  // waves per workgroup of attn_pv_kernel (attn_kernel: 4 or 8)
constexpr int kThreads = 64 * kWaves;
constexpr int kVecPerBlock = (int)(kBlockBytes / 16);  // uint4 per K+V block (512)
constexpr float kLn2 = 0.693147180559945309f;

struct AttnArgs {
    const uint16_t *q;
    const uint16_t *kv;
    int P;
    const int32_t *tbl_slot;
    const int32_t *tbl_block;
    const int32_t *tbl_n;
    int T;
    const int32_t *ctx_len;
    float scale_log2;  // sm_scale * log2(e)
    int H_q, H_kv, n_q, n_split;
    uint16_t *out;
    float *lse;
    float *ws;
};

__device__ __forceinline__ float exp2_(float x) { return __builtin_amdgcn_exp2f(x); }

// A wave's table entries i0 + wave + W * k (k < nk), W the workgroup's
// waves: up to 64 at a time sit in the lanes (one load), with a mask of the
// valid ones (slot in [0, P), block in [0, nb)), so the loop takes (slot,
// block) from a lane rather than reading memory before each block's loads.
struct TableCursor {
    const int32_t *ts, *tb;
    int base, stride, nk, P, nb, lane;
    int slot = -1, blk = -1, chunk = 0;
    unsigned long long mask = 0;

    __device__ void load(int c) {
        chunk = c;
        const int k = c + lane;
        int s = -1, b = -1;
        if (k < nk) {
            s = ts[base + k * stride];
            b = tb[base + k * stride];
        }
        slot = s;
        blk = b;
        mask = __ballot(k < nk && s >= 0 && s < P && b >= 0 && b < nb);
    }
    // next valid entry (wave-uniform): its slot and block; false at the end
    __device__ bool next(int &s, int &b) {
        for (;;) {
            if (mask) {
                const int bit = __ffsll((long long)mask) - 1;
                mask &= mask - 1;
                s = __builtin_amdgcn_readlane(slot, bit);
                b = __builtin_amdgcn_readlane(blk, bit);
                return true;
            }
            if (chunk + 64 >= nk) return false;
            load(chunk + 64);
        }
    }
};

// GP: columns compiled in (a power of two >= n_q * G, at most 8); G = H_q /
// H_kv at run time.  W: waves per workgroup (4 or 8).  Waves per SIMD the
// kernel is compiled for: four for up to four columns (1024 workgroups of the
// 8-KV-head layers at batch 128 then fit the 256 compute units in one round);
// eight columns need more registers: at least two (166 registers currently
// fit three).  More columns run in attn_pv_kernel below.
template <int GP>
constexpr int attn_waves_per_simd() { return GP <= 4 ? 4 : 2; }

template <int GP, int W>
__global__ __launch_bounds__(64 * W, attn_waves_per_simd<GP>()) void attn_kernel(AttnArgs a) {
    constexpr int kWg = 64 * W;  // threads
    __shared__ float p_lds[W][17][16];  // per wave: p[token][head]; row 16 = rescale
    // Q^T in the MFMA B layout, one 16-byte chunk per (head slot, 8 dims);
    // rows padded by 16 bytes so the 16 head slots fall in distinct banks
    __shared__ uint4 q_lds[16][17];
    __shared__ float m_lds[W][16];
    __shared__ float l_lds[W][16];
    __shared__ float o_lds[W][GP][kD];

    const int rh = blockIdx.x;
    const int split = blockIdx.y;
    const int r = rh / a.H_kv;
    const int h = rh - r * a.H_kv;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 15;  // MFMA row / column index
    const int grp = lane >> 4;  // lane group 0..3
    const int G = a.H_q / a.H_kv;
    const int NC = a.n_q * G;  // columns in use

    const int ctx = a.ctx_len[r];
    const int nb = ctx <= 0 ? 0 : (ctx + kBs - 1) / kBs;
    int n = a.tbl_n[rh];
    n = n < 0 ? 0 : (n > a.T ? a.T : n);
    const int per = (n + a.n_split - 1) / a.n_split;
    const int i0 = split * per;
    const int i1 = min(n, i0 + per);

    // Q^T as the MFMA B operand: lane (col, grp) brings column `col`, dims
    // kk * 32 + grp * 8 + [0, 8) for k-step kk; staged once in LDS (columns
    // past n_q * G are zero) and read back per block, which keeps registers
    // for the loads in flight.  The query load, the table load and the first
    // block's loads are all issued before the query goes to LDS, so their
    // latencies overlap (183 against 190 us alone at batch 128 / 16K).
    const int qc = tid >> 4, qchunk = tid & 15;  // threads 0..255: 16 columns x 16 chunks
    uint4 qv = make_uint4(0, 0, 0, 0);
    if (qc < NC) {  // NC <= 16, so only threads below 256
        const int qi = qc / G, g = qc - qi * G;
        qv = reinterpret_cast<const uint4 *>(a.q + (((size_t)r * a.n_q + qi) * a.H_q + (size_t)h * G + g) * kD)[qchunk];
    }

    const int32_t *ts = a.tbl_slot + (size_t)rh * a.T;
    const int32_t *tb = a.tbl_block + (size_t)rh * a.T;
    const uint4 *pool = reinterpret_cast<const uint4 *>(a.kv) + (size_t)rh * a.P * kVecPerBlock;

    TableCursor cur{ts, tb, i0 + wave, W, i1 - i0 - wave > 0 ? (i1 - i0 - wave + W - 1) / W : 0, a.P, nb, lane};
    cur.load(0);
    // next valid entry (wave-uniform); nullptr at the end
    auto next_valid = [&](int &blk) -> const uint4 * {
        int s;
        return cur.next(s, blk) ? pool + (size_t)s * kVecPerBlock : nullptr;
    };
    auto load = [&](const uint4 *src, uint4 (&kr)[4], uint4 (&vr)[4]) {
#pragma unroll
        for (int kk = 0; kk < 4; kk++) kr[kk] = src[col * 16 + kk * 4 + grp];
#pragma unroll
        for (int qq = 0; qq < 4; qq++) vr[qq] = src[256 + (qq * 4 + grp) * 16 + col];
    };

    int blk_c = 0;
    const uint4 *src_c = next_valid(blk_c);
    uint4 kc[4], vc[4];
    if (src_c) load(src_c, kc, vc);

    if (tid < 256) q_lds[qc][qchunk] = qv;
    __syncthreads();

    float acc[GP][8];
#pragma unroll
    for (int g = 0; g < GP; g++)
#pragma unroll
        for (int e = 0; e < 8; e++) acc[g][e] = 0.f;
    float m_run = -INFINITY, l_run = 0.f;

    float(*pl)[16] = p_lds[wave];
    while (src_c) {
        int blk_n = 0;
        const uint4 *src_n = next_valid(blk_n);
        uint4 kn[4], vn[4];
        if (src_n) load(src_n, kn, vn);

        // logits of column `col` for tokens 4 * grp + [0, 4)
        f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < 4; kk++)
            c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kc[kk]),
                                                         __builtin_bit_cast(bf16x8, q_lds[col][kk * 4 + grp]), c,
                                                         0, 0, 0);
        const int valid = ctx - blk_c * kBs;
        float sv[4];
#pragma unroll
        for (int t = 0; t < 4; t++) sv[t] = (4 * grp + t < valid) ? c[t] * a.scale_log2 : -INFINITY;
        float mx = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float m_new = fmaxf(m_run, mx);
        const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
        const float alpha = exp2_(m_run - m_use);
        float psum = 0.f;
#pragma unroll
        for (int t = 0; t < 4; t++) {
            const float p = exp2_(sv[t] - m_use);
            pl[4 * grp + t][col] = p;
            psum += p;
        }
        l_run = l_run * alpha + psum;
        // the accumulators need rescaling only if some column's running max
        // moved (otherwise alpha is exactly 1, or 0 on still-zero sums)
        const bool moved = __ballot(m_new != m_run) != 0;
        m_run = m_new;
        if (grp == 0) pl[16][col] = alpha;
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

        // rows past the context get p = 0, but 0 * V is NaN when the pool's
        // padding holds NaN or Inf: their V words are zeroed instead
        if (valid < kBs) {
#pragma unroll
            for (int qq = 0; qq < 4; qq++)
                if (qq * 4 + grp >= valid) vc[qq] = make_uint4(0, 0, 0, 0);
        }
        if (moved) {
#pragma unroll
            for (int g = 0; g < GP; g++) {
                const float al = pl[16][g];
#pragma unroll
                for (int e = 0; e < 8; e++) acc[g][e] *= al;
            }
        }
#pragma unroll
        for (int qq = 0; qq < 4; qq++) {
            const int t = qq * 4 + grp;
            const uint32_t w[4] = {vc[qq].x, vc[qq].y, vc[qq].z, vc[qq].w};
            float v[8];
#pragma unroll
            for (int e = 0; e < 4; e++) {
                v[2 * e] = bf16_lo(w[e]);
                v[2 * e + 1] = bf16_hi(w[e]);
            }
#pragma unroll
            for (int g = 0; g < GP; g++) {
                const float p = pl[t][g];
#pragma unroll
                for (int e = 0; e < 8; e++) acc[g][e] = fmaf(p, v[e], acc[g][e]);
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

        if (!src_n) break;
        // the entry just prefetched becomes current
        src_c = src_n;
        blk_c = blk_n;
#pragma unroll
        for (int x = 0; x < 4; x++) {
            kc[x] = kn[x];
            vc[x] = vn[x];
        }
    }

    // sum the four token groups of this wave
    l_run += __shfl_xor(l_run, 16);
    l_run += __shfl_xor(l_run, 32);
#pragma unroll
    for (int g = 0; g < GP; g++)
#pragma unroll
        for (int e = 0; e < 8; e++) {
            float x = acc[g][e];
            x += __shfl_xor(x, 16);
            x += __shfl_xor(x, 32);
            acc[g][e] = x;
        }
    if (grp == 0) {
#pragma unroll
        for (int g = 0; g < GP; g++)
#pragma unroll
            for (int e = 0; e < 8; e++) o_lds[wave][g][col * 8 + e] = acc[g][e];
        m_lds[wave][col] = m_run;
        l_lds[wave][col] = l_run;
    }
    __syncthreads();

    // merge the waves; one thread per (column, dim)
    for (int idx = tid; idx < NC * kD; idx += kWg) {
        const int g = idx / kD, d = idx - g * kD;  // g: column
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < W; w++) M = fmaxf(M, m_lds[w][g]);
        float o = 0.f, L = 0.f;
        if (M != -INFINITY) {
#pragma unroll
            for (int w = 0; w < W; w++) {
                const float mw = m_lds[w][g];
                const float f = (mw == -INFINITY) ? 0.f : exp2_(mw - M);
                o += f * o_lds[w][g][d];
                L += f * l_lds[w][g];
            }
        }
        const int qi = g / G;
        const size_t row = ((size_t)r * a.n_q + qi) * a.H_q + (size_t)h * G + (g - qi * G);
        if (a.n_split == 1) {
            a.out[row * kD + d] = f32_to_bf16(L > 0.f ? o / L : 0.f);
            if (d == 0 && a.lse)
                a.lse[row] = (M == -INFINITY || !(L > 0.f)) ? -INFINITY : (M + __log2f(L)) * kLn2;
        } else {
            float *part = a.ws + (row * a.n_split + split) * (kD + 2);
            part[d] = o;
            if (d == 0) {
                part[kD] = M;
                part[kD + 1] = L;
            }
        }
    }
}

// V^T tile of one block in LDS, per wave: [128 dims][16 tokens + 4 pad]
// halfwords, so that a lane's four tokens of one dim are 8 aligned bytes.
constexpr int kVtStride = 20;
constexpr int kVtBytes = kD * kVtStride * 2;                 // 5 KiB per wave
constexpr int kOBytes = 16 * kD * 4;                          // 8 KiB per wave
constexpr int kScratchBytes = kWaves * (kVtBytes > kOBytes ? kVtBytes : kOBytes);

typedef short s16x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kThreads, 4) void attn_pv_kernel(AttnArgs a) {
    // Q^T in the MFMA B layout, one 16-byte chunk per (column, 8 dims); rows
    // padded by 16 bytes so the 16 columns fall in distinct banks
    __shared__ uint4 q_lds[16][17];
    __shared__ float m_lds[kWaves][16];
    __shared__ float l_lds[kWaves][16];
    // per wave: V^T of the current block inside the loop, then the wave's
    // unnormalised output [16 columns][128 dims] for the merge
    __shared__ __attribute__((aligned(16))) unsigned char scratch[kScratchBytes];

    const int rh = blockIdx.x;
    const int split = blockIdx.y;
    const int r = rh / a.H_kv;
    const int h = rh - r * a.H_kv;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int col = lane & 15;  // MFMA row / column index
    const int grp = lane >> 4;  // lane group 0..3
    const int G = a.H_q / a.H_kv;
    const int NC = a.n_q * G;  // columns in use

    const int ctx = a.ctx_len[r];
    const int nb = ctx <= 0 ? 0 : (ctx + kBs - 1) / kBs;
    int n = a.tbl_n[rh];
    n = n < 0 ? 0 : (n > a.T ? a.T : n);
    const int per = (n + a.n_split - 1) / a.n_split;
    const int i0 = split * per;
    const int i1 = min(n, i0 + per);

    // Q^T as the MFMA B operand: lane (col, grp) brings column `col`, dims
    // kk * 32 + grp * 8 + [0, 8) for k-step kk; staged once in LDS (columns
    // past n_q * G are zero) and read back per block, which keeps registers
    // for the loads in flight.  As in attn_kernel, the query, table and first
    // block loads are issued together before the query goes to LDS.
    const int qc = tid >> 4, qchunk = tid & 15;  // 256 threads = 16 columns x 16 chunks
    uint4 qv = make_uint4(0, 0, 0, 0);
    if (qc < NC) {
        const int qi = qc / G, g = qc - qi * G;
        qv = reinterpret_cast<const uint4 *>(a.q + (((size_t)r * a.n_q + qi) * a.H_q + (size_t)h * G + g) * kD)[qchunk];
    }

    const int32_t *ts = a.tbl_slot + (size_t)rh * a.T;
    const int32_t *tb = a.tbl_block + (size_t)rh * a.T;
    const uint4 *pool = reinterpret_cast<const uint4 *>(a.kv) + (size_t)rh * a.P * kVecPerBlock;
    uint16_t(*vt)[kVtStride] = reinterpret_cast<uint16_t(*)[kVtStride]>(scratch + wave * kVtBytes);

    TableCursor cur{ts, tb, i0 + wave, kWaves, i1 - i0 - wave > 0 ? (i1 - i0 - wave + kWaves - 1) / kWaves : 0, a.P,
                    nb, lane};
    cur.load(0);
    // next valid entry (wave-uniform); nullptr at the end
    auto next_valid = [&](int &blk) -> const uint4 * {
        int s;
        return cur.next(s, blk) ? pool + (size_t)s * kVecPerBlock : nullptr;
    };
    auto load = [&](const uint4 *src, uint4 (&kr)[4], uint4 (&vr)[4]) {
#pragma unroll
        for (int kk = 0; kk < 4; kk++) kr[kk] = src[col * 16 + kk * 4 + grp];
#pragma unroll
        for (int qq = 0; qq < 4; qq++) vr[qq] = src[256 + (qq * 4 + grp) * 16 + col];
    };

    int blk_c = 0;
    const uint4 *src_c = next_valid(blk_c);
    uint4 kc[4], vc[4];
    if (src_c) load(src_c, kc, vc);

    q_lds[qc][qchunk] = qv;
    __syncthreads();

    // output accumulator in the MFMA C layout: acc[tt][e] = O^T[dim tt * 16 +
    // 4 * grp + e][column col], so every value of a lane belongs to its own
    // column and the rescale needs no exchange
    f32x4 acc[8];
#pragma unroll
    for (int tt = 0; tt < 8; tt++) acc[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.f;

    while (src_c) {
        int blk_n = 0;
        const uint4 *src_n = next_valid(blk_n);
        uint4 kn[4], vn[4];
        if (src_n) load(src_n, kn, vn);

        // V^T into this wave's LDS tile: lane (col, grp) holds token
        // qq * 4 + grp, dims col * 8 + [0, 8) of vc[qq]; rows past the
        // context go in as zeros (their p is 0, but 0 * NaN or 0 * Inf
        // padding would not be)
        const int valid = ctx - blk_c * kBs;
#pragma unroll
        for (int qq = 0; qq < 4; qq++) {
            const bool keep = qq * 4 + grp < valid;
            const uint32_t w[4] = {keep ? vc[qq].x : 0u, keep ? vc[qq].y : 0u, keep ? vc[qq].z : 0u,
                                   keep ? vc[qq].w : 0u};
#pragma unroll
            for (int e = 0; e < 4; e++) {
                vt[col * 8 + 2 * e][qq * 4 + grp] = (uint16_t)(w[e] & 0xffffu);
                vt[col * 8 + 2 * e + 1][qq * 4 + grp] = (uint16_t)(w[e] >> 16);
            }
        }

        // logits of column `col` for tokens 4 * grp + [0, 4)
        f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < 4; kk++)
            c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kc[kk]),
                                                         __builtin_bit_cast(bf16x8, q_lds[col][kk * 4 + grp]), c,
                                                         0, 0, 0);
        float sv[4];
#pragma unroll
        for (int t = 0; t < 4; t++) sv[t] = (4 * grp + t < valid) ? c[t] * a.scale_log2 : -INFINITY;
        float mx = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float m_new = fmaxf(m_run, mx);
        const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
        const float alpha = exp2_(m_run - m_use);
        // p goes to the matrix cores as two bf16 parts, p = hi + lo with
        // hi = bf16(p) and lo = bf16(p - hi), so the weights keep ~17
        // significant bits (one bf16 alone, 2^-9, is too coarse for outputs
        // near zero) and each bf16 x bf16 product is exact in the fp32
        // accumulator
        s16x4 pb_hi, pb_lo;
        float psum = 0.f;
#pragma unroll
        for (int t = 0; t < 4; t++) {
            const float p = exp2_(sv[t] - m_use);
            const uint16_t hi = f32_to_bf16(p);
            pb_hi[t] = (short)hi;
            pb_lo[t] = (short)f32_to_bf16(p - __uint_as_float((uint32_t)hi << 16));
            psum += p;
        }
        l_run = l_run * alpha + psum;
        m_run = m_new;

        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

        // p . V on the matrix cores: O^T[dims][columns] += V^T[dims][tokens]
        // P[tokens][columns]; A = the V^T tile rows tt * 16 + col, tokens
        // 4 * grp + [0, 4); B = P (hi, then lo), already in the B layout
        // (the logits' output layout)
#pragma unroll
        for (int tt = 0; tt < 8; tt++) {
            const uint2 av = *reinterpret_cast<const uint2 *>(&vt[tt * 16 + col][4 * grp]);
            const s16x4 va = __builtin_bit_cast(s16x4, av);
            acc[tt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, pb_hi, acc[tt] * alpha, 0, 0, 0);
            acc[tt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, pb_lo, acc[tt], 0, 0, 0);
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

        if (!src_n) break;
        // the entry just prefetched becomes current
        src_c = src_n;
        blk_c = blk_n;
#pragma unroll
        for (int x = 0; x < 4; x++) {
            kc[x] = kn[x];
            vc[x] = vn[x];
        }
    }

    // the denominator: sum the four token groups of the column
    l_run += __shfl_xor(l_run, 16);
    l_run += __shfl_xor(l_run, 32);
    __syncthreads();  // every wave is done with its V^T tile
    float(*o_lds)[kD] = reinterpret_cast<float(*)[kD]>(scratch + wave * kOBytes);
#pragma unroll
    for (int tt = 0; tt < 8; tt++)
#pragma unroll
        for (int e = 0; e < 4; e++) o_lds[col][tt * 16 + 4 * grp + e] = acc[tt][e];
    if (grp == 0) {
        m_lds[wave][col] = m_run;
        l_lds[wave][col] = l_run;
    }
    __syncthreads();

    // merge the waves; one thread per (column, dim)
    for (int idx = tid; idx < NC * kD; idx += kThreads) {
        const int g = idx / kD, d = idx - g * kD;  // g: column
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < kWaves; w++) M = fmaxf(M, m_lds[w][g]);
        float o = 0.f, L = 0.f;
        if (M != -INFINITY) {
#pragma unroll
            for (int w = 0; w < kWaves; w++) {
                const float mw = m_lds[w][g];
                const float f = (mw == -INFINITY) ? 0.f : exp2_(mw - M);
                o += f * reinterpret_cast<const float(*)[kD]>(scratch + w * kOBytes)[g][d];
                L += f * l_lds[w][g];
            }
        }
        const int qi = g / G;
        const size_t row = ((size_t)r * a.n_q + qi) * a.H_q + (size_t)h * G + (g - qi * G);
        if (a.n_split == 1) {
            a.out[row * kD + d] = f32_to_bf16(L > 0.f ? o / L : 0.f);
            if (d == 0 && a.lse)
                a.lse[row] = (M == -INFINITY || !(L > 0.f)) ? -INFINITY : (M + __log2f(L)) * kLn2;
        } else {
            float *part = a.ws + (row * a.n_split + split) * (kD + 2);
            part[d] = o;
            if (d == 0) {
                part[kD] = M;
                part[kD + 1] = L;
            }
        }
    }
}

__global__ __launch_bounds__(kD) void attn_combine_kernel(const float *__restrict__ ws, int n_split,
                                                          uint16_t *__restrict__ out,
                                                          float *__restrict__ lse) {
    const size_t row = blockIdx.x;
    const int d = threadIdx.x;
    const float *base = ws + row * n_split * (kD + 2);
    float M = -INFINITY;
    for (int s = 0; s < n_split; s++) M = fmaxf(M, base[s * (kD + 2) + kD]);
    float o = 0.f, L = 0.f;
    if (M != -INFINITY) {
        for (int s = 0; s < n_split; s++) {
            const float ms = base[s * (kD + 2) + kD];
            const float f = (ms == -INFINITY) ? 0.f : exp2_(ms - M);
            o += f * base[s * (kD + 2) + d];
            L += f * base[s * (kD + 2) + kD + 1];
        }
    }
    out[row * kD + d] = f32_to_bf16(L > 0.f ? o / L : 0.f);
    if (d == 0 && lse) lse[row] = (M == -INFINITY || !(L > 0.f)) ? -INFINITY : (M + __log2f(L)) * kLn2;
}

template <int GP>
hipError_t launch_g(const oasis_dims &d, const AttnArgs &a, int waves, hipStream_t s, hipEvent_t done) {
    dim3 grid((unsigned)(d.B * d.H_kv), (unsigned)a.n_split);
    if (waves == 8)
        hipExtLaunchKernelGGL(attn_kernel<GP, 8>, grid, dim3(64 * 8), 0, s, nullptr, done, 0, a);
    else
        hipExtLaunchKernelGGL(attn_kernel<GP, 4>, grid, dim3(64 * 4), 0, s, nullptr, done, 0, a);
    return hipGetLastError();
}

}  // namespace

// Split-K partials of oasis_sparse_decode_attn_static: a fixed array in
// device memory for callers that cannot allocate.  Each device the library
// runs on holds its own copy until the process ends.  In host code `scratch`
// names a host-side stand-in, not the device array: kernels get the address
// that hipGetSymbolAddress returns for the current device.
constexpr size_t kStaticScratchBytes = size_t(8) << 20;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

size_t attn_static_scratch_bytes() { return kStaticScratchBytes; }

// Device address of this device's `scratch`, looked up once per device (with
// that device current) and kept.
hipError_t attn_static_scratch(void **ptr) {
    static std::mutex mu;
    static void *addr[kMaxDevices] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lk(mu);
    if (!addr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        addr[dev] = p;
    }
    *ptr = addr[dev];
    return hipSuccess;
}

// The launch shape aims at two waves per SIMD (8 per compute unit) over the
// (request, KV head) pairs: one split of four-wave workgroups when the pairs
// alone fill the machine; otherwise eight-wave workgroups (VALU kernel) over
// as few splits as reach the target, each split keeping at least four table
// entries per wave (two in attn_pv_kernel's four-wave workgroups).  A split
// adds a combine kernel and its partial outputs,
// which in the pipeline cost more than wider workgroups: Qwen3-8B in HBM at
// batch 32 (256 pairs, G = 4), one split of eight waves against two of four,
// 462-466k against 413k tok/s (alone 50.0 against 52.1 us); the ragged
// 32B-class layer (128 pairs, G = 8), two splits of eight waves against four
// of four, alone 33.1 against 35.9 us.  Four-wave workgroups stay faster
// wherever they fill the machine (the reasoning layer, 512 pairs: 356k
// against 334k with eight waves).  With few table entries the combine costs
// more than a second split saves: one request of 8 / 2 heads over 32 blocks,
// 60.2k tok/s with one split against 51.4k with two (two entries per wave).
int attn_waves(const oasis_dims &d, int n_q, int T, int splits) {
    if (n_q * (d.H_q / d.H_kv) > 8) return kWaves;  // attn_pv_kernel
    const long pairs = (long)d.B * d.H_kv;
    const long target = 8L * device_cu_count();
    return pairs * splits * 4 < target && (long)T >= 16L * splits ? 8 : 4;
}

int attn_splits(const oasis_dims &d, int n_q, int T, int n_split) {
    if (n_split > 0) return n_split < 64 ? n_split : 64;
    const long pairs = (long)d.B * d.H_kv;
    if (pairs <= 0 || T <= 0) return 1;
    const long target = 8L * device_cu_count();  // waves: two per SIMD
    if (pairs * 4 >= target) return 1;
    // eight-wave workgroups for the VALU kernel (a split keeps four table
    // entries per wave), four for attn_pv_kernel (two per wave)
    const bool valu = n_q * (d.H_q / d.H_kv) <= 8;
    const long wg_waves = valu ? 8 : 4;
    long s = (target + wg_waves * pairs - 1) / (wg_waves * pairs);
    const long cap = valu ? T / 32 : (T + 7) / 8;
    if (s > cap) s = cap;
    if (s > 64) s = 64;
    if (s < 1) s = 1;
    return (int)s;
}

size_t attn_ws_bytes(const oasis_dims &d, int n_q, int T, int n_split) {
    const int s = attn_splits(d, n_q, T, n_split);
    if (s <= 1) return 0;
    return (size_t)d.B * n_q * d.H_q * s * (kD + 2) * sizeof(float);
}

hipError_t launch_attn(const oasis_dims &d, int n_q, const uint16_t *q, const uint16_t *kv_pool, int P,
                       const int32_t *tbl_slot, const int32_t *tbl_block, const int32_t *tbl_n,
                       int T, const int32_t *ctx_len, float sm_scale, uint16_t *out, float *lse,
                       float *ws, int n_split, hipStream_t s, hipEvent_t done) {
    AttnArgs a;
    a.q = q;
    a.kv = kv_pool;
    a.P = P;
    a.tbl_slot = tbl_slot;
    a.tbl_block = tbl_block;
    a.tbl_n = tbl_n;
    a.T = T;
    a.ctx_len = ctx_len;
    a.scale_log2 = sm_scale * 1.4426950408889634f;
    a.H_q = d.H_q;
    a.H_kv = d.H_kv;
    a.n_q = n_q;
    a.n_split = n_split;
    a.out = out;
    a.lse = lse;
    a.ws = ws;
    const int NC = n_q * (d.H_q / d.H_kv);
    const int waves = attn_waves(d, n_q, T, n_split);
    // `done` on the last kernel (the combine, if any)
    hipEvent_t first = n_split <= 1 ? done : nullptr;
    hipError_t e;
    if (NC <= 1) e = launch_g<1>(d, a, waves, s, first);
    else if (NC <= 2) e = launch_g<2>(d, a, waves, s, first);
    else if (NC <= 4) e = launch_g<4>(d, a, waves, s, first);
    else if (NC <= 8) e = launch_g<8>(d, a, waves, s, first);
    else {
        dim3 grid((unsigned)(d.B * d.H_kv), (unsigned)n_split);
        hipExtLaunchKernelGGL(attn_pv_kernel, grid, dim3(kThreads), 0, s, nullptr, first, 0, a);
        e = hipGetLastError();
    }
    if (e != hipSuccess || n_split <= 1) return e;
    hipExtLaunchKernelGGL(attn_combine_kernel, dim3((unsigned)(d.B * n_q * d.H_q)), dim3(kD), 0, s, nullptr,
                          done, 0, ws, n_split, out, lse);
    return hipGetLastError();
}

}  // namespace oasis
