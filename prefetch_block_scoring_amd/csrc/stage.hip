// KV selection and staging into the HBM working set.
//
// OasisKV (arXiv 2608.08097), paperlayer summary, section 4.  Each step, a
// (request, KV head) pair's predicted blocks that already sit in its HBM
// working set stay there; up to C of the others are brought in from the host
// copy of the cache, each taking the place of the resident block that was
// predicted longest ago once the budget is full.
//
// plan kernel: one workgroup per (request, KV head) updates that pair's slot
//   table in LDS (the whole state is a few hundred integers) and emits the
//   copy plan and the next attention table.  Admitted blocks go to slots that
//   were free before this step, never to a slot evicted in this step, so the
//   attention that still reads the previous table is not raced; with
//   S >= K_b + C slots there are always enough of them.
// prefix kernel: packed positions of the admits (the order in which a copy
//   engine stages them).
// Copy engines (the pinned pool's blocks to their slots):
//   DMA: the host reads the plan back, packs the admitted blocks into a
//     pinned staging buffer on worker threads, and one hipMemcpyAsync moves
//     them over PCIe; the scatter kernel then places them.  The DMA engines
//     leave the compute units and their memory path to the HBM-bound kernels
//     that run at the same time.
//   kernel: a gather kernel of a few workgroups reads the pool through its device
//     mapping.  No host work, but its PCIe reads hold the memory path and
//     slow concurrent HBM-bound kernels down.
#include "oasis_internal.h"

namespace oasis {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
// the plan's bounds (checked at the entry points): K_sel <= 1024 predicted
// ids and S <= 2048 slots per (request, KV head)
constexpr int kMaxIdsPerThread = 1024 / kThreads;
constexpr int kMaxSlotsPerThread = 2048 / kThreads;

// Workgroups of one zero-copy gather.  Its PCIe reads wait microseconds and,
// while they wait, slow the kernels that run beside them.  When a step can
// admit thousands of blocks (the Qwen3-8B layer at batch 128: 1024 pairs x C)
// the layer pipeline runs two gathers at once, and 24 workgroups each keep
// the link at the pinned-memcpy rate (12 or 16: 1-2% slower; at a cap of two
// blocks 16 is 17% slower).  With at most kFewAdmits admits per step, 16
// leave more compute units to the latency-bound kernels beside them: the
// ragged 32B-class layer (128 pairs, C = 6) runs at 176k tok/s against
// 171-173k with 24 (12: 154-156k, 20: 173-176k).
constexpr int kGatherWgs = 24;
constexpr int kGatherWgsFew = 16;
constexpr long kFewAdmits = 1024;

__device__ __forceinline__ int wg_exclusive_scan(int v, int *tmp, int *total) {
    const int lane = threadIdx.x % 64, wave = threadIdx.x / 64;
    int inc = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(inc, o, 64);
        if (lane >= o) inc += y;
    }
    if (lane == 63) tmp[wave] = inc;
    __syncthreads();
    int before = 0, all = 0;
#pragma unroll
    for (int w = 0; w < kWaves; w++) {
        const int t = tmp[w];
        before += (w < wave) ? t : 0;
        all += t;
    }
    __syncthreads();
    *total = all;
    return before + inc - v;
}

// Compact the indices i in [0, n) with flag(i) into out[] in ascending order;
// returns the count.  Thread t owns the contiguous range [t*per, t*per + per).
template <class F>
__device__ int wg_compact(int n, F flag, int *out, int *tmp) {
    const int per = (n + kThreads - 1) / kThreads;
    const int lo = min(n, (int)threadIdx.x * per), hi = min(n, lo + per);
    int c = 0;
    for (int i = lo; i < hi; i++) c += flag(i) ? 1 : 0;
    int total;
    int pos = wg_exclusive_scan(c, tmp, &total);
    for (int i = lo; i < hi; i++)
        if (flag(i)) out[pos++] = i;
    __syncthreads();
    return total;
}

struct PlanArgs {
    const int32_t *sel;
    const int32_t *n_sel;
    int K_sel;
    const float *scores;
    int K_b, C, S, step;
    int32_t *slot_block;
    int32_t *slot_stamp;
    const int32_t *ctx_len;
    int32_t *tbl_slot;
    int32_t *tbl_block;
    int32_t *tbl_n;
    int32_t *plan;
    int H_kv, NB_max;
};

__global__ __launch_bounds__(kThreads) void stage_plan_kernel(PlanArgs a) {
    extern __shared__ int smem[];
    const int S = a.S, K = a.K_sel;
    int *sb = smem;              // [S] block held by each slot (-1 free)
    int *st = sb + S;            // [S] stamp of each slot
    int *in_p = st + S;          // [S] 1 if the slot's block is predicted
    int *victim = in_p + S;      // [S] 1 if evicted this step
    int *list_s = victim + S;    // [S] scratch list over slots
    int *pv = list_s + S;        // [K] valid predicted ids, ascending
    int *res_of = pv + K;        // [K] slot holding pv[k], -1 if not resident
    int *cand = res_of + K;      // [K] indices k of non-resident predicted blocks
    uint32_t *ckey = (uint32_t *)(cand + K);  // [K] rank keys of the candidates
    int *adm = (int *)(ckey + K);            // [K] admitted block per admission rank
    __shared__ int tmp[kWaves];

    const int rh = blockIdx.x;
    const int r = rh / a.H_kv;
    const int tid = threadIdx.x;
    const int32_t *P = a.sel + (size_t)rh * K;
    int32_t *slot_block = a.slot_block + (size_t)rh * S;
    int32_t *slot_stamp = a.slot_stamp + (size_t)rh * S;
    const float *sc = a.scores + (size_t)rh * a.NB_max;

    // Every read that needs nothing else is issued first, so their latencies
    // overlap: the context length, the selection count, this thread's
    // predicted ids (a contiguous range of the K, with the one before it) and
    // its slots of the table.  Indices are clamped into the rows; the copies
    // past their ends are never used.
    const int ctx = a.ctx_len[r];
    int np = a.n_sel[rh];
    const int per = (K + kThreads - 1) / kThreads;  // <= kMaxIdsPerThread
    const int lo = min(K, tid * per);
    int pid[kMaxIdsPerThread + 1];  // P[lo - 1 + u]
#pragma unroll
    for (int u = 0; u <= kMaxIdsPerThread; u++) pid[u] = P[min(max(lo - 1 + u, 0), K - 1)];
    int sbr[kMaxSlotsPerThread], str[kMaxSlotsPerThread];  // slot tid + u * kThreads
#pragma unroll
    for (int u = 0; u < kMaxSlotsPerThread; u++) {
        const int sl = min(tid + u * kThreads, S - 1);
        sbr[u] = slot_block[sl];
        str[u] = slot_stamp[sl];
    }
    const int nb = n_blocks_of(ctx, a.NB_max);
    np = np < 0 ? 0 : (np > K ? K : np);

    // 1. predicted ids: keep those in range and strictly ascending (rows from
    //    top-K are), compacted into pv in order
    int npv;
    {
        const int hi = min(np, lo + per);
        int c = 0;
#pragma unroll
        for (int u = 0; u < kMaxIdsPerThread; u++) {
            const int i = lo + u, p = pid[u + 1];
            c += (i < hi && p >= 0 && p < nb && (i == 0 || p > pid[u])) ? 1 : 0;
        }
        int pos = wg_exclusive_scan(c, tmp, &npv);
#pragma unroll
        for (int u = 0; u < kMaxIdsPerThread; u++) {
            const int i = lo + u, p = pid[u + 1];
            if (i < hi && p >= 0 && p < nb && (i == 0 || p > pid[u])) pv[pos++] = p;
        }
    }
    for (int k = tid; k < npv; k += kThreads) res_of[k] = -1;
    // 2. slot table; anything outside [0, nb) counts as free
#pragma unroll
    for (int u = 0; u < kMaxSlotsPerThread; u++) {
        const int sl = tid + u * kThreads;
        if (sl < S) {
            int b = sbr[u];
            if (b < 0 || b >= nb) b = -1;
            sb[sl] = b;
            st[sl] = b >= 0 ? str[u] : -1;
            in_p[sl] = 0;
            victim[sl] = 0;
        }
    }
    __syncthreads();
    // 3. resident predicted blocks: binary search of each held block in pv
    for (int s = tid; s < S; s += kThreads) {
        const int b = sb[s];
        if (b < 0) continue;
        int lo = 0, hi = npv;
        while (lo < hi) {
            const int mid = (lo + hi) >> 1;
            if (pv[mid] < b) lo = mid + 1; else hi = mid;
        }
        if (lo < npv && pv[lo] == b) {
            in_p[s] = 1;
            res_of[lo] = s;
            st[s] = a.step;
        }
    }
    __syncthreads();
    // 4. candidates for admission, counts
    const int nc = wg_compact(npv, [&](int k) { return res_of[k] < 0; }, cand, tmp);
    for (int i = tid; i < nc; i += kThreads) ckey[i] = rank_key(sc[pv[cand[i]]]);
    int n_res, n_elig;
    {
        int c1 = 0, c2 = 0;
        for (int s = tid; s < S; s += kThreads) {
            c1 += sb[s] >= 0;
            c2 += sb[s] >= 0 && !in_p[s];
        }
        int t;
        wg_exclusive_scan(c1, tmp, &n_res);
        wg_exclusive_scan(c2, tmp, &t);
        n_elig = t;
    }
    // free slots before this step's evictions, ascending
    const int nfree = wg_compact(S, [&](int s) { return sb[s] < 0; }, list_s, tmp);
    const int free_cap = max(0, a.K_b - n_res);
    int n_adm = min(a.C, nc);
    n_adm = min(n_adm, nfree);
    n_adm = min(n_adm, free_cap + n_elig);
    n_adm = max(n_adm, 0);
    const int need = max(0, n_adm - free_cap);

    // 5. admission ranks: (score desc, id asc) among candidates
    for (int i = tid; i < nc; i += kThreads) {
        const uint32_t ki = ckey[i];
        const int bi = pv[cand[i]];
        int rank = 0;
        for (int j = 0; j < nc; j++) {
            const uint32_t kj = ckey[j];
            rank += (kj > ki) || (kj == ki && pv[cand[j]] < bi);
        }
        if (rank < n_adm) adm[rank] = bi;
    }
    // 6. eviction ranks: (stamp asc, id asc) among resident, non-predicted
    for (int s = tid; s < S; s += kThreads) {
        const int b = sb[s];
        if (b < 0 || in_p[s]) continue;
        const int ts = st[s];
        int rank = 0;
        for (int u = 0; u < S; u++) {
            const int bu = sb[u];
            if (bu < 0 || in_p[u]) continue;
            rank += (st[u] < ts) || (st[u] == ts && bu < b);
        }
        victim[s] = rank < need;
    }
    __syncthreads();
    // 7. apply: evict, then place admits into the pre-step free slots
    int32_t *plan = a.plan + (size_t)rh * plan_row(a.C);
    for (int s = tid; s < S; s += kThreads) {
        if (victim[s]) {
            sb[s] = -1;
            st[s] = -1;
        }
    }
    __syncthreads();
    for (int i = tid; i < n_adm; i += kThreads) {
        const int s = list_s[i];
        sb[s] = adm[i];
        st[s] = a.step;
        plan[kPlanHead + 2 * i] = s;
        plan[kPlanHead + 2 * i + 1] = adm[i];
    }
    if (tid == 0) {
        plan[0] = n_adm;
        plan[1] = need;
        plan[2] = 0;
        plan[3] = nc - n_adm;  // deferred: predicted, not resident, not admitted
    }
    __syncthreads();
    for (int s = tid; s < S; s += kThreads) {
        slot_block[s] = sb[s];
        slot_stamp[s] = st[s];
    }
    // 8. next attention table: held slots, ascending
    const int nheld = wg_compact(S, [&](int s) { return sb[s] >= 0; }, list_s, tmp);
    const int nt = min(nheld, a.K_b);
    int32_t *ts = a.tbl_slot + (size_t)rh * a.K_b;
    int32_t *tb = a.tbl_block + (size_t)rh * a.K_b;
    for (int i = tid; i < a.K_b; i += kThreads) {
        ts[i] = i < nt ? list_s[i] : -1;
        tb[i] = i < nt ? sb[list_s[i]] : -1;
    }
    if (tid == 0) a.tbl_n[rh] = nt;
}

// Exclusive prefix of the admit counts over (r, h), written to each row's
// packed position, and the step's totals after the rows: admits, evictions,
// deferred admits and the pairs with any deferred.  With `accum` (device
// int64[4]) the same admits, evictions and deferred admits, and 1 for the
// step, are added to it.  One workgroup.
__global__ __launch_bounds__(1024) void stage_prefix_kernel(int32_t *__restrict__ plan, int row, int pairs,
                                                            unsigned long long *__restrict__ accum) {
    __shared__ int tmp[16];
    __shared__ int red[3][16];
    __shared__ int carry;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    if (tid == 0) carry = 0;
    __syncthreads();
    int n_ev = 0, n_def = 0, n_cap = 0;
    for (int base = 0; base < pairs; base += 1024) {
        const int rh = base + tid;
        int v = 0;
        if (rh < pairs) {
            const int32_t *p = plan + (size_t)rh * row;
            v = p[0];
            n_ev += p[1];
            n_def += p[3];
            n_cap += p[3] > 0;
        }
        int inc = v;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int y = __shfl_up(inc, o, 64);
            if (lane >= o) inc += y;
        }
        if (lane == 63) tmp[wave] = inc;
        __syncthreads();
        int before = carry, all = carry;
        for (int w = 0; w < 16; w++) {
            before += (w < wave) ? tmp[w] : 0;
            all += tmp[w];
        }
        if (rh < pairs) plan[(size_t)rh * row + 2] = before + inc - v;
        __syncthreads();
        if (tid == 0) carry = all;
        __syncthreads();
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        n_ev += __shfl_xor(n_ev, o, 64);
        n_def += __shfl_xor(n_def, o, 64);
        n_cap += __shfl_xor(n_cap, o, 64);
    }
    if (lane == 0) {
        red[0][wave] = n_ev;
        red[1][wave] = n_def;
        red[2][wave] = n_cap;
    }
    __syncthreads();
    if (tid == 0) {
        int ev = 0, def = 0, cap = 0;
        for (int w = 0; w < 16; w++) {
            ev += red[0][w];
            def += red[1][w];
            cap += red[2][w];
        }
        int32_t *tail = plan + (size_t)pairs * row;
        tail[0] = carry;
        tail[1] = ev;
        tail[2] = def;
        tail[3] = cap;
        if (accum) {
            atomicAdd(accum + 0, (unsigned long long)carry);
            atomicAdd(accum + 1, (unsigned long long)ev);
            atomicAdd(accum + 2, (unsigned long long)def);
            atomicAdd(accum + 3, 1ull);
        }
    }
}

// Packed positions: the admits of one step, numbered in (pair, admission)
// order; row[2] of each pair holds the position of its first admit (the
// exclusive prefix of the admit counts) and the total follows the rows.  A
// workgroup of the copy kernels takes a contiguous range of positions, finds
// the pair of its first position, and walks forward, so pairs with fewer
// admits than C cost nothing.

// The pair holding position k (0 <= k < total): the last pair whose first
// position is <= k, by binary search over the rows' positions (they are
// non-decreasing); -1 if even the first row starts after k.  Uniform across
// the workgroup.
__device__ int pair_of_position(const int32_t *__restrict__ plan, int row, int pairs, int k) {
    if (plan[2] > k) return -1;
    int lo = 0, hi = pairs - 1;
    while (lo < hi) {
        const int mid = lo + ((hi - lo + 1) >> 1);
        if (plan[(size_t)mid * row + 2] <= k) lo = mid;
        else hi = mid - 1;
    }
    return lo;
}

// Copy the blocks of positions [k0, k1): for each, the source returned by
// src_of(k, rh, block) into the admit's slot of pair rh.  pairs' admit counts are
// clamped to [0, C] and slots to [0, S); a pair index past the rows ends the
// walk.
template <class SrcOf>
__device__ void copy_positions(const int32_t *__restrict__ plan, int row, int pairs, int C, int S, int k0,
                               int k1, uint4 *__restrict__ ws_pool, SrcOf src_of) {
    constexpr int kVec = (int)(kBlockBytes / sizeof(uint4));  // 512
    if (k0 >= k1) return;
    int rh = pair_of_position(plan, row, pairs, k0);
    if (rh < 0) return;
    const int32_t *p = plan + (size_t)rh * row;
    int pos = p[2], n = min(max(p[0], 0), C);
    for (int k = k0; k < k1; k++) {
        while (k >= pos + n) {
            if (++rh >= pairs) return;
            p = plan + (size_t)rh * row;
            pos = p[2];
            n = min(max(p[0], 0), C);
        }
        const int i = k - pos;
        if (i < 0) continue;  // inconsistent plan: skip, never index past it
        const int slot = p[kPlanHead + 2 * i];
        const uint4 *src = src_of(k, rh, p[kPlanHead + 2 * i + 1]);
        if (slot < 0 || slot >= S || !src) continue;
        uint4 *dst = ws_pool + ((size_t)rh * S + slot) * kVec;
        const uint4 a = src[threadIdx.x];
        const uint4 b = src[threadIdx.x + 256];
        dst[threadIdx.x] = a;
        dst[threadIdx.x + 256] = b;
    }
}

// Zero-copy engine: kGatherWgs (kGatherWgsFew) workgroups split the step's packed positions
// into contiguous ranges; each thread keeps two 16-byte PCIe reads in flight
// per block.
__global__ __launch_bounds__(256) void stage_gather_kernel(
    const int32_t *__restrict__ plan, int row, int pairs, int C, const uint4 *__restrict__ host_pool,
    uint4 *__restrict__ ws_pool, int NB_max, int S) {
    constexpr int kVec = (int)(kBlockBytes / sizeof(uint4));
    const int total = (int)min((long)max(plan[(size_t)pairs * row], 0), (long)pairs * C);
    const int per = (total + gridDim.x - 1) / gridDim.x;
    const int k0 = min(total, (int)blockIdx.x * per), k1 = min(total, k0 + per);
    copy_positions(plan, row, pairs, C, S, k0, k1, ws_pool, [&](int, int rh, int blk) -> const uint4 * {
        if (blk < 0 || blk >= NB_max) return nullptr;
        return host_pool + ((size_t)rh * NB_max + blk) * kVec;
    });
}

// DMA engine, device half: the packed blocks of positions [lo, hi) sit in
// the device staging buffer in position order; copy each into its slot.
__global__ __launch_bounds__(256) void stage_scatter_kernel(
    const int32_t *__restrict__ plan, int row, int pairs, int C, const uint4 *__restrict__ staged, int lo,
    int hi, uint4 *__restrict__ ws_pool, int S) {
    constexpr int kVec = (int)(kBlockBytes / sizeof(uint4));
    const int total = (int)min((long)max(plan[(size_t)pairs * row], 0), (long)pairs * C);
    hi = min(hi, total);
    const int n = max(hi - lo, 0);
    const int per = (n + gridDim.x - 1) / gridDim.x;
    const int k0 = lo + min(n, (int)blockIdx.x * per), k1 = lo + min(n, (int)blockIdx.x * per + per);
    copy_positions(plan, row, pairs, C, S, k0, k1, ws_pool, [&](int k, int, int) -> const uint4 * {
        return staged + (size_t)(k - lo) * kVec;
    });
}

}  // namespace

size_t stage_plan_lds_bytes(int S, int K_sel) {
    return (size_t)(5 * S + 5 * K_sel) * sizeof(int);
}

hipError_t launch_stage_plan(const oasis_dims &d, const oasis_stage_args &a, hipStream_t s) {
    PlanArgs p;
    p.sel = a.sel;
    p.n_sel = a.n_sel;
    p.K_sel = a.K_sel;
    p.scores = a.scores;
    p.K_b = a.K_b;
    p.C = a.C;
    p.S = a.S;
    p.step = a.step;
    p.slot_block = a.slot_block;
    p.slot_stamp = a.slot_stamp;
    p.ctx_len = a.ctx_len;
    p.tbl_slot = a.tbl_slot;
    p.tbl_block = a.tbl_block;
    p.tbl_n = a.tbl_n;
    p.plan = a.plan;
    p.H_kv = d.H_kv;
    p.NB_max = d.NB_max;
    hipLaunchKernelGGL(stage_plan_kernel, dim3((unsigned)(d.B * d.H_kv)), dim3(kThreads),
                       stage_plan_lds_bytes(a.S, a.K_sel), s, p);
    return hipGetLastError();
}

hipError_t launch_stage_prefix(const oasis_dims &d, const oasis_stage_args &a, hipStream_t s,
                               hipEvent_t done) {
    hipExtLaunchKernelGGL(stage_prefix_kernel, dim3(1), dim3(1024), 0, s, nullptr, done, 0, a.plan,
                          plan_row(a.C), d.B * d.H_kv, reinterpret_cast<unsigned long long *>(a.stats_accum));
    return hipGetLastError();
}

hipError_t launch_stage_scatter(const oasis_dims &d, const oasis_stage_args &a, int lo, int hi,
                                hipStream_t s) {
    if (a.C <= 0 || hi <= lo) return hipSuccess;
    const int cap = 4 * device_cu_count();
    const int wgs = hi - lo < cap ? hi - lo : cap;
    hipLaunchKernelGGL(stage_scatter_kernel, dim3((unsigned)wgs), dim3(256), 0, s, a.plan, plan_row(a.C),
                       d.B * d.H_kv, a.C, reinterpret_cast<const uint4 *>(a.stage_dev), lo, hi,
                       reinterpret_cast<uint4 *>(a.ws_pool), a.S);
    return hipGetLastError();
}

hipError_t launch_stage_gather(const oasis_dims &d, const oasis_stage_args &a,
                               const void *host_pool_dev, hipStream_t s, hipEvent_t done) {
    if (a.C <= 0) return record_done(done, s);
    const long most = (long)d.B * d.H_kv * a.C;  // admits of the step are at most this many
    const int want = most <= kFewAdmits ? kGatherWgsFew : kGatherWgs;
    const int wgs = most < want ? (int)most : want;
    hipExtLaunchKernelGGL(stage_gather_kernel, dim3((unsigned)wgs), dim3(256), 0, s, nullptr, done, 0, a.plan,
                          plan_row(a.C), d.B * d.H_kv, a.C, reinterpret_cast<const uint4 *>(host_pool_dev),
                          reinterpret_cast<uint4 *>(a.ws_pool), d.NB_max, a.S);
    return hipGetLastError();
}

}  // namespace oasis
