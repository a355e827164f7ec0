/*
 * CPU oracle for the lookahead block-scoring decode path.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the package's smoke check and
 * the benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header, table or helper with the HIP library: it is a plain, slow, fp64
 * restatement of what the method computes, written step by step in the order
 * the OasisKV pages give (arXiv 2608.08097, "OasisKV: Scaling In-Decode KV
 * Cache Beyond HBM with Lookahead Sparse Prefetching"; the paperlayer summary,
 * section 4 "System Design", is the authority for every step here).
 *
 * The pages name the steps but print no formula; where they are silent this
 * file takes the plainest reading and says which one at the function.
 *
 * Conventions (the caller's arrays, row-major):
 *   bf16 values arrive as raw uint16_t bit patterns.
 *   q_look  [B][J][H_q][D]             lookahead (draft) queries
 *   q       [B][H_q][D]                attention query
 *   kv      [B][H_kv][NB_max][2][bs][D] K (index 0) then V (index 1) per block
 *   kminmax [B][H_kv][NB_max][2][D]    index 0 = coordinate-wise min, 1 = max
 *   ctx_len [B]; the request's blocks are 0 .. ceil(ctx_len/bs) - 1
 *   Query head g belongs to KV head g / (H_q / H_kv).
 *
 * Parity pins: every function is checked in the CPU test suite against
 * brute force, closed forms or invariants; see the test files for which.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

static double bf16_value(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

static int n_blocks_of(int32_t ctx, int bs)
{
    if (ctx <= 0) return 0;
    return (ctx + bs - 1) / bs;
}

/* ------------------------------------------------------------------------ */
/* Block summaries.                                                          */
/* Section 4: the prototype keeps, per block, the coordinate-wise minimum and */
/* maximum of the block's keys (two vectors instead of the block's keys).     */
/* Reading: only tokens inside the request's context count; blocks past the   */
/* context are left untouched.  A min or max of bf16 values is one of them,   */
/* so the result is exact; on equal values the first token's bits are kept.  */
/* ------------------------------------------------------------------------ */
void oracle_build_summaries(int B, int H_kv, int NB_max, int bs, int D,
                            const uint16_t *kv, const int32_t *ctx_len,
                            uint16_t *kminmax)
{
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int r = 0; r < B; r++) {
        for (int h = 0; h < H_kv; h++) {
            int nb = n_blocks_of(ctx_len[r], bs);
            if (nb > NB_max) nb = NB_max;
            for (int b = 0; b < nb; b++) {
                const uint16_t *K = kv + ((((size_t)r * H_kv + h) * NB_max + b) * 2 + 0) * bs * D;
                uint16_t *smin = kminmax + ((((size_t)r * H_kv + h) * NB_max + b) * 2 + 0) * D;
                uint16_t *smax = smin + D;
                for (int d = 0; d < D; d++) {
                    int first = 1;
                    uint16_t lo = 0, hi = 0;
                    for (int t = 0; t < bs; t++) {
                        if ((int64_t)b * bs + t >= ctx_len[r]) break;
                        uint16_t x = K[(size_t)t * D + d];
                        if (first || bf16_value(x) < bf16_value(lo)) lo = x;
                        if (first || bf16_value(x) > bf16_value(hi)) hi = x;
                        first = 0;
                    }
                    smin[d] = lo;
                    smax[d] = hi;
                }
            }
        }
    }
}

/* ------------------------------------------------------------------------ */
/* Lookahead block scoring.                                                  */
/* Section 4: the draft queries scan the per-block key summaries to rank the */
/* blocks.  Reading: the score of block b for KV head h is the bound, over   */
/* the block's bounding box [kmin, kmax], of the query-key products, summed   */
/* over the lookahead drafts j and the query heads g of h's group:           */
/*     s = sum_j sum_g sum_d max(q[j,g,d] * kmax[d], q[j,g,d] * kmin[d]).     */
/* Every product of two bf16 values is exact in fp64; the sum is taken in    */
/* fp64 in the order j, g, d and rounded once to fp32.  Blocks at or past     */
/* the request's last block score -inf.                                      */
/* ------------------------------------------------------------------------ */
void oracle_score(int B, int J, int H_q, int H_kv, int D, int NB_max, int bs,
                  const uint16_t *q_look, const uint16_t *kminmax,
                  const int32_t *ctx_len, float *scores)
{
    const int G = H_q / H_kv;
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int r = 0; r < B; r++) {
        for (int h = 0; h < H_kv; h++) {
            int nb = n_blocks_of(ctx_len[r], bs);
            float *out = scores + ((size_t)r * H_kv + h) * NB_max;
            for (int b = 0; b < NB_max; b++) {
                if (b >= nb) { out[b] = -INFINITY; continue; }
                const uint16_t *kmin = kminmax + ((((size_t)r * H_kv + h) * NB_max + b) * 2 + 0) * D;
                const uint16_t *kmax = kmin + D;
                double s = 0.0;
                for (int j = 0; j < J; j++) {
                    for (int gi = 0; gi < G; gi++) {
                        int g = h * G + gi;
                        const uint16_t *q = q_look + (((size_t)r * J + j) * H_q + g) * D;
                        for (int d = 0; d < D; d++) {
                            double qd = bf16_value(q[d]);
                            double a = qd * bf16_value(kmax[d]);
                            double c = qd * bf16_value(kmin[d]);
                            s += (a > c) ? a : c;
                        }
                    }
                }
                out[b] = (float)s;
            }
        }
    }
}

/* ------------------------------------------------------------------------ */
/* Top-K block selection under the token budget.                             */
/* Sections 4 and 5: per KV head, the K_b = budget / bs best-scoring blocks   */
/* are predicted for the next step (budget 2048 tokens).  Reading: order by   */
/* fp32 score descending, equal scores by lower block id first, NaN below     */
/* -inf; when the request has at most K_b blocks all are taken.  The chosen   */
/* ids are written in ascending order, -1 padded to K_b.                     */
/* ------------------------------------------------------------------------ */
typedef struct { float s; int32_t id; } scored_block;

/* 1 if a ranks before b */
static int ranks_before(float sa, int32_t ia, float sb, int32_t ib)
{
    int na = isnan(sa), nb = isnan(sb);
    if (na != nb) return nb;              /* a number ranks before NaN */
    if (!na && sa != sb) return sa > sb;
    return ia < ib;
}

static int cmp_rank(const void *pa, const void *pb)
{
    const scored_block *a = pa, *b = pb;
    if (a->id == b->id) return 0;
    return ranks_before(a->s, a->id, b->s, b->id) ? -1 : 1;
}

static int cmp_int32(const void *pa, const void *pb)
{
    int32_t a = *(const int32_t *)pa, b = *(const int32_t *)pb;
    return (a > b) - (a < b);
}

void oracle_select(int B, int H_kv, int NB_max, int bs, const float *scores,
                   const int32_t *ctx_len, int K_b, int32_t *sel, int32_t *n_sel)
{
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int r = 0; r < B; r++) {
        for (int h = 0; h < H_kv; h++) {
            int nb = n_blocks_of(ctx_len[r], bs);
            if (nb > NB_max) nb = NB_max;
            const float *row = scores + ((size_t)r * H_kv + h) * NB_max;
            int32_t *out = sel + ((size_t)r * H_kv + h) * K_b;
            scored_block *all = malloc(sizeof(scored_block) * (nb > 0 ? nb : 1));
            for (int b = 0; b < nb; b++) { all[b].s = row[b]; all[b].id = b; }
            qsort(all, nb, sizeof(scored_block), cmp_rank);
            int k = nb < K_b ? nb : K_b;
            for (int i = 0; i < k; i++) out[i] = all[i].id;
            qsort(out, k, sizeof(int32_t), cmp_int32);
            for (int i = k; i < K_b; i++) out[i] = -1;
            n_sel[(size_t)r * H_kv + h] = k;
            free(all);
        }
    }
}

/* ------------------------------------------------------------------------ */
/* Fetch cap: blocks per KV head per layer per step.                         */
/* Section 4 bounds the transfer to at most C blocks per KV head per layer;  */
/* section 5 and the agihunt summary express the cap as a fraction (default  */
/* 0.05, swept from 0.01 to fetch-all).  Reading: C = max(1, floor(cap*K_b))  */
/* for 0 < cap < 1, C = K_b for cap >= 1 (fetch-all), C = 0 for cap <= 0.     */
/* The 0.30 GB/step traffic printed for cap 0.01 pins the floor.             */
/* ------------------------------------------------------------------------ */
int oracle_fetch_cap_blocks(double cap, int K_b)
{
    if (!(cap > 0.0)) return 0;
    if (cap >= 1.0) return K_b;
    int c = (int)floor(cap * (double)K_b);
    return c < 1 ? 1 : c;
}

/* ------------------------------------------------------------------------ */
/* KV selection and staging, one step.                                       */
/* Section 4: selection keeps resident predicted blocks, and pairs admitted   */
/* non-resident predicted blocks with least-recently-selected eviction        */
/* targets; at most C blocks per KV head are transferred.                    */
/* State per (r, h): res_stamp[b] = -1 when block b is not resident, else the */
/* last step at which b was predicted or admitted.  Given the predicted set   */
/* P of step `step`:                                                          */
/*   1. every resident predicted block gets stamp = step;                    */
/*   2. the admitted list A is the first min(C, |P \ R|) blocks of P \ R,     */
/*      ordered by fp32 score descending, then block id ascending;           */
/*   3. free capacity K_b - |R| is used first; the remaining |A| - free       */
/*      admits each evict one block of R \ P, in order of stamp ascending,    */
/*      then block id ascending;                                              */
/*   4. R <- (R minus victims) plus A, with stamp = step for every admit;     */
/*   5. each admitted block is copied whole (K then V) from the host pool:    */
/*      the caller does that from `admitted`.                                */
/* Readings: admits beyond C are dropped this step (a later prediction may   */
/* bring them back); resident blocks no longer predicted stay resident until */
/* evicted.  Predicted ids outside [0, n_b) or repeated are ignored.          */
/* admitted [B][H_kv][max(C,1)] in admission order, evicted likewise.         */
/* n_deferred [B][H_kv] (may be NULL): |P \ R| - |A|, the predicted blocks    */
/* that were neither resident nor admitted, i.e. held back by the cap C.      */
/* ------------------------------------------------------------------------ */
typedef struct { int32_t key; int32_t id; } stamped_block;

static int cmp_stamp(const void *pa, const void *pb)
{
    const stamped_block *a = pa, *b = pb;
    if (a->key != b->key) return (a->key > b->key) - (a->key < b->key);
    return (a->id > b->id) - (a->id < b->id);
}

void oracle_stage(int B, int H_kv, int NB_max, int bs, const int32_t *ctx_len,
                  const int32_t *sel, const int32_t *n_sel, int K_sel,
                  const float *scores, int K_b, int C, int step,
                  int32_t *res_stamp, int32_t *admitted, int32_t *n_admitted,
                  int32_t *evicted, int32_t *n_evicted, int32_t *n_deferred)
{
    const int Cs = C > 0 ? C : 1;
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int r = 0; r < B; r++) {
        for (int h = 0; h < H_kv; h++) {
            const size_t rh = (size_t)r * H_kv + h;
            int nb = n_blocks_of(ctx_len[r], bs);
            if (nb > NB_max) nb = NB_max;
            int32_t *stamp = res_stamp + rh * NB_max;
            const float *sc = scores + rh * NB_max;
            const int32_t *P = sel + rh * K_sel;
            int np = n_sel[rh];
            if (np > K_sel) np = K_sel;
            if (np < 0) np = 0;

            char *pred = calloc(nb > 0 ? nb : 1, 1);
            int n_pred = 0;
            for (int i = 0; i < np; i++) {
                int b = P[i];
                if (b < 0 || b >= nb || pred[b]) continue;
                pred[b] = 1;
                n_pred++;
            }
            int n_res = 0;
            for (int b = 0; b < nb; b++) n_res += stamp[b] >= 0;

            /* 1 */
            for (int b = 0; b < nb; b++)
                if (pred[b] && stamp[b] >= 0) stamp[b] = step;

            /* 2 */
            scored_block *cand = malloc(sizeof(scored_block) * (n_pred > 0 ? n_pred : 1));
            int nc = 0;
            for (int b = 0; b < nb; b++)
                if (pred[b] && stamp[b] < 0) { cand[nc].s = sc[b]; cand[nc].id = b; nc++; }
            qsort(cand, nc, sizeof(scored_block), cmp_rank);
            int na = nc < C ? nc : C;
            if (na < 0) na = 0;

            /* 3 */
            int free_cap = K_b - n_res;
            if (free_cap < 0) free_cap = 0;
            int need = na - free_cap;
            if (need < 0) need = 0;
            stamped_block *old = malloc(sizeof(stamped_block) * (nb > 0 ? nb : 1));
            int no = 0;
            for (int b = 0; b < nb; b++)
                if (stamp[b] >= 0 && !pred[b]) { old[no].key = stamp[b]; old[no].id = b; no++; }
            qsort(old, no, sizeof(stamped_block), cmp_stamp);
            if (need > no) need = no;   /* cannot happen for |P| <= K_b, |R| <= K_b */

            /* 4 */
            for (int i = 0; i < need; i++) {
                stamp[old[i].id] = -1;
                evicted[rh * Cs + i] = old[i].id;
            }
            for (int i = 0; i < na; i++) {
                stamp[cand[i].id] = step;
                admitted[rh * Cs + i] = cand[i].id;
            }
            n_admitted[rh] = na;
            n_evicted[rh] = need;
            if (n_deferred) n_deferred[rh] = nc - na;
            free(old);
            free(cand);
            free(pred);
        }
    }
}

/* ------------------------------------------------------------------------ */
/* Sparse decode attention over the resident set.                            */
/* Sections 4 and 7: attention runs over the blocks staged in HBM only.      */
/* For query head g of request r (KV head h = g / G) the token set S is every */
/* token t of the listed blocks with t < ctx_len[r];                          */
/*     l_t = sm_scale * sum_d q[d] k_t[d],  m = max_t l_t,                    */
/*     out = sum_t exp(l_t - m) v_t / sum_t exp(l_t - m),                     */
/*     lse = m + log(sum_t exp(l_t - m)),                                     */
/* all in fp64, tokens taken in table order then position order.  Reading: a  */
/* softmax scale of 1/sqrt(D) by default (the caller passes it), no sink, no  */
/* positional bias; an empty set gives out = 0 and lse = -inf; listed ids     */
/* outside [0, n_b) are skipped.                                              */
/* blocks [B][H_kv][T] (-1 padded), n_blocks [B][H_kv].                       */
/* ------------------------------------------------------------------------ */
void oracle_attend(int B, int H_q, int H_kv, int D, int NB_max, int bs,
                   const uint16_t *q, const uint16_t *kv, const int32_t *ctx_len,
                   const int32_t *blocks, const int32_t *n_blocks, int T,
                   double sm_scale, double *out, double *lse)
{
    const int G = H_q / H_kv;
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int r = 0; r < B; r++) {
        for (int g = 0; g < H_q; g++) {
            const int h = g / G;
            const size_t rh = (size_t)r * H_kv + h;
            int nb = n_blocks_of(ctx_len[r], bs);
            if (nb > NB_max) nb = NB_max;
            const uint16_t *qv = q + ((size_t)r * H_q + g) * D;
            double *o = out + ((size_t)r * H_q + g) * D;
            int n = n_blocks[rh];
            if (n > T) n = T;
            if (n < 0) n = 0;

            /* logits, in table order */
            int cap = n * bs;
            double *logit = malloc(sizeof(double) * (cap > 0 ? cap : 1));
            const uint16_t **vrow = malloc(sizeof(uint16_t *) * (cap > 0 ? cap : 1));
            int cnt = 0;
            for (int i = 0; i < n; i++) {
                int b = blocks[rh * T + i];
                if (b < 0 || b >= nb) continue;
                const uint16_t *K = kv + ((rh * NB_max + b) * 2 + 0) * bs * D;
                const uint16_t *V = K + (size_t)bs * D;
                for (int t = 0; t < bs; t++) {
                    if ((int64_t)b * bs + t >= ctx_len[r]) break;
                    double dot = 0.0;
                    for (int d = 0; d < D; d++)
                        dot += bf16_value(qv[d]) * bf16_value(K[(size_t)t * D + d]);
                    logit[cnt] = sm_scale * dot;
                    vrow[cnt] = V + (size_t)t * D;
                    cnt++;
                }
            }
            for (int d = 0; d < D; d++) o[d] = 0.0;
            if (cnt == 0) {
                lse[(size_t)r * H_q + g] = -INFINITY;
            } else {
                double m = logit[0];
                for (int i = 1; i < cnt; i++) if (logit[i] > m) m = logit[i];
                double den = 0.0;
                for (int i = 0; i < cnt; i++) {
                    double p = exp(logit[i] - m);
                    den += p;
                    for (int d = 0; d < D; d++) o[d] += p * bf16_value(vrow[i][d]);
                }
                for (int d = 0; d < D; d++) o[d] /= den;
                lse[(size_t)r * H_q + g] = m + log(den);
            }
            free(vrow);
            free(logit);
        }
    }
}

/* ------------------------------------------------------------------------ */
/* Appending one decoded token per request.                                   */
/* Section 4: the full KV lives off-GPU while HBM keeps the per-block key     */
/* summaries.  When request r's next token (position c = ctx_len[r]) gets its */
/* K and V, they are written at block c / bs, row c % bs of every KV head in  */
/* the pool, that block's summary becomes the min / max over its valid keys   */
/* including the new one, and ctx_len[r] becomes c + 1.  Reading: the summary */
/* of a block is its valid keys' coordinate-wise min and max (as built above:  */
/* the first of equal extreme values in position order is kept), so the new    */
/* key replaces a bound only when strictly below the min or above the max,    */
/* and a fresh block (c % bs == 0) starts from the new key.  A request whose  */
/* pool is full (c >= NB_max * bs), or with c < 0, is left unchanged.        */
/* k_new, v_new [B][H_kv][D]; kv and kminmax as above, updated in place.      */
/* ------------------------------------------------------------------------ */
void oracle_append(int B, int H_kv, int NB_max, int bs, int D,
                   const uint16_t *k_new, const uint16_t *v_new, int32_t *ctx_len,
                   uint16_t *kv, uint16_t *kminmax)
{
    for (int r = 0; r < B; r++) {
        const int32_t c = ctx_len[r];
        if (c < 0 || (int64_t)c >= (int64_t)NB_max * bs) continue;
        const int b = c / bs, row = c % bs;
        for (int h = 0; h < H_kv; h++) {
            const size_t rh = (size_t)r * H_kv + h;
            const uint16_t *k = k_new + rh * D;
            const uint16_t *v = v_new + rh * D;
            uint16_t *K = kv + ((rh * NB_max + b) * 2 + 0) * bs * D;
            uint16_t *V = K + (size_t)bs * D;
            uint16_t *smin = kminmax + ((rh * NB_max + b) * 2 + 0) * D;
            uint16_t *smax = smin + D;
            for (int d = 0; d < D; d++) {
                K[(size_t)row * D + d] = k[d];
                V[(size_t)row * D + d] = v[d];
                if (row == 0 || bf16_value(k[d]) < bf16_value(smin[d])) smin[d] = k[d];
                if (row == 0 || bf16_value(k[d]) > bf16_value(smax[d])) smax[d] = k[d];
            }
        }
        ctx_len[r] = c + 1;
    }
}

/* ------------------------------------------------------------------------ */
/* Exact attention mass per block (for the lookahead-agreement analogue).     */
/* Section 4 reports how often the draft-based top-K agrees with the true     */
/* next token's top-K set.  Reading: the true set of KV head h is the top-K   */
/* by the next query's exact attention mass over the whole context, summed    */
/* over the query heads g of h's group:                                       */
/*     mass[b] = sum_g sum_{t in block b, t < ctx} softmax_g(t),              */
/*     softmax_g(t) = exp(l_t - m) / sum_{t' < ctx} exp(l_t' - m),            */
/*     l_t = sm_scale * q_g . k_t,                                            */
/* in fp64.  Blocks at or past the request's last block get 0; a request with */
/* an empty context gets 0 everywhere.                                        */
/* q [B][H_q][D]; kv [B][H_kv][NB_max][2][bs][D]; mass [B][H_kv][NB_max].     */
/* ------------------------------------------------------------------------ */
void oracle_block_mass(int B, int H_q, int H_kv, int D, int NB_max, int bs,
                       const uint16_t *q, const uint16_t *kv, const int32_t *ctx_len,
                       double sm_scale, double *mass)
{
    const int G = H_q / H_kv;
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int r = 0; r < B; r++) {
        for (int h = 0; h < H_kv; h++) {
            const size_t rh = (size_t)r * H_kv + h;
            double *out = mass + rh * NB_max;
            for (int b = 0; b < NB_max; b++) out[b] = 0.0;
            int64_t n_tok = ctx_len[r];
            if (n_tok > (int64_t)NB_max * bs) n_tok = (int64_t)NB_max * bs;
            if (n_tok <= 0) continue;
            double *logit = malloc(sizeof(double) * (size_t)n_tok);
            for (int gi = 0; gi < G; gi++) {
                const uint16_t *qv = q + ((size_t)r * H_q + (size_t)h * G + gi) * D;
                double m = -INFINITY;
                for (int64_t t = 0; t < n_tok; t++) {
                    const uint16_t *k = kv + ((rh * NB_max + t / bs) * 2 + 0) * bs * D + (size_t)(t % bs) * D;
                    double dot = 0.0;
                    for (int d = 0; d < D; d++) dot += bf16_value(qv[d]) * bf16_value(k[d]);
                    logit[t] = sm_scale * dot;
                    if (logit[t] > m) m = logit[t];
                }
                double den = 0.0;
                for (int64_t t = 0; t < n_tok; t++) den += exp(logit[t] - m);
                for (int64_t t = 0; t < n_tok; t++) out[t / bs] += exp(logit[t] - m) / den;
            }
            free(logit);
        }
    }
}

/* Number of threads the OpenMP loops above use (for reporting). */
#ifdef _OPENMP
#include <omp.h>
#endif
int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
