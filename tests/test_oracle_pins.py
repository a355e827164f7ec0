"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each test names what fixes the expected value: brute force written differently
(NumPy / Python sort), a closed form, an invariant stated by the OasisKV pages
(arXiv 2608.08097, paperlayer summary, section 4 "System Design"), or a case
worked by hand from that section's staging rule.  No GPU is used.
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle
import workloads as wl


def u16(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def f64(a_u16: np.ndarray) -> np.ndarray:
    return (a_u16.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def tiny(**kw):
    base = dict(name="tiny", B=2, H_q=8, H_kv=2, ctx=(70, 200), budget=64, J=2,
                structure="none", seed=7)
    base.update(kw)
    return wl.Workload(**base)


def inputs(w):
    ctx = wl.context_lengths(w).numpy()
    kv = u16(wl.kv_pool(w))
    ql = u16(wl.lookahead(w, 0))
    return ctx, kv, ql


# --------------------------------------------------------------------------
# block summaries


def np_summaries(kv, ctx, bs):
    B, H, NB, _, _, D = kv.shape
    K = f64(kv[:, :, :, 0])                                 # [B][H][NB][bs][D]
    lo = np.full((B, H, NB, D), np.nan)
    hi = np.full((B, H, NB, D), np.nan)
    for r in range(B):
        n_b = -(-int(ctx[r]) // bs)
        for b in range(n_b):
            valid = min(bs, int(ctx[r]) - b * bs)
            lo[r, :, b] = K[r, :, b, :valid].min(axis=1)
            hi[r, :, b] = K[r, :, b, :valid].max(axis=1)
    return lo, hi


def test_summaries_equal_numpy_min_max_over_valid_tokens():
    w = tiny()
    ctx, kv, _ = inputs(w)
    s = oracle.build_summaries(kv, ctx, w.bs)
    lo, hi = np_summaries(kv, ctx, w.bs)
    got = f64(s)
    for r in range(w.B):
        n_b = -(-int(ctx[r]) // w.bs)
        np.testing.assert_array_equal(got[r, :, :n_b, 0], lo[r, :, :n_b])
        np.testing.assert_array_equal(got[r, :, :n_b, 1], hi[r, :, :n_b])
    # the padding value never reaches a summary of a partial block
    assert np.all(got[:, :, :, 1] < wl.PAD_VALUE)


# --------------------------------------------------------------------------
# scoring


def test_score_matches_signed_split_identity():
    """sum_{j,g,d} max(q kmax, q kmin) = sum_d Qp_d kmax_d + Qm_d kmin_d with
    Qp = sum_{j,g} max(q, 0), Qm = sum_{j,g} min(q, 0): a different formula,
    evaluated in NumPy on NumPy-built summaries."""
    w = tiny()
    ctx, kv, ql = inputs(w)
    s = oracle.score(ql, oracle.build_summaries(kv, ctx, w.bs), ctx, w.bs, w.H_kv)
    lo, hi = np_summaries(kv, ctx, w.bs)
    q = f64(ql).reshape(w.B, w.J, w.H_kv, w.G, w.D)
    Qp = np.maximum(q, 0).sum(axis=(1, 3))                      # [B][H][D]
    Qm = np.minimum(q, 0).sum(axis=(1, 3))
    for r in range(w.B):
        n_b = -(-int(ctx[r]) // w.bs)
        ref = (Qp[r][:, None, :] * hi[r, :, :n_b] + Qm[r][:, None, :] * lo[r, :, :n_b]).sum(-1)
        got = s[r, :, :n_b].astype(np.float64)
        ulp = np.spacing(np.abs(ref).astype(np.float32)).astype(np.float64)
        assert np.all(np.abs(got - ref) <= ulp), np.max(np.abs(got - ref) / ulp)
        assert np.all(np.isneginf(s[r, :, n_b:]))


def test_score_bounds_every_key_of_the_block():
    """The bounding-box score is at least sum_{j,g} max_t q . k_t over the
    block's valid keys (brute force over tokens)."""
    w = tiny()
    ctx, kv, ql = inputs(w)
    s = oracle.score(ql, oracle.build_summaries(kv, ctx, w.bs), ctx, w.bs, w.H_kv)
    K = f64(kv[:, :, :, 0])
    q = f64(ql)
    for r in range(w.B):
        n_b = -(-int(ctx[r]) // w.bs)
        for h in range(w.H_kv):
            for b in range(n_b):
                valid = min(w.bs, int(ctx[r]) - b * w.bs)
                keys = K[r, h, b, :valid]                          # [t][D]
                qs = q[r][:, h * w.G:(h + 1) * w.G].reshape(-1, w.D)  # [(j,g)][D]
                lower = (qs @ keys.T).max(axis=1).sum()
                assert s[r, h, b] >= np.float32(lower) - 1e-3


def test_score_is_exact_dot_for_single_token_and_constant_blocks():
    """A block holding one token, or 16 equal keys, has kmin = kmax = k, so the
    score is exactly sum_{j,g} q_{j,g} . k (NumPy, fp64, then fp32)."""
    w = tiny(ctx=16 * 5 + 1, B=1)                 # last block holds one token
    ctx = wl.context_lengths(w).numpy()
    kvt = wl.kv_pool(w)
    kvt[0, :, 2, 0] = kvt[0, :, 2, 0, 3:4]        # block 2: every key equal to its 4th key
    kv = u16(kvt)
    ql = u16(wl.lookahead(w, 0))
    s = oracle.score(ql, oracle.build_summaries(kv, ctx, w.bs), ctx, w.bs, w.H_kv)
    q = f64(ql)
    K = f64(kv[:, :, :, 0])
    for h in range(w.H_kv):
        qs = q[0][:, h * w.G:(h + 1) * w.G].reshape(-1, w.D)
        for b, t in ((5, 0), (2, 3)):
            exact = (qs @ K[0, h, b, t]).sum()
            assert s[0, h, b] == np.float32(exact)


def test_score_sums_over_drafts_and_group_heads():
    """Doubling the drafts with an identical copy doubles every score (the sum
    over j is linear), and a group's score is the sum of one-head scores."""
    w = tiny(J=1)
    ctx, kv, ql = inputs(w)
    summ = oracle.build_summaries(kv, ctx, w.bs)
    s1 = oracle.score(ql, summ, ctx, w.bs, w.H_kv)
    s2 = oracle.score(np.concatenate([ql, ql], axis=1), summ, ctx, w.bs, w.H_kv)
    fin = np.isfinite(s1)
    np.testing.assert_allclose(s2[fin], 2 * s1[fin].astype(np.float64), rtol=2e-7)
    # one query head per KV head: split the group into G single-head problems
    heads = np.zeros_like(s1, dtype=np.float64)
    for gi in range(w.G):
        sub = ql.reshape(w.B, 1, w.H_kv, w.G, w.D)[:, :, :, gi]           # [B][1][H_kv][D]
        heads += oracle.score(np.ascontiguousarray(sub), summ, ctx, w.bs, w.H_kv).astype(np.float64)
    np.testing.assert_allclose(s1[fin], heads[fin], rtol=1e-6, atol=1e-3)


# --------------------------------------------------------------------------
# selection


def brute_select(row, n_b, K):
    def key(b):
        v = float(row[b])
        return (1 if math.isnan(v) else 0, 0.0 if math.isnan(v) else -v, b)
    return sorted(sorted(range(n_b), key=key)[:K])


@pytest.mark.parametrize("ties", [0, 3, 40])
def test_select_matches_python_sort(ties):
    w = tiny(B=3, ctx=(20, 900), budget=160)
    ctx = wl.context_lengths(w).numpy()
    sc = wl.random_scores(w, tie_levels=ties).numpy()
    sel, n = oracle.select(sc, ctx, w.bs, w.K_b)
    for r in range(w.B):
        n_b = -(-int(ctx[r]) // w.bs)
        for h in range(w.H_kv):
            ref = brute_select(sc[r, h], n_b, w.K_b)
            assert n[r, h] == len(ref)
            assert sel[r, h, :len(ref)].tolist() == ref
            assert np.all(sel[r, h, len(ref):] == -1)


def test_select_nan_ranks_below_minus_inf_and_short_rows_take_all():
    w = tiny(B=2, ctx=(40, 40), budget=32)       # 3 blocks per request, K_b = 2
    sc = np.array([[[np.nan, -np.inf, 1.0], [5.0, 5.0, 5.0]],
                   [[2.0, np.nan, np.nan], [-1.0, -2.0, -3.0]]], dtype=np.float32)
    ctx = np.array([40, 40], dtype=np.int32)
    sel, n = oracle.select(sc, ctx, w.bs, 2)
    assert sel.tolist() == [[[1, 2], [0, 1]], [[0, 1], [0, 1]]]
    sel, n = oracle.select(sc, np.array([17, 33], dtype=np.int32), w.bs, 4)
    assert sel.tolist() == [[[0, 1, -1, -1], [0, 1, -1, -1]], [[0, 1, 2, -1], [0, 1, 2, -1]]]
    assert n.tolist() == [[2, 2], [3, 3]]


@pytest.mark.parametrize("name", ["parity_8q2kv_4k", "qwen3_8b_16k_b32_hbm"])
def test_planted_blocks_are_all_selected(name):
    """Recall of the planted heavy-hitter blocks is 1: the planted shift
    dominates the summary-bound noise."""
    w = wl.WORKLOADS[name]
    if w.B > 2:
        w = w.shrink(B=2)
    ctx, kv, ql = inputs(w)
    s = oracle.score(ql, oracle.build_summaries(kv, ctx, w.bs), ctx, w.bs, w.H_kv)
    sel, _ = oracle.select(s, ctx, w.bs, w.K_b)
    for r, heads in enumerate(wl.planted_blocks(w)):
        for h, planted in enumerate(heads):
            assert set(planted) <= set(sel[r, h].tolist())


# --------------------------------------------------------------------------
# fetch cap and staging


def _golden(name):
    """key -> float from a fixture under tests/golden/ (# lines are comments)."""
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", name)
    out = {}
    for line in open(path):
        line = line.strip()
        if line and not line.startswith("#"):
            k, v = line.split()
            out[k] = float(v)
    return out


def test_fetch_cap_closed_forms():
    """The pages' traffic at the lowest fetch cap (agihunt summary,
    fetch-cap ablation; fixture tests/golden/fetch_cap_ablation.txt): the
    oracle's cap rule gives C = 1 block of 8 KiB K+V per KV head and layer,
    which over 8 KV heads, 36 layers and 128 requests is the printed 0.30 GB
    per step in decimal GB (a ceiling would give 0.60)."""
    g = _golden("fetch_cap_ablation.txt")
    bs, D = int(g["block_tokens"]), int(g["head_dim"])
    K_b = int(g["kv_budget_tokens"]) // bs
    block_bytes = 2 * bs * D * 2
    per_step = block_bytes * g["kv_heads"] * g["layers"] * g["batch"]
    C = oracle.fetch_cap_blocks(g["cap_low"], K_b)
    assert C == 1
    assert round(C * per_step / 1e9, 2) == g["traffic_gb_per_step_at_cap_low"]
    # fetch-all moves every newly selected block: the printed 5.05 GB per
    # step is ~16.7 blocks per (request, KV head, layer), within the budget
    fetch_all_blocks = g["traffic_gb_per_step_fetch_all"] * 1e9 / per_step
    assert 16 < fetch_all_blocks < 17 and fetch_all_blocks < K_b
    assert oracle.fetch_cap_blocks(0.05, K_b) == 6
    assert oracle.fetch_cap_blocks(1.0, K_b) == K_b
    assert oracle.fetch_cap_blocks(0.0, K_b) == 0
    assert oracle.fetch_cap_blocks(1e-9, K_b) == 1


def run_stage(steps_P, steps_scores, n_b, K_b, Cs, deferred=None):
    """Drive the oracle for one (r, h) through hand-written predicted sets;
    `deferred` (a list) receives the held-back count of each step."""
    NB = n_b
    st = oracle.StageState(1, 1, NB)
    ctx = np.array([n_b * 16], dtype=np.int32)
    log = []
    deferred = [] if deferred is None else deferred
    for s, (P, sc, C) in enumerate(zip(steps_P, steps_scores, Cs)):
        sel = np.full((1, 1, K_b), -1, dtype=np.int32)
        sel[0, 0, :len(P)] = sorted(P)
        n = np.array([[len(P)]], dtype=np.int32)
        score = np.zeros((1, 1, NB), dtype=np.float32)
        for b, v in sc.items():
            score[0, 0, b] = v
        adm, na, ev, ne = oracle.stage(st, sel, n, score, ctx, 16, K_b, C, s)
        log.append((adm[0, 0, :na[0, 0]].tolist(), ev[0, 0, :ne[0, 0]].tolist(),
                    {int(b): int(st.stamp[0, 0, b]) for b in st.resident(0, 0)}))
        deferred.append(int(st.deferred[0, 0]))
    return log


def test_stage_worked_example():
    """Section 4's rule applied by hand to 6 blocks, K_b = 3:
    step 0 (C = 3, empty): P = {1,3,5} -> admit 1,3,5 (equal scores: by id).
    step 1 (C = 2): P = {0,3,4}, s4 = 7 > s0 = 5.  3 is kept and re-stamped;
      admits in score order 4, 0; no free room, so two victims from R \\ P =
      {1, 5}, both stamped 0, by id: 1, 5.  R = {0:1, 3:1, 4:1}.
    step 2 (C = 1): P = {2,3,5}, s5 = 9 > s2 = 1.  3 -> stamp 2; only 5 is
      admitted (cap 1); victim among {0, 4} (stamps 1, 1) by id: 0.
      R = {3:2, 4:1, 5:2}.
    step 3 (C = 1): P = {2,3} (a short prediction).  3 -> 3; admit 2; victim
      among {4 (stamp 1), 5 (stamp 2)}: the least recently selected, 4.
      R = {2:3, 3:3, 5:2}.
    step 4 (C = 1): P = {0,1,3}, s0 = s1 = 2.  3 -> 4; tie -> admit 0; victim
      among {2 (stamp 3), 5 (stamp 2)}: 5, though its id is larger.
      R = {0:4, 2:3, 3:4}.
    Held back by the cap (predicted, neither resident nor admitted): step 2
    leaves block 2 out, step 4 block 1; the other steps admit every missing
    predicted block."""
    deferred = []
    log = run_stage(
        steps_P=[[1, 3, 5], [0, 3, 4], [2, 3, 5], [2, 3], [0, 1, 3]],
        steps_scores=[{}, {0: 5, 4: 7}, {2: 1, 5: 9}, {}, {0: 2, 1: 2}],
        n_b=6, K_b=3, Cs=[3, 2, 1, 1, 1], deferred=deferred)
    assert deferred == [0, 0, 1, 0, 1]
    assert log[0] == ([1, 3, 5], [], {1: 0, 3: 0, 5: 0})
    assert log[1] == ([4, 0], [1, 5], {0: 1, 3: 1, 4: 1})
    assert log[2] == ([5], [0], {3: 2, 4: 1, 5: 2})
    assert log[3] == ([2], [4], {2: 3, 3: 3, 5: 2})
    assert log[4] == ([0], [5], {0: 4, 2: 3, 3: 4})


def test_stage_free_capacity_is_used_before_eviction():
    log = run_stage(steps_P=[[0, 1], [0, 1, 2, 3]], steps_scores=[{}, {2: 1, 3: 2}],
                    n_b=8, K_b=4, Cs=[4, 1])
    assert log[1] == ([3], [], {0: 1, 1: 1, 3: 1})


@pytest.mark.parametrize("C,turnover", [(1, 3), (6, 6), (6, 20), (128, 20)])
def test_stage_invariants_over_random_sequences(C, turnover):
    """Invariants of section 4 over 12 steps: resident predicted blocks stay;
    at most C admits; the working set never exceeds the budget; every admit is
    a predicted non-resident block; every victim is a resident block that is
    not predicted and was selected no later than any non-predicted block that
    stays; with C = K_b (fetch-all) the new resident set equals the prediction."""
    w = tiny(B=2, H_kv=2, H_q=4, ctx=(3000, 5000), budget=2048)
    K_b = w.K_b
    ctx = wl.context_lengths(w).numpy()
    sels, nsels, scores = wl.predicted_set_sequence(w, 12, turnover)
    st = oracle.StageState(w.B, w.H_kv, w.NB_max)
    for s in range(12):
        Cs = K_b if s == 0 else C
        before = st.stamp.copy()
        adm, na, ev, ne = oracle.stage(st, sels[s].numpy(), nsels[s].numpy(), scores[s].numpy(),
                                       ctx, w.bs, K_b, Cs, s)
        for r in range(w.B):
            for h in range(w.H_kv):
                P = set(sels[s][r, h, :nsels[s][r, h]].tolist())
                R0 = set(np.nonzero(before[r, h] >= 0)[0].tolist())
                R1 = set(st.resident(r, h).tolist())
                A = adm[r, h, :na[r, h]].tolist()
                E = ev[r, h, :ne[r, h]].tolist()
                assert P & R0 <= R1
                assert len(A) <= Cs and len(R1) <= K_b
                assert set(A) <= P - R0 and R1 == (R0 - set(E)) | set(A)
                assert len(A) == min(Cs, len(P - R0))
                # the held-back count: missing predicted blocks not admitted
                assert int(st.deferred[r, h]) == len(P - R0) - len(A)
                if Cs == K_b:
                    assert int(st.deferred[r, h]) == 0
                # admitted are the best-scoring of P \ R0
                sc = scores[s][r, h].numpy()
                rest = (P - R0) - set(A)
                if A and rest:
                    worst = min((float(sc[a]), -a) for a in A)
                    assert all((float(sc[b]), -b) < worst for b in rest)
                # victims are least recently selected among the non-predicted
                kept_old = (R0 - P) - set(E)
                if E and kept_old:
                    newest_victim = max((int(before[r, h, e]), e) for e in E)
                    assert all((int(before[r, h, k]), k) > newest_victim for k in kept_old)
                for b in R1:
                    if b in P or b in A:
                        assert st.stamp[r, h, b] == s
                if Cs == K_b:
                    assert R1 == P


# --------------------------------------------------------------------------
# attention


def np_attend(q, kv, ctx, blocks, sm_scale):
    """NumPy fp64 softmax attention for one (r, g) over the listed blocks."""
    K = f64(kv[:, 0])
    V = f64(kv[:, 1])
    ks, vs = [], []
    for b in blocks:
        valid = max(0, min(16, ctx - b * 16))
        ks.append(K[b, :valid])
        vs.append(V[b, :valid])
    if not ks or sum(len(k) for k in ks) == 0:
        return np.zeros(q.shape[-1]), -np.inf
    K = np.concatenate(ks)
    V = np.concatenate(vs)
    l = sm_scale * (K @ f64(q))
    m = l.max()
    p = np.exp(l - m)
    return (p @ V) / p.sum(), m + np.log(p.sum())


@pytest.mark.parametrize("T", [1, 5, 64])
def test_attend_matches_numpy_softmax(T):
    w = tiny(B=2, ctx=(30, 1000))
    ctx = wl.context_lengths(w).numpy()
    kv = u16(wl.kv_pool(w))
    q = u16(wl.attention_query(w))
    tbl, n = wl.random_table(w, T)
    tbl, n = tbl.numpy(), n.numpy()
    sm = 1 / math.sqrt(w.D)
    out, lse = oracle.attend(q, kv, ctx, tbl, n, sm)
    for r in range(w.B):
        for g in range(w.H_q):
            h = g // w.G
            ref, ref_lse = np_attend(q[r, g], kv[r, h], int(ctx[r]), tbl[r, h, :n[r, h]].tolist(), sm)
            np.testing.assert_allclose(out[r, g], ref, rtol=1e-11, atol=1e-12)
            assert abs(lse[r, g] - ref_lse) <= 1e-11 * max(1, abs(ref_lse))


def test_attend_full_budget_is_dense_attention():
    """With every block of the request listed, sparse attention is dense
    softmax attention over the whole context (the full-attention anchor the
    pages compare against)."""
    w = tiny(B=2, ctx=(100, 300))
    ctx = wl.context_lengths(w).numpy()
    kvt = wl.kv_pool(w)
    kv = u16(kvt)
    q = u16(wl.attention_query(w))
    T = w.NB_max
    tbl = np.full((w.B, w.H_kv, T), -1, dtype=np.int32)
    n = np.zeros((w.B, w.H_kv), dtype=np.int32)
    for r in range(w.B):
        n_b = -(-int(ctx[r]) // w.bs)
        tbl[r, :, :n_b] = np.arange(n_b)
        n[r] = n_b
    out, _ = oracle.attend(q, kv, ctx, tbl, n, 0.1)
    for r in range(w.B):
        L = int(ctx[r])
        for g in range(w.H_q):
            h = g // w.G
            K = f64(kv[r, h, :, 0].reshape(-1, w.D)[:L])        # dense K in token order
            V = f64(kv[r, h, :, 1].reshape(-1, w.D)[:L])
            a = 0.1 * K @ f64(q[r, g])
            p = np.exp(a - a.max())
            np.testing.assert_allclose(out[r, g], p @ V / p.sum(), rtol=1e-11, atol=1e-12)


def test_attend_closed_forms():
    """Equal keys give the mean of V; a one-token set gives that token's V;
    an empty set gives zeros and lse = -inf."""
    w = tiny(B=1, ctx=64 + 1, H_q=4, H_kv=2)
    kvt = wl.kv_pool(w)
    kvt[0, :, :, 0] = kvt[0, 0, 0, 0, 0]                 # every key the same vector
    kv = u16(kvt)
    q = u16(wl.attention_query(w))
    ctx = np.array([65], dtype=np.int32)
    tbl = np.array([[[0, 1, 2, 3, 4], [4, -1, -1, -1, -1]]], dtype=np.int32)
    n = np.array([[5, 1]], dtype=np.int32)
    out, lse = oracle.attend(q, kv, ctx, tbl, n, 0.3)
    V = f64(kv[0, :, :, 1])
    mean0 = V[0].reshape(-1, w.D)[:65].mean(axis=0)
    np.testing.assert_allclose(out[0, 0], mean0, rtol=1e-12, atol=1e-13)
    np.testing.assert_array_equal(out[0, 2], V[1, 4, 0])          # block 4 holds one token
    n0 = np.zeros_like(n)
    out, lse = oracle.attend(q, kv, ctx, tbl, n0, 0.3)
    assert np.all(out == 0) and np.all(np.isneginf(lse))


# --------------------------------------------------------------------------
# append: one decoded token per request


def np_first_extreme_bits(kv, r, h, b, valid):
    """bf16 bits of the coordinate-wise min and max over the first `valid`
    keys of a block, the first of equal values in position order (NumPy's
    argmin / argmax return the first occurrence)."""
    K = kv[r, h, b, 0, :valid]
    vals = f64(K)
    cols = np.arange(K.shape[1])
    return K[vals.argmin(axis=0), cols], K[vals.argmax(axis=0), cols]


def test_append_matches_numpy_rebuild_token_by_token():
    """Appending tokens one at a time, across block boundaries and up to the
    pool's capacity: every block summary equals NumPy's min / max over the
    updated pool's valid keys, the K / V rows land at the context position,
    nothing else in the pool changes, and a full request stays unchanged."""
    w = tiny(ctx=(14, 40))                     # NB_max = 3 blocks = 48 tokens
    ctx, kv, _ = inputs(w)
    summ = oracle.build_summaries(kv, ctx, w.bs)
    cap = w.NB_max * w.bs
    g = torch.Generator().manual_seed(11)
    for step in range(cap - int(ctx.min()) + 2):      # until every request is full, then two more
        k = u16(torch.randn((w.B, w.H_kv, w.D), generator=g).to(torch.bfloat16))
        v = u16(torch.randn((w.B, w.H_kv, w.D), generator=g).to(torch.bfloat16))
        ctx2, kv2, summ2 = oracle.append(k, v, ctx, kv, summ, w.bs)
        for r in range(w.B):
            c = int(ctx[r])
            if c >= cap:
                assert ctx2[r] == c
                np.testing.assert_array_equal(kv2[r], kv[r])
                np.testing.assert_array_equal(summ2[r], summ[r])
                continue
            assert ctx2[r] == c + 1
            b, row = divmod(c, w.bs)
            np.testing.assert_array_equal(kv2[r, :, b, 0, row], k[r])
            np.testing.assert_array_equal(kv2[r, :, b, 1, row], v[r])
            changed = np.zeros(kv.shape[1:], dtype=bool)
            changed[:, b, :, row] = True
            np.testing.assert_array_equal(kv2[r][~changed], kv[r][~changed])
            for h in range(w.H_kv):
                for bb in range(-(-(c + 1) // w.bs)):
                    valid = min(w.bs, c + 1 - bb * w.bs)
                    lo, hi = np_first_extreme_bits(kv2, r, h, bb, valid)
                    np.testing.assert_array_equal(summ2[r, h, bb, 0], lo, err_msg=f"step {step} r {r} b {bb}")
                    np.testing.assert_array_equal(summ2[r, h, bb, 1], hi)
        ctx, kv, summ = ctx2, kv2, summ2
    assert np.all(ctx == cap)                  # every request reached the capacity


def test_append_keeps_the_first_of_equal_bounds_and_starts_fresh_blocks():
    """+0 then -0 (equal values, different bits): the bound keeps the first;
    a token that starts a block sets both bounds to its key whatever the stale
    summary held."""
    B, H, NB, bs, D = 1, 1, 2, 16, 128
    kv = np.zeros((B, H, NB, 2, bs, D), dtype=np.uint16)
    summ = np.zeros((B, H, NB, 2, D), dtype=np.uint16)
    ctx = np.array([1], dtype=np.int32)        # token 0 holds +0 everywhere
    neg0 = np.full((B, H, D), 0x8000, dtype=np.uint16)
    ctx, kv, summ = oracle.append(neg0, neg0, ctx, kv, summ, bs)
    assert np.all(summ[0, 0, 0] == 0x0000)      # the first (+0) stays
    one = np.full((B, H, D), 0x3F80, dtype=np.uint16)          # 1.0
    summ[0, 0, 1] = 0x7F80                      # stale +inf in the next block
    ctx = np.array([bs], dtype=np.int32)
    ctx, kv, summ = oracle.append(one, one, ctx, kv, summ, bs)
    assert ctx[0] == bs + 1
    assert np.all(summ[0, 0, 1] == 0x3F80)


def test_append_skips_negative_context():
    w = tiny()
    ctx, kv, _ = inputs(w)
    summ = oracle.build_summaries(kv, ctx, w.bs)
    ctx = ctx.copy()
    ctx[0] = -1
    k = np.zeros((w.B, w.H_kv, w.D), dtype=np.uint16)
    ctx2, kv2, summ2 = oracle.append(k, k, ctx, kv, summ, w.bs)
    assert ctx2[0] == -1
    np.testing.assert_array_equal(kv2[0], kv[0])
    assert ctx2[1] == ctx[1] + 1


# --------------------------------------------------------------------------
# exact block attention mass and agreement (lookahead-agreement analogue)


def np_block_mass(q, kv, ctx, sm):
    """Dense softmax in NumPy (matrix products, exp, block sums): a second
    implementation of the same definition."""
    B, H_kv, NB, _, bs, D = kv.shape
    H_q = q.shape[1]
    G = H_q // H_kv
    out = np.zeros((B, H_kv, NB))
    for r in range(B):
        n = min(int(ctx[r]), NB * bs)
        if n <= 0:
            continue
        for h in range(H_kv):
            K = f64(kv[r, h, :, 0]).reshape(NB * bs, D)[:n]
            Q = f64(q[r, h * G:(h + 1) * G])                      # [G][D]
            L = sm * Q @ K.T                                     # [G][n]
            P = np.exp(L - L.max(axis=1, keepdims=True))
            P /= P.sum(axis=1, keepdims=True)
            per_tok = P.sum(axis=0)
            out[r, h] = np.bincount(np.arange(n) // bs, weights=per_tok, minlength=NB)[:NB]
    return out


def test_block_mass_matches_numpy_dense_softmax():
    w = tiny(ctx=(70, 200), structure="planted", planted=2)
    ctx, kv, _ = inputs(w)
    q = u16(wl.attention_query(w, 1))
    sm = 1 / math.sqrt(w.D)
    got = oracle.block_mass(q, kv, ctx, sm)
    ref = np_block_mass(q, kv, ctx, sm)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-15)
    # each query head's softmax sums to one: G per (request, KV head)
    np.testing.assert_allclose(got.sum(axis=2), np.full((w.B, w.H_kv), w.G), rtol=1e-12)
    for r in range(w.B):
        assert np.all(got[r, :, -(-int(ctx[r]) // w.bs):] == 0)


def test_block_mass_of_equal_keys_counts_tokens():
    """All keys equal: every token has the same weight, so a block's mass is
    G * (its valid tokens) / context."""
    w = tiny(ctx=(37, 90))
    ctx, kv, _ = inputs(w)
    kv = kv.copy()
    kv[:, :, :, 0] = kv[:, :, :1, 0, :1]
    q = u16(wl.attention_query(w, 1))
    got = oracle.block_mass(q, kv, ctx, 0.1)
    for r in range(w.B):
        c = int(ctx[r])
        valid = np.clip(c - np.arange(w.NB_max) * w.bs, 0, w.bs)
        np.testing.assert_allclose(got[r], np.broadcast_to(w.G * valid / c, got[r].shape), rtol=1e-12)


def test_block_mass_empty_context_and_agreement_by_hand():
    w = tiny()
    ctx, kv, _ = inputs(w)
    ctx = ctx.copy()
    ctx[0] = 0
    q = u16(wl.attention_query(w, 1))
    assert np.all(oracle.block_mass(q, kv, ctx, 0.1)[0] == 0)
    pred = np.array([[[1, 2, 3, -1]]], dtype=np.int32)
    true = np.array([[[2, 3, 4, 7]]], dtype=np.int32)
    a = oracle.agreement(pred, np.array([[3]]), true, np.array([[3]]))
    assert a[0, 0] == 2 / 3
    assert oracle.agreement(pred, np.array([[3]]), true, np.array([[0]]))[0, 0] == 1.0
