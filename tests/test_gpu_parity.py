"""Parity of the HIP path (through the C ABI) against the CPU oracle.

Both sides receive the same seeded inputs from `workloads`; nothing the GPU
computes is fed to the oracle.  Bars: integer work (summaries, selections on
shared scores, staging state, copied bytes) bit-exact; scores within one fp32
ulp (both round an fp64 sum of exact products); selections on each side's own
scores equal except for swaps between blocks tied within 1e-6 relative;
attention |out - ref| <= 2e-3 + 1e-2 |ref| against the fp64 oracle.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from helpers import (assert_attn_close, assert_scores_close, assert_selection_matches,
                     bf16_to_f64, gpu_stage_state, n_blocks, u16)

pytestmark = pytest.mark.gpu

DEV = "cuda"


def oa():
    import prefetch_block_scoring_amd as m
    return m


def small_workloads():
    W = wl.WORKLOADS
    return [
        W["parity_8q2kv_4k"],
        W["qwen3_8b_16k_b32_hbm"].shrink(B=2),
        W["reasoning_32k_b64_j4"].shrink(B=2, ctx=8192 + 5),
        W["gqa32b_ragged_b16_staged"].shrink(B=3, ctx=(100, 5000), cap=None),
        wl.Workload("odd_g3_ragged", B=4, H_q=12, H_kv=4, ctx=(1, 700), budget=160, J=2,
                    structure="none", seed=77),
        wl.Workload("g1_g16", B=2, H_q=16, H_kv=1, ctx=(17, 300), budget=64, J=1,
                    structure="none", seed=78),
    ]


IDS = [w.name for w in small_workloads()]


class Inputs:
    def __init__(self, w):
        self.w = w
        self.ctx_cpu = wl.context_lengths(w)
        self.kv_cpu = wl.kv_pool(w)
        self.ql_cpu = wl.lookahead(w, 0)
        self.q_cpu = wl.attention_query(w, 1)
        self.ctx = self.ctx_cpu.to(DEV)
        self.kv = self.kv_cpu.to(DEV)
        self.ql = self.ql_cpu.to(DEV)
        self.q = self.q_cpu.to(DEV)
        self.ctx_np = self.ctx_cpu.numpy()
        self.kv_np = u16(self.kv_cpu)
        self.ql_np = u16(self.ql_cpu)
        self.q_np = u16(self.q_cpu)


_cache = {}


def inputs(w):
    if w.name not in _cache:
        _cache[w.name] = Inputs(w)
    return _cache[w.name]


# ---------------------------------------------------------------- summaries / scores


@pytest.mark.parametrize("w", small_workloads(), ids=IDS)
def test_summaries_bit_exact(w):
    x = inputs(w)
    got = u16(oa().oasis_build_summaries(x.kv, x.ctx))
    ref = oracle.build_summaries(x.kv_np, x.ctx_np, w.bs)
    for r in range(w.B):
        nb = n_blocks(x.ctx_np[r])
        np.testing.assert_array_equal(bf16_to_f64(got[r, :, :nb]), bf16_to_f64(ref[r, :, :nb]))


@pytest.mark.parametrize("w", small_workloads(), ids=IDS)
def test_scores_within_one_ulp(w):
    x = inputs(w)
    summ = oa().oasis_build_summaries(x.kv, x.ctx)
    got = oa().oasis_score_blocks(x.ql, summ, x.ctx).cpu().numpy()
    ref = oracle.score(x.ql_np, oracle.build_summaries(x.kv_np, x.ctx_np, w.bs), x.ctx_np, w.bs, w.H_kv)
    assert_scores_close(got, ref, x.ctx_np)


def test_scores_from_host_pool_summaries():
    """Summaries built straight from a pinned host pool match the oracle."""
    w = small_workloads()[0]
    x = inputs(w)
    host = x.kv_cpu.pin_memory()
    got = u16(oa().oasis_build_summaries(host, x.ctx))
    ref = oracle.build_summaries(x.kv_np, x.ctx_np, w.bs)
    np.testing.assert_array_equal(got, ref)


# ---------------------------------------------------------------- selection


@pytest.mark.parametrize("ties", [0, 2, 50])
@pytest.mark.parametrize("w", small_workloads(), ids=IDS)
def test_select_bit_exact_on_shared_scores(w, ties):
    x = inputs(w)
    sc = wl.random_scores(w, tie_levels=ties)
    sel, n = oa().oasis_select_topk(sc.to(DEV), x.ctx, w.K_b)
    rsel, rn = oracle.select(sc.numpy(), x.ctx_np, w.bs, w.K_b)
    np.testing.assert_array_equal(n.cpu().numpy(), rn)
    np.testing.assert_array_equal(sel.cpu().numpy(), rsel)


def test_select_special_values():
    """NaN below -inf, -0 equal to +0 (ties by id), short rows take all."""
    w = wl.Workload("sv", B=2, H_q=2, H_kv=2, ctx=(40, 40), budget=32, structure="none")
    sc = torch.tensor([[[float("nan"), float("-inf"), 1.0], [-0.0, 0.0, -1.0]],
                       [[2.0, float("nan"), float("nan")], [float("inf"), -2.0, float("inf")]]])
    ctx = torch.tensor([40, 40], dtype=torch.int32)
    sel, n = oa().oasis_select_topk(sc.to(DEV), ctx.to(DEV), 2)
    rsel, rn = oracle.select(sc.numpy(), ctx.numpy(), 16, 2)
    np.testing.assert_array_equal(sel.cpu().numpy(), rsel)
    assert rsel.tolist() == [[[1, 2], [0, 1]], [[0, 1], [0, 2]]]


@pytest.mark.parametrize("w", small_workloads(), ids=IDS)
def test_selection_chain_matches_oracle(w):
    x = inputs(w)
    summ = oa().oasis_build_summaries(x.kv, x.ctx)
    sc = oa().oasis_score_blocks(x.ql, summ, x.ctx)
    sel, n = oa().oasis_select_topk(sc, x.ctx, w.K_b)
    rsc = oracle.score(x.ql_np, oracle.build_summaries(x.kv_np, x.ctx_np, w.bs), x.ctx_np, w.bs, w.H_kv)
    rsel, rn = oracle.select(rsc, x.ctx_np, w.bs, w.K_b)
    assert_selection_matches(sel.cpu().numpy(), n.cpu().numpy(), rsel, rn, rsc)
    if w.structure == "planted" and w.planted:
        s = sel.cpu().numpy()
        for r, heads in enumerate(wl.planted_blocks(w)):
            for h, planted in enumerate(heads):
                assert set(planted) <= set(s[r, h].tolist())


# ---------------------------------------------------------------- attention


def attn_ref(x, tbl, n, sm):
    return oracle.attend(x.q_np, x.kv_np, x.ctx_np, tbl, n, sm)


@pytest.mark.parametrize("n_split", [0, 1, 3])
@pytest.mark.parametrize("T", [1, 7, 128])
@pytest.mark.parametrize("w", small_workloads(), ids=IDS)
def test_attention_full_pool(w, T, n_split):
    x = inputs(w)
    tbl, n = wl.random_table(w, T, seed_index=T)
    sm = 1.0 / math.sqrt(w.D)
    out, lse = oa().oasis_sparse_decode_attn(x.q, x.kv, tbl.to(DEV), tbl.to(DEV), n.to(DEV), x.ctx,
                                             sm_scale=sm, n_split=n_split, want_lse=True)
    ref, ref_lse = attn_ref(x, tbl.numpy(), n.numpy(), sm)
    assert_attn_close(bf16_to_f64(u16(out)), ref)
    np.testing.assert_allclose(lse.cpu().numpy(), ref_lse, rtol=1e-5, atol=1e-4)


def test_attention_working_set_slots_and_invalid_entries():
    """Blocks placed at shuffled slots of a smaller pool; entries with an
    out-of-range slot or block id are skipped; an empty row gives zeros."""
    w = small_workloads()[3]
    x = inputs(w)
    T = 40
    tbl, n = wl.random_table(w, T, seed_index=5)
    S = T + 3
    g = torch.Generator().manual_seed(9)
    ws = torch.zeros((w.B, w.H_kv, S, 2, w.bs, w.D), dtype=torch.bfloat16)
    slots = torch.full_like(tbl, -1)
    for r in range(w.B):
        for h in range(w.H_kv):
            perm = torch.randperm(S, generator=g)
            for i in range(int(n[r, h])):
                ws[r, h, perm[i]] = x.kv_cpu[r, h, tbl[r, h, i]]
                slots[r, h, i] = perm[i]
    ref_tbl = tbl.clone()
    # corrupt entries: these must be skipped by the kernel and are dropped from the reference
    bad_tbl, bad_slots, ref_n = tbl.clone(), slots.clone(), n.clone()
    bad_slots[0, 0, 0] = S + 5            # slot out of range
    bad_tbl[0, 1, 1] = 10 ** 6            # block out of range
    ref_tbl[0, 0, 0] = -1
    ref_tbl[0, 1, 1] = -1
    n_zero = n.clone()
    n_zero[1, 0] = 0                      # empty row
    ref_n = n_zero
    sm = 0.05
    out, lse = oa().oasis_sparse_decode_attn(x.q, ws.to(DEV), bad_slots.to(DEV), bad_tbl.to(DEV),
                                             n_zero.to(DEV), x.ctx, sm_scale=sm, want_lse=True)
    ref, ref_lse = attn_ref(x, ref_tbl.numpy(), ref_n.numpy(), sm)
    assert_attn_close(bf16_to_f64(u16(out)), ref)
    o = out.cpu()
    G = w.G
    assert torch.all(o[1, 0:G] == 0)
    assert torch.all(torch.isneginf(lse.cpu()[1, 0:G]))


def test_attention_budget_equal_to_context_is_dense():
    """Listing every block reproduces dense softmax attention (the oracle's
    dense case is pinned against NumPy in the CPU suite)."""
    w = small_workloads()[4]
    x = inputs(w)
    T = w.NB_max
    tbl = torch.full((w.B, w.H_kv, T), -1, dtype=torch.int32)
    n = torch.zeros((w.B, w.H_kv), dtype=torch.int32)
    for r in range(w.B):
        nb = n_blocks(x.ctx_np[r])
        tbl[r, :, :nb] = torch.arange(nb, dtype=torch.int32)
        n[r] = nb
    sm = 1 / math.sqrt(128)
    out = oa().oasis_sparse_decode_attn(x.q, x.kv, tbl.to(DEV), tbl.to(DEV), n.to(DEV), x.ctx, sm_scale=sm)
    ref, _ = attn_ref(x, tbl.numpy(), n.numpy(), sm)
    assert_attn_close(bf16_to_f64(u16(out)), ref)


# ---------------------------------------------------------------- staging


@pytest.mark.parametrize("copy_mode,stage_blocks,split", [(0, 0, False), (1, 7, False), (1, 4096, False),
                                                         (0, 0, True), (1, 64, True)])
@pytest.mark.parametrize("C,turnover", [(1, 3), (6, 5), (6, 30)])
def test_stage_matches_oracle(copy_mode, stage_blocks, split, C, turnover):
    """Both copy engines, through oasis_stage_blocks or its two halves; the
    DMA engine with a 7-block staging buffer moves every step in rounds."""
    w = wl.Workload("stage", B=3, H_q=8, H_kv=2, ctx=(1500, 3000), budget=512, J=1,
                    structure="none", seed=31)
    K_b, NB, steps = w.K_b, w.NB_max, 6
    S = K_b + C
    ctx_cpu = wl.context_lengths(w)
    host = oa().oasis_host_empty((w.B, w.H_kv, NB, 2, w.bs, w.D))
    host.copy_(wl.kv_pool(w))
    host_np = u16(host)
    sels, nsels, scores = wl.predicted_set_sequence(w, steps, turnover)
    dev = lambda t: t.to(DEV)
    slot_block = torch.full((w.B, w.H_kv, S), -1, dtype=torch.int32, device=DEV)
    slot_stamp = torch.full((w.B, w.H_kv, S), -1, dtype=torch.int32, device=DEV)
    ws = torch.zeros((w.B, w.H_kv, S, 2, w.bs, w.D), dtype=torch.bfloat16, device=DEV)
    tbl_slot = torch.empty((w.B, w.H_kv, K_b), dtype=torch.int32, device=DEV)
    tbl_block = torch.empty_like(tbl_slot)
    tbl_n = torch.empty((w.B, w.H_kv), dtype=torch.int32, device=DEV)
    nbytes = oa().oasis_stage_plan_bytes(w.B, w.H_kv, K_b)
    plan = torch.empty(nbytes // 4, dtype=torch.int32, device=DEV)
    host_plan = torch.empty(nbytes // 4, dtype=torch.int32).pin_memory()
    sbytes = oa().oasis_stage_buffer_bytes(max(stage_blocks, 1))
    stage_host = [torch.empty(sbytes, dtype=torch.uint8).pin_memory() for _ in range(2)]
    stage_dev = torch.empty(sbytes, dtype=torch.uint8, device=DEV)
    ctx = dev(ctx_cpu)
    copy_stream = torch.cuda.Stream()
    accum = torch.zeros(4, dtype=torch.int64, device=DEV)
    st = oracle.StageState(w.B, w.H_kv, NB)
    totals = np.zeros(4, dtype=np.int64)
    for s in range(steps):
        Cs = K_b if s == 0 else C
        kw = dict(sel=dev(sels[s]), n_sel=dev(nsels[s]), scores=dev(scores[s]), ctx_len=ctx,
                  K_b=K_b, C=Cs, step=s, slot_block=slot_block, slot_stamp=slot_stamp,
                  host_pool=host, ws_pool=ws, tbl_slot=tbl_slot, tbl_block=tbl_block,
                  tbl_n=tbl_n, plan=plan, host_plan=host_plan, stage_host=stage_host[s % 2],
                  stage_dev=stage_dev, copy_mode=copy_mode, stats_accum=accum)
        if split:
            planned = torch.cuda.Event()
            oa().oasis_stage_plan(plan_event=planned, **kw)
            oa().oasis_stage_copy(plan_event=planned, copy_stream=copy_stream, **kw)
            stats = oa().oasis_stage_read_stats(plan, w.B, w.H_kv, Cs)
        else:
            stats = oa().oasis_stage_blocks(want_stats=True, **kw)
        torch.cuda.synchronize()
        adm, na, ev, ne = oracle.stage(st, sels[s].numpy(), nsels[s].numpy(), scores[s].numpy(),
                                       ctx_cpu.numpy(), w.bs, K_b, Cs, s)
        got = gpu_stage_state(slot_block, slot_stamp, NB)
        np.testing.assert_array_equal(got, st.stamp, err_msg=f"step {s}")
        row = 4 + 2 * max(Cs, 1)
        flat = plan.cpu().numpy()
        p = flat[: w.B * w.H_kv * row].reshape(w.B, w.H_kv, row)
        np.testing.assert_array_equal(p[:, :, 0], na)
        np.testing.assert_array_equal(p[:, :, 1], ne)
        # packed positions: running total of admits in (r, h) order
        np.testing.assert_array_equal(p[:, :, 2].ravel(), np.concatenate([[0], np.cumsum(na.ravel())[:-1]]))
        # deferred admits: predicted blocks the cap held back
        np.testing.assert_array_equal(p[:, :, 3], st.deferred)
        tail = flat[w.B * w.H_kv * row: w.B * w.H_kv * row + 4]
        assert tail.tolist() == [na.sum(), ne.sum(), st.deferred.sum(), (st.deferred > 0).sum()]
        assert stats == {"admits": na.sum(), "evictions": ne.sum(), "deferred": st.deferred.sum(),
                         "capped_pairs": (st.deferred > 0).sum(), "bytes": na.sum() * 8192}
        totals += [na.sum(), ne.sum(), st.deferred.sum(), 1]
        assert accum.cpu().tolist() == totals.tolist()
        for r in range(w.B):
            for h in range(w.H_kv):
                k = int(na[r, h])
                assert p[r, h, 5:5 + 2 * k:2].tolist() == adm[r, h, :k].tolist()
        # table lists exactly the held slots; every held slot holds its host block's bytes
        wsn = u16(ws)
        sb = slot_block.cpu().numpy()
        tn, tsl, tbk = tbl_n.cpu().numpy(), tbl_slot.cpu().numpy(), tbl_block.cpu().numpy()
        for r in range(w.B):
            for h in range(w.H_kv):
                held = [i for i in range(S) if sb[r, h, i] >= 0]
                assert tn[r, h] == len(held)
                assert tsl[r, h, :len(held)].tolist() == held
                assert tbk[r, h, :len(held)].tolist() == [int(sb[r, h, i]) for i in held]
                for i in held:
                    assert np.array_equal(wsn[r, h, i], host_np[r, h, sb[r, h, i]]), (s, r, h, i)


# ---------------------------------------------------------------- whole chain


def run_chain_gpu(w, steps, C, copy_mode=0):
    """score -> select -> stage -> attend for `steps` steps; returns per-step
    (scores, sel, n_sel, stamps, out, attended blocks, their count) on the
    CPU."""
    m = oa()
    ctx_cpu = wl.context_lengths(w)
    ctx = ctx_cpu.to(DEV)
    host = wl.kv_pool(w).pin_memory()
    summ = m.oasis_build_summaries(host, ctx)
    K_b, S = w.K_b, w.K_b + C
    slot_block = torch.full((w.B, w.H_kv, S), -1, dtype=torch.int32, device=DEV)
    slot_stamp = torch.full_like(slot_block, -1)
    ws = torch.zeros((w.B, w.H_kv, S, 2, w.bs, w.D), dtype=torch.bfloat16, device=DEV)
    tabs = [(torch.empty((w.B, w.H_kv, K_b), dtype=torch.int32, device=DEV),
             torch.empty((w.B, w.H_kv, K_b), dtype=torch.int32, device=DEV),
             torch.zeros((w.B, w.H_kv), dtype=torch.int32, device=DEV)) for _ in range(2)]
    plan = torch.empty(m.oasis_stage_plan_bytes(w.B, w.H_kv, K_b) // 4, dtype=torch.int32, device=DEV)
    host_plan = torch.empty(plan.numel(), dtype=torch.int32).pin_memory()
    sbytes = m.oasis_stage_buffer_bytes(w.B * w.H_kv * C)
    stage_host = torch.empty(sbytes, dtype=torch.uint8).pin_memory()
    stage_dev = torch.empty(sbytes, dtype=torch.uint8, device=DEV)
    hist = []
    for s in range(steps):
        ql = wl.lookahead(w, s).to(DEV)
        sc = m.oasis_score_blocks(ql, summ, ctx)
        sel, n = m.oasis_select_topk(sc, ctx, K_b)
        t = tabs[s % 2]
        m.oasis_stage_blocks(sel=sel, n_sel=n, scores=sc, ctx_len=ctx, K_b=K_b, C=K_b if s == 0 else C,
                             step=s, slot_block=slot_block, slot_stamp=slot_stamp, host_pool=host,
                             ws_pool=ws, tbl_slot=t[0], tbl_block=t[1], tbl_n=t[2], plan=plan,
                             host_plan=host_plan, stage_host=stage_host, stage_dev=stage_dev,
                             copy_mode=copy_mode)
        q = wl.attention_query(w, s + 1).to(DEV)
        out = m.oasis_sparse_decode_attn(q, ws, t[0], t[1], t[2], ctx)
        torch.cuda.synchronize()
        hist.append((sc.cpu().numpy(), sel.cpu().numpy(), n.cpu().numpy(),
                     gpu_stage_state(slot_block, slot_stamp, w.NB_max), u16(out),
                     t[1].cpu().numpy(), t[2].cpu().numpy()))
    return hist


@pytest.mark.parametrize("name,B,ctx", [("qwen3_8b_16k_b128_staged", 2, 16384),
                                        ("gqa32b_ragged_b16_staged", 2, (3000, 9000))])
@pytest.mark.parametrize("copy_mode", [0, 1])
def test_chain_end_to_end(name, B, ctx, copy_mode):
    """Every step is compared in full.  Scores and the selection against the
    oracle's own (the selection up to tied swaps); the staging step by
    running the oracle's stage on the GPU's selection and scores, so the two
    states follow the same predictions even after a tied swap; attention
    against the oracle's attention over the GPU's resident set."""
    w = wl.WORKLOADS[name].shrink(B=B, ctx=ctx)
    C = oracle.fetch_cap_blocks(w.cap, w.K_b)
    steps = 5
    g = run_chain_gpu(w, steps, C, copy_mode)
    ctx_np = wl.context_lengths(w).numpy()
    kv = u16(wl.kv_pool(w))
    summ = oracle.build_summaries(kv, ctx_np, w.bs)
    st = oracle.StageState(w.B, w.H_kv, w.NB_max)
    compared = 0
    for s in range(steps):
        gs, gsel, gn, gst, gout, gblk, gnblk = g[s]
        os_ = oracle.score(u16(wl.lookahead(w, s)), summ, ctx_np, w.bs, w.H_kv)
        osel, on = oracle.select(os_, ctx_np, w.bs, w.K_b)
        assert_scores_close(gs, os_, ctx_np)
        assert_selection_matches(gsel, gn, osel, on, os_)
        oracle.stage(st, gsel, gn, gs, ctx_np, w.bs, w.K_b, w.K_b if s == 0 else C, s)
        np.testing.assert_array_equal(gst, st.stamp, err_msg=f"step {s}")
        for r in range(w.B):
            for h in range(w.H_kv):
                assert sorted(gblk[r, h, :gnblk[r, h]].tolist()) == st.resident(r, h).tolist()
        oout, _ = oracle.attend(u16(wl.attention_query(w, s + 1)), kv, ctx_np, gblk, gnblk, 1 / math.sqrt(w.D))
        assert_attn_close(bf16_to_f64(gout), oout)
        compared += 1
    assert compared == steps


ODD_SHAPES = [
    # name, B, H_q, H_kv, ctx, budget (tokens), J, cap, structure, copy engine
    ("g1_tiny", 6, 4, 4, (1, 120), 96, 1, 0.1, "drift", 0),
    ("g16_j2", 2, 32, 2, (900, 2100), 272, 2, 0.07, "drift", 1),
    ("g2_j3", 5, 16, 8, (100, 5000), 208, 3, 0.2, "none", 0),
    ("g8_hkv3", 1, 24, 3, 3333, 512, 1, 0.02, "drift", 1),
    ("g8_hkv1_zipf", 4, 8, 1, (2000, 6000), 1024, 4, 0.05, "zipf", 0),
    ("g3_fetch_all", 7, 12, 4, (16, 1600), 160, 1, 1.0, "none", 1),
]


@pytest.mark.parametrize("name,B,H_q,H_kv,ctx,budget,J,cap,structure,copy_mode", ODD_SHAPES,
                         ids=[x[0] for x in ODD_SHAPES])
def test_odd_shapes_chain_matches_oracle(name, B, H_q, H_kv, ctx, budget, J, cap, structure, copy_mode):
    """The staged chain on shapes away from the workloads: groups of 1, 2, 3,
    8 and 16 query heads, one or three KV heads, budgets that are not
    multiples of 64 blocks' worth, contexts from one token to many blocks
    past the budget, up to four drafts, caps from one block to fetch-all.
    Each step is compared in full, as in test_chain_end_to_end."""
    w = wl.Workload(name, B=B, H_q=H_q, H_kv=H_kv, ctx=ctx, budget=budget, J=J, cap=cap, structure=structure,
                    seed=97)
    C = oracle.fetch_cap_blocks(cap, w.K_b)
    steps = 4
    g = run_chain_gpu(w, steps, C, copy_mode)
    ctx_np = wl.context_lengths(w).numpy()
    kv = u16(wl.kv_pool(w))
    summ = oracle.build_summaries(kv, ctx_np, w.bs)
    st = oracle.StageState(w.B, w.H_kv, w.NB_max)
    for s in range(steps):
        gs, gsel, gn, gst, gout, gblk, gnblk = g[s]
        os_ = oracle.score(u16(wl.lookahead(w, s)), summ, ctx_np, w.bs, w.H_kv)
        osel, on = oracle.select(os_, ctx_np, w.bs, w.K_b)
        assert_scores_close(gs, os_, ctx_np)
        assert_selection_matches(gsel, gn, osel, on, os_)
        oracle.stage(st, gsel, gn, gs, ctx_np, w.bs, w.K_b, w.K_b if s == 0 else C, s)
        np.testing.assert_array_equal(gst, st.stamp, err_msg=f"step {s}")
        for r in range(w.B):
            for h in range(w.H_kv):
                assert sorted(gblk[r, h, :gnblk[r, h]].tolist()) == st.resident(r, h).tolist()
        oout, _ = oracle.attend(u16(wl.attention_query(w, s + 1)), kv, ctx_np, gblk, gnblk, 1 / math.sqrt(w.D))
        assert_attn_close(bf16_to_f64(gout), oout)


# ---------------------------------------------------------------- pipelined layers


@pytest.mark.parametrize("copy_mode,joint,compute_streams,issue_threads",
                         [(0, False, 0, 0), (1, False, 0, 0), (0, True, 0, 0), (0, False, 1, 0), (1, False, 1, 0),
                          (2, False, 0, 0), (2, False, 1, 0), (0, False, -1, 0), (1, False, -1, 0),
                          (0, False, 0, -1), (1, False, 0, -1), (2, False, 0, -1)])
def test_layer_pipeline_matches_oracle(copy_mode, joint, compute_streams, issue_threads):
    """Three layers in flight on separate streams (the schedule the benchmark
    times): every layer's attention output at every step equals the oracle
    chain run serially for that layer.  joint: look-ahead attention of the
    normal query and the step's draft queries (n_q = 1 + J), each query
    against the oracle's attention for it alone.  compute_streams 0 is the
    automatic choice (two here: 16 (request, KV head) pairs); 1 puts every
    layer's scores, top-K and plan on one stream beside two copy streams;
    -1 runs them on the main stream after each layer's attention.
    issue_threads 0: with compute streams of their own, worker threads
    enqueue the chain and the copies; -1: the calling thread enqueues all.
    copy_mode 2 (mixed): layers 0 and 2 stage through the DMA engine, layer 1
    through the gather kernel."""
    from prefetch_block_scoring_amd.pipeline import LayerPipeline
    m = oa()
    w = wl.WORKLOADS["qwen3_8b_16k_b128_staged"].shrink(B=2, ctx=(3000, 9000))
    C = oracle.fetch_cap_blocks(w.cap, w.K_b)
    L, steps = 3, 6
    ctx_cpu = wl.context_lengths(w)
    ctx = ctx_cpu.to(DEV)
    host = m.oasis_host_empty((w.B, w.H_kv, w.NB_max, 2, w.bs, w.D))
    host.copy_(wl.kv_pool(w))
    summ = m.oasis_build_summaries(host, ctx)
    looks = [wl.lookahead(w, s).to(DEV) for s in range(steps + 2 * L)]
    attn_q = [looks[max(s - 1, 0)][:, 0].contiguous() for s in range(steps + 2 * L)]
    if joint:
        attn_q = [torch.cat([attn_q[s][:, None], looks[s]], dim=1).contiguous() for s in range(steps + 2 * L)]
    n_q = 1 + w.J if joint else 1
    pipe = LayerPipeline(pool=host, summ=summ, ctx=ctx, H_q=w.H_q, K_b=w.K_b, C=C, n_layers=L, staged=True, J=w.J,
                         copy_mode=copy_mode, host_threads=4, n_q=n_q, compute_streams=compute_streams,
                         issue_threads=issue_threads)
    assert pipe.compute_streams == (compute_streams or 2)
    assert pipe.issue_threads == (compute_streams != -1 and issue_threads == 0)
    outs = {}
    for t in range(steps):
        for l in range(L):
            s = t + 2 * l
            pipe.layer_step(l, t, looks[s], attn_q[s])
            if t >= 1:
                # stream-ordered snapshot on the main stream: no host wait, so
                # the compute and copy streams keep running ahead as they would
                with torch.cuda.stream(pipe.main):
                    outs[(l, t)] = pipe.layers[l].out.clone()
    pipe.close()
    torch.cuda.synchronize()
    outs = {k: u16(v) for k, v in outs.items()}
    # oracle: per layer, the serial chain with the same lookahead phase
    ctx_np = ctx_cpu.numpy()
    kv = u16(host)
    summ_o = oracle.build_summaries(kv, ctx_np, w.bs)
    for l in range(L):
        st = oracle.StageState(w.B, w.H_kv, w.NB_max)
        for t in range(steps - 1):
            s = t + 2 * l
            sc = oracle.score(u16(looks[s]), summ_o, ctx_np, w.bs, w.H_kv)
            sel, n = oracle.select(sc, ctx_np, w.bs, w.K_b)
            oracle.stage(st, sel, n, sc, ctx_np, w.bs, w.K_b, w.K_b if t == 0 else C, t)
            blocks = np.full((w.B, w.H_kv, w.K_b), -1, dtype=np.int32)
            nb = np.zeros((w.B, w.H_kv), dtype=np.int32)
            for r in range(w.B):
                for h in range(w.H_kv):
                    res = st.resident(r, h)
                    blocks[r, h, :len(res)] = res
                    nb[r, h] = len(res)
            got = bf16_to_f64(outs[(l, t + 1)])
            if not joint:
                ref, _ = oracle.attend(u16(attn_q[s + 1]), kv, ctx_np, blocks, nb, 1 / math.sqrt(w.D))
                assert_attn_close(got, ref)
                continue
            for qi in range(n_q):
                ref, _ = oracle.attend(u16(attn_q[s + 1][:, qi]), kv, ctx_np, blocks, nb, 1 / math.sqrt(w.D))
                assert_attn_close(got[:, qi], ref)


@pytest.mark.parametrize("compute_streams,issue_threads", [(0, 0), (0, -1), (2, 1), (2, -1), (-1, 0)])
def test_unstaged_pipeline_matches_oracle(compute_streams, issue_threads):
    """The pipeline with K/V in HBM (no staging), three layers in flight:
    every layer's attention at step t + 1 over the blocks the oracle selects
    at step t equals the oracle's.  issue_threads 0 (automatic) and 1: a
    worker thread enqueues the scores and top-K, and the calling thread waits
    for the selection of step t - 1 on the host before it enqueues the
    attention; -1: stream waits.  compute_streams 0 is the automatic choice
    (one stream); -1 runs the chain on the main stream (no issue threads)."""
    from prefetch_block_scoring_amd.pipeline import LayerPipeline
    w = wl.WORKLOADS["qwen3_8b_16k_b32_hbm"].shrink(B=3, ctx=(3000, 9000))
    L, steps = 3, 6
    ctx_cpu = wl.context_lengths(w)
    ctx = ctx_cpu.to(DEV)
    pool = wl.kv_pool(w, device=DEV)
    summ = oa().oasis_build_summaries(pool, ctx)
    looks = [wl.lookahead(w, s).to(DEV) for s in range(steps + 2 * L)]
    attn_q = [looks[max(s - 1, 0)][:, 0].contiguous() for s in range(steps + 2 * L)]
    pipe = LayerPipeline(pool=pool, summ=summ, ctx=ctx, H_q=w.H_q, K_b=w.K_b, C=0, n_layers=L, staged=False, J=w.J,
                         compute_streams=compute_streams, issue_threads=issue_threads)
    assert pipe.compute_streams == (compute_streams or 1)
    assert pipe.issue_threads == (issue_threads >= 0 and compute_streams != -1)
    outs = {}
    for t in range(steps):
        for l in range(L):
            s = t + 2 * l
            pipe.layer_step(l, t, looks[s], attn_q[s])
            if t >= 1:
                with torch.cuda.stream(pipe.main):
                    outs[(l, t)] = pipe.layers[l].out.clone()
    pipe.close()
    torch.cuda.synchronize()
    ctx_np = ctx_cpu.numpy()
    kv = u16(pool)
    summ_o = oracle.build_summaries(kv, ctx_np, w.bs)
    for l in range(L):
        for t in range(steps - 1):
            s = t + 2 * l
            sc = oracle.score(u16(looks[s]), summ_o, ctx_np, w.bs, w.H_kv)
            sel, n = oracle.select(sc, ctx_np, w.bs, w.K_b)
            ref, _ = oracle.attend(u16(attn_q[s + 1]), kv, ctx_np, sel, n, 1 / math.sqrt(w.D))
            assert_attn_close(bf16_to_f64(u16(outs[(l, t + 1)])), ref)


ODD_PIPELINES = [
    # name, B, H_q, H_kv, ctx, budget, J, cap (None: K/V in HBM), structure, copy engine
    ("g16_zero_copy", 2, 32, 2, (900, 2100), 272, 2, 0.07, "drift", 0),
    ("g3_fetch_all_dma", 3, 12, 4, (16, 1600), 160, 1, 1.0, "none", 1),
    ("g8_hkv1_mixed", 2, 8, 1, (2000, 6000), 1024, 4, 0.05, "zipf", 2),
    ("g1_hbm", 3, 4, 4, (1, 900), 96, 1, None, "none", 0),
]


@pytest.mark.parametrize("name,B,H_q,H_kv,ctx,budget,J,cap,structure,copy_mode", ODD_PIPELINES,
                         ids=[x[0] for x in ODD_PIPELINES])
def test_odd_shapes_pipeline_matches_oracle(name, B, H_q, H_kv, ctx, budget, J, cap, structure, copy_mode):
    """The layer pipeline (three layers in flight, automatic streams and
    issue threads) on shapes away from the workloads, staged through each
    copy engine or with K/V in HBM: every layer's attention output at every
    step equals the oracle chain run serially for that layer."""
    from prefetch_block_scoring_amd.pipeline import LayerPipeline
    m = oa()
    staged = cap is not None
    w = wl.Workload(name, B=B, H_q=H_q, H_kv=H_kv, ctx=ctx, budget=budget, J=J, cap=cap, structure=structure,
                    seed=101)
    C = oracle.fetch_cap_blocks(cap, w.K_b) if staged else 0
    L, steps = 3, 5
    ctx_cpu = wl.context_lengths(w)
    ctx = ctx_cpu.to(DEV)
    if staged:
        pool = m.oasis_host_empty((w.B, w.H_kv, w.NB_max, 2, w.bs, w.D))
        pool.copy_(wl.kv_pool(w))
    else:
        pool = wl.kv_pool(w, device=DEV)
    summ = m.oasis_build_summaries(pool, ctx)
    looks = [wl.lookahead(w, s).to(DEV) for s in range(steps + 2 * L)]
    attn_q = [looks[max(s - 1, 0)][:, 0].contiguous() for s in range(steps + 2 * L)]
    pipe = LayerPipeline(pool=pool, summ=summ, ctx=ctx, H_q=w.H_q, K_b=w.K_b, C=C, n_layers=L, staged=staged,
                         J=w.J, copy_mode=copy_mode, host_threads=4)
    outs = {}
    for t in range(steps):
        for l in range(L):
            s = t + 2 * l
            pipe.layer_step(l, t, looks[s], attn_q[s])
            if t >= 1:
                with torch.cuda.stream(pipe.main):
                    outs[(l, t)] = pipe.layers[l].out.clone()
    pipe.close()
    torch.cuda.synchronize()
    outs = {k: u16(v) for k, v in outs.items()}
    ctx_np = ctx_cpu.numpy()
    kv = u16(pool)
    summ_o = oracle.build_summaries(kv, ctx_np, w.bs)
    for l in range(L):
        st = oracle.StageState(w.B, w.H_kv, w.NB_max)
        for t in range(steps - 1):
            s = t + 2 * l
            sc = oracle.score(u16(looks[s]), summ_o, ctx_np, w.bs, w.H_kv)
            sel, n = oracle.select(sc, ctx_np, w.bs, w.K_b)
            if staged:
                oracle.stage(st, sel, n, sc, ctx_np, w.bs, w.K_b, w.K_b if t == 0 else C, t)
                sel = np.full((w.B, w.H_kv, w.K_b), -1, dtype=np.int32)
                n = np.zeros((w.B, w.H_kv), dtype=np.int32)
                for r in range(w.B):
                    for h in range(w.H_kv):
                        res = st.resident(r, h)
                        sel[r, h, :len(res)] = res
                        n[r, h] = len(res)
            ref, _ = oracle.attend(u16(attn_q[s + 1]), kv, ctx_np, sel, n, 1 / math.sqrt(w.D))
            assert_attn_close(bf16_to_f64(outs[(l, t + 1)]), ref)


def test_pipeline_timing_values_match_totals():
    """Per-launch timings of the native pipeline: one value per timed launch
    of each kind (attention from step 1 on), all positive, summing to the
    kind's total; launches past the capacity are not timed."""
    from prefetch_block_scoring_amd.pipeline import LayerPipeline
    m = oa()
    w = wl.WORKLOADS["qwen3_8b_16k_b128_staged"].shrink(B=2, ctx=(3000, 9000))
    C = oracle.fetch_cap_blocks(w.cap, w.K_b)
    L, steps, cap = 2, 5, 6
    ctx = wl.context_lengths(w).to(DEV)
    host = m.oasis_host_empty((w.B, w.H_kv, w.NB_max, 2, w.bs, w.D))
    host.copy_(wl.kv_pool(w))
    summ = m.oasis_build_summaries(host, ctx)
    looks = [wl.lookahead(w, s).to(DEV) for s in range(steps)]
    attn_q = [looks[max(s - 1, 0)][:, 0].contiguous() for s in range(steps)]
    pipe = LayerPipeline(pool=host, summ=summ, ctx=ctx, H_q=w.H_q, K_b=w.K_b, C=C, n_layers=L, staged=True, J=w.J)
    pipe.enable_timing(cap, ("attn", "score", "topk", "plan"))
    for t in range(steps):
        for l in range(L):
            pipe.layer_step(l, t, looks[t], attn_q[t])
    launches = {"attn": (steps - 1) * L, "score": steps * L, "topk": steps * L, "plan": steps * L}
    for kind, n in launches.items():
        vals = pipe.timing_values(kind, 64)
        avg, count = pipe.timing(kind)
        assert count == min(n, cap) == len(vals), kind
        assert all(v > 0 for v in vals), kind
        assert abs(sum(vals) / count - avg) <= 1e-3 * avg + 1e-3, kind
    assert len(pipe.timing_values("attn", 2)) == 2
    pipe.close()


@pytest.mark.parametrize("staged", [True, False])
def test_pipeline_timing_rearm_keeps_results(staged):
    """The timing events are bound to the launches they time, and re-arming
    the timers binds them to later launches again.  Re-arming mid-run (with
    one launch in every 2, then every 3, timed) changes no result: every
    layer-step's attention output equals that of the same run without
    timing, bit for bit, and each kind counts the launches its stride
    picks."""
    from prefetch_block_scoring_amd.pipeline import LayerPipeline
    m = oa()
    name = "qwen3_8b_16k_b128_staged" if staged else "qwen3_8b_16k_b32_hbm"
    w = wl.WORKLOADS[name].shrink(B=3, ctx=(3000, 9000))
    C = oracle.fetch_cap_blocks(w.cap, w.K_b) if staged else 0
    L, steps = 3, 8
    kinds = ("attn", "score", "topk", "plan") if staged else ("attn", "score", "topk")
    ctx = wl.context_lengths(w).to(DEV)
    if staged:
        pool = m.oasis_host_empty((w.B, w.H_kv, w.NB_max, 2, w.bs, w.D))
        pool.copy_(wl.kv_pool(w))
    else:
        pool = wl.kv_pool(w, device=DEV)
    summ = m.oasis_build_summaries(pool, ctx)
    looks = [wl.lookahead(w, s).to(DEV) for s in range(steps)]
    attn_q = [looks[max(s - 1, 0)][:, 0].contiguous() for s in range(steps)]

    def run(timing):
        pipe = LayerPipeline(pool=pool, summ=summ, ctx=ctx, H_q=w.H_q, K_b=w.K_b, C=C, n_layers=L, staged=staged,
                             J=w.J)
        outs, counts = [], None
        if timing:
            pipe.enable_timing(64, kinds)
        for t in range(steps):
            if timing and t in (3, 5):
                pipe.enable_timing(64, kinds, every=2 if t == 3 else 3)
            for l in range(L):
                pipe.layer_step(l, t, looks[t], attn_q[t])
                if t >= 1:
                    # in stream order after the attention, without a host wait
                    with torch.cuda.stream(pipe.main):
                        outs.append(pipe.layers[l].out.clone())
        if timing:
            counts = {k: pipe.timing(k)[1] for k in kinds}
        pipe.drain()
        torch.cuda.synchronize()
        pipe.close()
        return outs, counts

    timed_outs, counts = run(True)
    plain_outs, _ = run(False)
    assert len(timed_outs) == len(plain_outs) == (steps - 1) * L
    for i, (a, b) in enumerate(zip(timed_outs, plain_outs)):
        assert torch.equal(a, b), f"layer-step {i}"
    # armed at step 5 with every = 3: steps 5..7 launch 3 * L of each kind
    assert counts == {k: -(-(steps - 5) * L // 3) for k in kinds}
