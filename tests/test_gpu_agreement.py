"""Lookahead-agreement analogue: exact per-block attention mass of the next
query (the true top-K side) and the overlap of two top-K lists, against the
oracle (whose block mass is pinned to a NumPy dense softmax in the CPU
suite).  Masses are fp32 sums of exponentials on the GPU, so they match the
fp64 oracle within 1e-6 + 1e-4 relative, and the true sets match except for
swaps of blocks whose oracle masses tie within 1e-4 relative."""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from helpers import assert_selection_matches, u16

pytestmark = pytest.mark.gpu

DEV = "cuda"


def oa():
    import prefetch_block_scoring_amd as m
    return m


W = wl.WORKLOADS
CASES = [
    W["parity_8q2kv_4k"],
    W["qwen3_8b_16k_b32_hbm"].shrink(B=2, ctx=8192 + 5),
    W["reasoning_32k_b64_j4"].shrink(B=2, ctx=(3000, 9000)),
    W["gqa32b_ragged_b16_staged"].shrink(B=3, ctx=(100, 5000), cap=None),
    wl.Workload("odd_g3_ragged", B=4, H_q=12, H_kv=4, ctx=(1, 700), budget=160, J=2, structure="none", seed=77),
    wl.Workload("g1_g16", B=2, H_q=16, H_kv=1, ctx=(17, 300), budget=64, J=1, structure="none", seed=78),
]
IDS = [w.name for w in CASES]


@pytest.mark.parametrize("sigma", [0.0, 0.5])
@pytest.mark.parametrize("w", CASES, ids=IDS)
def test_block_mass_and_true_set_match_oracle(w, sigma):
    m = oa()
    ctx_cpu = wl.context_lengths(w)
    kv_cpu = wl.kv_pool(w)
    q = wl.true_next_query(w, 2, sigma)
    sm = 1 / math.sqrt(w.D)
    ctx = ctx_cpu.to(DEV)
    mass = m.oasis_block_attention_mass(q.to(DEV), kv_cpu.to(DEV), ctx, sm_scale=sm)
    ref = oracle.block_mass(u16(q), u16(kv_cpu), ctx_cpu.numpy(), sm)
    got = mass.cpu().numpy().astype(np.float64)
    np.testing.assert_allclose(got, ref, rtol=1e-4, atol=1e-6)
    sel, n = m.oasis_select_topk(mass, ctx, w.K_b)
    rsel, rn = oracle.select(ref.astype(np.float32), ctx_cpu.numpy(), w.bs, w.K_b)
    assert_selection_matches(sel.cpu().numpy(), n.cpu().numpy(), rsel, rn, ref, rel=1e-4)


def test_block_mass_from_pinned_host_pool():
    m = oa()
    w = W["gqa32b_ragged_b16_staged"].shrink(B=2, ctx=(100, 3000))
    ctx_cpu = wl.context_lengths(w)
    kv_cpu = wl.kv_pool(w)
    host = m.oasis_host_empty(tuple(kv_cpu.shape))
    host.copy_(kv_cpu)
    q = wl.true_next_query(w, 1, 0.3)
    a = m.oasis_block_attention_mass(q.to(DEV), host, ctx_cpu.to(DEV))
    b = m.oasis_block_attention_mass(q.to(DEV), kv_cpu.to(DEV), ctx_cpu.to(DEV))
    assert torch.equal(a, b)


def test_topk_overlap_counts_set_intersections():
    m = oa()
    w = W["qwen3_8b_16k_b32_hbm"].shrink(B=3, ctx=(200, 4000))
    ctx = wl.context_lengths(w).to(DEV)
    sa, na = m.oasis_select_topk(wl.random_scores(w, 0).to(DEV), ctx, w.K_b)
    sb, nb = m.oasis_select_topk(wl.random_scores(w.shrink(seed=w.seed + 1), 3).to(DEV), ctx, w.K_b)
    ov = m.oasis_topk_overlap(sa, na, sb, nb).cpu().numpy()
    A, NA, B_, NB = sa.cpu().numpy(), na.cpu().numpy(), sb.cpu().numpy(), nb.cpu().numpy()
    for r in range(w.B):
        for h in range(w.H_kv):
            expect = len(set(A[r, h, :NA[r, h]].tolist()) & set(B_[r, h, :NB[r, h]].tolist()))
            assert ov[r, h] == expect
    agree = oracle.agreement(A, NA, B_, NB)
    np.testing.assert_allclose(ov / np.maximum(NB, 1), np.where(NB > 0, agree, 0.0))
