"""Look-ahead attention: the normal query and the draft queries of a request
attend over the same listed blocks in one pass (paperlayer summary,
section 4).  Parity: each query's output against the oracle's attention for
that query alone (the oracle's attention is pinned in the CPU suite), within
|out - ref| <= 2e-3 + 1e-2 |ref|; the single-query case is bit-identical to
oasis_sparse_decode_attn.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from helpers import assert_attn_close, bf16_to_f64, u16

pytestmark = pytest.mark.gpu

DEV = "cuda"


def oa():
    import prefetch_block_scoring_amd as m
    return m


W = wl.WORKLOADS
CASES = [
    # (workload, n_q): the columns n_q * G of one tile go from 2 to 16
    (W["parity_8q2kv_4k"], 1),
    (W["parity_8q2kv_4k"], 2),
    (W["parity_8q2kv_4k"], 4),
    (W["qwen3_8b_16k_b32_hbm"].shrink(B=2), 3),
    (W["gqa32b_ragged_b16_staged"].shrink(B=3, ctx=(100, 5000), cap=None), 2),
    (wl.Workload("odd_g3_ragged", B=4, H_q=12, H_kv=4, ctx=(1, 700), budget=160, J=2,
                 structure="none", seed=77), 5),
    (wl.Workload("g1_mha", B=2, H_q=4, H_kv=4, ctx=(17, 900), budget=128, J=1, structure="none",
                 seed=79), 16),
]
IDS = [f"{w.name}-nq{n_q}" for w, n_q in CASES]


def joint_queries(w, n_q):
    """[B][n_q][H_q][D]: the normal query of step 1 followed by further query
    vectors (the attention queries of later steps stand in for drafts)."""
    return torch.stack([wl.attention_query(w, 1 + k) for k in range(n_q)], dim=1).contiguous()


@pytest.mark.parametrize("n_split", [0, 3])
@pytest.mark.parametrize("T", [7, 128])
@pytest.mark.parametrize("w,n_q", CASES, ids=IDS)
def test_lookahead_attention_matches_per_query_oracle(w, n_q, T, n_split):
    ctx = wl.context_lengths(w)
    kv = wl.kv_pool(w)
    q = joint_queries(w, n_q)
    tbl, n = wl.random_table(w, T, seed_index=T)
    sm = 1.0 / math.sqrt(w.D)
    out, lse = oa().oasis_lookahead_attn(q.to(DEV), kv.to(DEV), tbl.to(DEV), tbl.to(DEV), n.to(DEV), ctx.to(DEV),
                                         sm_scale=sm, n_split=n_split, want_lse=True)
    assert out.shape == (w.B, n_q, w.H_q, w.D) and lse.shape == (w.B, n_q, w.H_q)
    got, got_lse = bf16_to_f64(u16(out)), lse.cpu().numpy()
    kv_np, ctx_np = u16(kv), ctx.numpy()
    for qi in range(n_q):
        ref, ref_lse = oracle.attend(u16(q[:, qi]), kv_np, ctx_np, tbl.numpy(), n.numpy(), sm)
        assert_attn_close(got[:, qi], ref)
        np.testing.assert_allclose(got_lse[:, qi], ref_lse, rtol=1e-5, atol=1e-4)


@pytest.mark.parametrize("n_split", [0, 2])
def test_single_query_is_decode_attention(n_split):
    w = W["qwen3_8b_16k_b32_hbm"].shrink(B=3)
    ctx, kv = wl.context_lengths(w).to(DEV), wl.kv_pool(w).to(DEV)
    q = wl.attention_query(w, 1).to(DEV)
    tbl, n = wl.random_table(w, 128, seed_index=3)
    tbl, n = tbl.to(DEV), n.to(DEV)
    a = oa().oasis_sparse_decode_attn(q, kv, tbl, tbl, n, ctx, n_split=n_split)
    b = oa().oasis_lookahead_attn(q[:, None].contiguous(), kv, tbl, tbl, n, ctx, n_split=n_split)
    assert torch.equal(a, b[:, 0])


SHAPE_CASES = [
    # 256 (request, KV head) pairs: enough for eight-wave workgroups in one split
    (wl.Workload("pairs256_g4", B=32, H_q=32, H_kv=8, ctx=(17, 1500), budget=640, J=2, structure="none",
                 seed=81), n_q)
    for n_q in (1, 2)
] + [
    (wl.Workload("pairs256_g8", B=32, H_q=64, H_kv=8, ctx=(17, 1500), budget=640, J=1, structure="none",
                 seed=83), 1),
    # 128 pairs: eight-wave workgroups over two splits (72 table entries)
    (wl.Workload("pairs128_g8", B=16, H_q=64, H_kv=8, ctx=(1, 1500), budget=640, J=1, structure="none",
                 seed=85), 1),
]


@pytest.mark.parametrize("n_split", [0, 1, 2, 5])
@pytest.mark.parametrize("w,n_q", SHAPE_CASES, ids=[f"{w.name}-nq{n_q}" for w, n_q in SHAPE_CASES])
def test_attention_launch_shapes_match_oracle(w, n_q, n_split):
    """Both workgroup widths of the VALU attention kernel (four and eight
    waves, as oasis_attn_launch_shape picks them from the pairs, the columns
    and the split count) against the oracle, per query, over ragged contexts
    and tables with padding."""
    T = 72
    splits, waves = oa().oasis_attn_launch_shape(w.B, w.H_q, w.H_kv, n_q, T, n_split)
    expect_waves = {("pairs256_g4", 0): 8, ("pairs256_g4", 1): 8, ("pairs256_g4", 2): 4,
                    ("pairs256_g8", 0): 8, ("pairs128_g8", 0): 8, ("pairs128_g8", 5): 4}
    if (w.name, n_split) in expect_waves and n_q * (w.H_q // w.H_kv) <= 8:
        assert waves == expect_waves[(w.name, n_split)], (splits, waves)
    ctx = wl.context_lengths(w)
    kv = wl.kv_pool(w)
    q = joint_queries(w, n_q)
    tbl, n = wl.random_table(w, T, seed_index=11)
    sm = 1.0 / math.sqrt(w.D)
    out, lse = oa().oasis_lookahead_attn(q.to(DEV), kv.to(DEV), tbl.to(DEV), tbl.to(DEV), n.to(DEV), ctx.to(DEV),
                                         sm_scale=sm, n_split=n_split, want_lse=True)
    got, got_lse = bf16_to_f64(u16(out)), lse.cpu().numpy()
    kv_np, ctx_np = u16(kv), ctx.numpy()
    for qi in range(n_q):
        ref, ref_lse = oracle.attend(u16(q[:, qi]), kv_np, ctx_np, tbl.numpy(), n.numpy(), sm)
        assert_attn_close(got[:, qi], ref)
        np.testing.assert_allclose(got_lse[:, qi], ref_lse, rtol=1e-5, atol=1e-4)
