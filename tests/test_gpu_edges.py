"""Edge cases of the decode chain (summaries -> scores -> top-K -> attention)
against the CPU oracle, through the C ABI: the largest context the library
accepts (16384 blocks per (request, KV head), 256K tokens) and degenerate
contexts (empty, one token, one short of a block, one block, one past it).

Bars as in test_gpu_parity: summaries bit-exact, scores within one fp32 ulp,
selections equal up to swaps of blocks tied within 1e-6 relative,
attention |out - ref| <= 2e-3 + 1e-2 |ref|.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from helpers import (assert_attn_close, assert_scores_close, assert_selection_matches,
                     bf16_to_f64, n_blocks, u16)

pytestmark = pytest.mark.gpu

DEV = "cuda"
MAX_BLOCKS = 16384   # the library's limit on blocks per (request, KV head)


def oa():
    import prefetch_block_scoring_amd as m
    return m


def chain_vs_oracle(ctx_cpu, kv_cpu, ql_cpu, q_cpu, H_kv, K_b, n_split=0):
    """Runs the chain on the GPU and the oracle on the CPU from the same
    inputs and checks every stage."""
    m = oa()
    ctx = ctx_cpu.to(DEV)
    summ = m.oasis_build_summaries(kv_cpu.to(DEV), ctx)
    sc = m.oasis_score_blocks(ql_cpu.to(DEV), summ, ctx)
    sel, n = m.oasis_select_topk(sc, ctx, K_b)
    kv = kv_cpu.to(DEV)
    sm = 1.0 / math.sqrt(kv_cpu.shape[-1])
    out, lse = m.oasis_sparse_decode_attn(q_cpu.to(DEV), kv, sel, sel, n, ctx, sm_scale=sm, n_split=n_split,
                                          want_lse=True)
    torch.cuda.synchronize()

    ctx_np = ctx_cpu.numpy()
    kv_np = u16(kv_cpu)
    rsumm = oracle.build_summaries(kv_np, ctx_np, 16)
    got_summ = u16(summ)
    for r in range(len(ctx_np)):
        nb = n_blocks(ctx_np[r])
        np.testing.assert_array_equal(got_summ[r, :, :nb], rsumm[r, :, :nb])
    rsc = oracle.score(u16(ql_cpu), rsumm, ctx_np, 16, H_kv)
    assert_scores_close(sc.cpu().numpy(), rsc, ctx_np)
    rsel, rn = oracle.select(rsc, ctx_np, 16, K_b)
    gsel, gn = sel.cpu().numpy(), n.cpu().numpy()
    assert_selection_matches(gsel, gn, rsel, rn, rsc)
    # attention over the GPU's own selection (equal to the oracle's up to
    # tied swaps), so that both sides attend over the same blocks
    ref, ref_lse = oracle.attend(u16(q_cpu), kv_np, ctx_np, gsel, gn, sm)
    assert_attn_close(bf16_to_f64(u16(out)), ref)
    np.testing.assert_allclose(lse.cpu().numpy(), ref_lse, rtol=1e-5, atol=1e-4)
    return gsel, gn, out


def test_maximum_context():
    """One request at the largest context the library accepts, 8 planted
    heavy-hitter blocks per KV head, which the top-K must all find."""
    w = wl.Workload("max_ctx", B=1, H_q=8, H_kv=2, ctx=MAX_BLOCKS * 16, budget=2048, J=1,
                    structure="planted", planted=8, seed=91)
    assert w.NB_max == MAX_BLOCKS
    ctx_cpu = wl.context_lengths(w)
    kv_cpu = wl.kv_pool(w)
    gsel, gn, _ = chain_vs_oracle(ctx_cpu, kv_cpu, wl.lookahead(w, 0), wl.attention_query(w, 1), w.H_kv, w.K_b)
    assert np.all(gn == w.K_b)
    for h, planted in enumerate(wl.planted_blocks(w)[0]):
        assert set(planted) <= set(gsel[0, h].tolist())


def test_max_blocks_limit_is_enforced():
    """One block past the limit is refused with an error, not launched."""
    m = oa()
    ctx = torch.tensor([(MAX_BLOCKS + 1) * 16], dtype=torch.int32, device=DEV)
    summ = torch.zeros((1, 1, MAX_BLOCKS + 1, 2, 128), dtype=torch.bfloat16, device=DEV)
    q = torch.zeros((1, 1, 4, 128), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(m.OasisError) as e:
        m.oasis_score_blocks(q, summ, ctx)
    assert e.value.code == m.OASIS_EUNSUPPORTED


@pytest.mark.parametrize("n_split", [0, 1, 2])
def test_degenerate_contexts(n_split):
    """Contexts of 0, 1, 15, 16, 17 and 40 tokens beside a long one: an empty
    request selects nothing and attends to nothing (output 0, lse -inf);
    partial blocks are summarised and attended over their valid tokens only
    (the padding holds 64.0, which any unmasked use would show)."""
    ctxs = [0, 1, 15, 16, 17, 40, 3000]
    B, H_q, H_kv, D, K_b = len(ctxs), 8, 2, 128, 8
    NB = n_blocks(max(ctxs))
    g = torch.Generator().manual_seed(93)
    kv = torch.randn((B, H_kv, NB, 2, 16, D), generator=g).to(torch.bfloat16)
    for r, c in enumerate(ctxs):
        for b in range(c // 16, NB):
            kv[r, :, b, :, max(c - 16 * b, 0):] = 64.0
    ql = torch.randn((B, 1, H_q, D), generator=g).to(torch.bfloat16)
    q = torch.randn((B, H_q, D), generator=g).to(torch.bfloat16)
    ctx_cpu = torch.tensor(ctxs, dtype=torch.int32)
    gsel, gn, out = chain_vs_oracle(ctx_cpu, kv, ql, q, H_kv, K_b, n_split=n_split)
    for r, c in enumerate(ctxs):
        assert np.all(gn[r] == min(n_blocks(c), K_b))
    o = out.cpu()
    assert torch.all(o[0] == 0)          # empty context


@pytest.mark.parametrize("pad", ["nan", "inf", "-inf"])
@pytest.mark.parametrize("n_q", [1, 2, 3])
def test_nonfinite_padding_is_never_used(pad, n_q):
    """Positions past a request's context may hold anything, NaN and Inf
    included (a pool that appends fill token by token starts from
    uninitialised memory).  Their weight is 0, and 0 * NaN would still poison
    the output, so both p . V paths must leave those rows out: with G = 4,
    n_q = 1 and 2 give 4 and 8 columns (VALU p . V), n_q = 3 gives 12
    (matrix-core p . V).  Every listed table ends with the partial last
    block."""
    m = oa()
    ctxs = [1, 15, 17, 40, 3000]
    B, H_q, H_kv, D, T = len(ctxs), 8, 2, 128, 6
    NB = n_blocks(max(ctxs))
    g = torch.Generator().manual_seed(94)
    kv = torch.randn((B, H_kv, NB, 2, 16, D), generator=g).to(torch.bfloat16)
    for r, c in enumerate(ctxs):
        for b in range(c // 16, NB):
            kv[r, :, b, :, max(c - 16 * b, 0):] = float(pad)
    q = torch.randn((B, n_q, H_q, D), generator=g).to(torch.bfloat16)
    tbl = torch.full((B, H_kv, T), -1, dtype=torch.int32)
    n = torch.zeros((B, H_kv), dtype=torch.int32)
    for r, c in enumerate(ctxs):
        nb = n_blocks(c)
        ids = list(range(max(0, nb - T), nb))
        tbl[r, :, :len(ids)] = torch.tensor(ids, dtype=torch.int32)
        n[r] = len(ids)
    ctx_cpu = torch.tensor(ctxs, dtype=torch.int32)
    sm = 1.0 / math.sqrt(D)
    for n_split in (1, 2):
        out = m.oasis_lookahead_attn(q.to(DEV), kv.to(DEV), tbl.to(DEV), tbl.to(DEV), n.to(DEV), ctx_cpu.to(DEV),
                                     sm_scale=sm, n_split=n_split)
        torch.cuda.synchronize()
        o = out.cpu()
        assert torch.isfinite(o.float()).all(), f"pad {pad}, n_q {n_q}, n_split {n_split}"
        for j in range(n_q):
            ref, _ = oracle.attend(u16(q[:, j].contiguous()), u16(kv), ctx_cpu.numpy(), tbl.numpy(), n.numpy(), sm)
            assert_attn_close(bf16_to_f64(u16(o[:, j].contiguous())), ref)
