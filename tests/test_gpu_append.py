"""Appending one decoded token per request (paperlayer summary, section 4:
full KV off-GPU, block summaries and the working set in HBM): the GPU's
oasis_append_kv against the oracle's append, token by token, bit-exact on
contexts, pool bytes and summaries; the resident slot of the token's block
is updated, so the next attention over the working set matches the oracle's
attention over the resident blocks of the appended pool."""
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


def tokens(w, n, seed):
    g = torch.Generator().manual_seed(seed)
    return [(torch.randn((w.B, w.H_kv, w.D), generator=g).to(torch.bfloat16),
             torch.randn((w.B, w.H_kv, w.D), generator=g).to(torch.bfloat16)) for _ in range(n)]


@pytest.mark.parametrize("host_pool", [False, True])
@pytest.mark.parametrize("w", [
    wl.WORKLOADS["parity_8q2kv_4k"].shrink(ctx=4096 - 21),
    wl.Workload("ragged_append", B=5, H_q=16, H_kv=4, ctx=(1, 90), budget=64, J=1, structure="none", seed=81),
], ids=["parity_8q2kv_4k", "ragged"])
def test_append_matches_oracle_token_by_token(w, host_pool):
    m = oa()
    ctx_cpu = wl.context_lengths(w)
    kv_cpu = wl.kv_pool(w)
    if host_pool:
        pool = m.oasis_host_empty(tuple(kv_cpu.shape))
        pool.copy_(kv_cpu)
    else:
        pool = kv_cpu.to(DEV)
    ctx = ctx_cpu.to(DEV)
    summ = m.oasis_build_summaries(pool, ctx)
    o_ctx, o_kv = ctx_cpu.numpy(), u16(kv_cpu)
    o_summ = oracle.build_summaries(o_kv, o_ctx, w.bs)
    cap = w.NB_max * w.bs
    n_tok = min(cap - int(o_ctx.min()) + 2, 40)      # past the capacity for the longest requests
    for i, (k, v) in enumerate(tokens(w, n_tok, 5)):
        m.oasis_append_kv(k.to(DEV), v.to(DEV), ctx, summ, pool)
        o_ctx, o_kv, o_summ = oracle.append(u16(k), u16(v), o_ctx, o_kv, o_summ, w.bs)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(ctx.cpu().numpy(), o_ctx, err_msg=f"token {i}")
    np.testing.assert_array_equal(u16(pool), o_kv)
    got_s = u16(summ)
    for r in range(w.B):
        n_b = -(-int(o_ctx[r]) // w.bs)
        np.testing.assert_array_equal(got_s[r, :, :n_b], o_summ[r, :, :n_b], err_msg=f"request {r}")


def test_append_updates_the_resident_slot():
    """A working set holds the context's last block for some (request, KV
    head) pairs and not for others; after an append the slot of a resident
    block equals the appended pool block, other slots are untouched, and the
    attention over the working set equals the oracle's over the resident
    blocks of the appended pool (the new token is attended only where its
    block is resident)."""
    m = oa()
    w = wl.Workload("append_ws", B=4, H_q=16, H_kv=4, ctx=(40, 300), budget=64, J=1, structure="none", seed=83)
    # one request starts a fresh block with this token
    ctx_cpu = wl.context_lengths(w).clone()
    ctx_cpu[1] = 64
    kv_cpu = wl.kv_pool(w)
    host = m.oasis_host_empty(tuple(kv_cpu.shape))
    host.copy_(kv_cpu)
    S = 8
    g = torch.Generator().manual_seed(3)
    slot_block = torch.full((w.B, w.H_kv, S), -1, dtype=torch.int32)
    ws = torch.zeros((w.B, w.H_kv, S, 2, w.bs, w.D), dtype=torch.bfloat16)
    for r in range(w.B):
        c = int(ctx_cpu[r])
        last = c // w.bs                              # the block the next token goes to
        n_b = -(-c // w.bs)
        for h in range(w.H_kv):
            others = [b for b in torch.randperm(n_b, generator=g).tolist() if b != last][:5]
            blocks = others + ([last] if (r + h) % 2 == 0 and last < w.NB_max else [])
            slots = torch.randperm(S, generator=g)[:len(blocks)].tolist()
            for b, s in zip(blocks, slots):
                slot_block[r, h, s] = b
                if b < n_b:
                    ws[r, h, s] = kv_cpu[r, h, b]
    ws_d, sb_d, ctx = ws.to(DEV), slot_block.to(DEV), ctx_cpu.to(DEV)
    summ = m.oasis_build_summaries(host, ctx)
    k, v = tokens(w, 1, 9)[0]
    m.oasis_append_kv(k.to(DEV), v.to(DEV), ctx, summ, host, ws_pool=ws_d, slot_block=sb_d)
    o_ctx, o_kv, _ = oracle.append(u16(k), u16(v), ctx_cpu.numpy(), u16(kv_cpu),
                                   oracle.build_summaries(u16(kv_cpu), ctx_cpu.numpy(), w.bs), w.bs)
    torch.cuda.synchronize()
    got_ws = u16(ws_d)
    before = u16(ws)
    for r in range(w.B):
        for h in range(w.H_kv):
            for s in range(S):
                b = int(slot_block[r, h, s])
                if b < 0:
                    continue
                if b == int(ctx_cpu[r]) // w.bs:
                    # the valid rows of the appended block (attention masks the rest)
                    valid = min(w.bs, int(o_ctx[r]) - b * w.bs)
                    np.testing.assert_array_equal(got_ws[r, h, s, :, :valid], o_kv[r, h, b, :, :valid],
                                                  err_msg=f"{r} {h} {s}")
                else:
                    np.testing.assert_array_equal(got_ws[r, h, s], before[r, h, s])
    # attention over the working set after the append
    tbl_slot = torch.full((w.B, w.H_kv, S), -1, dtype=torch.int32)
    tbl_block = torch.full((w.B, w.H_kv, S), -1, dtype=torch.int32)
    tbl_n = torch.zeros((w.B, w.H_kv), dtype=torch.int32)
    for r in range(w.B):
        for h in range(w.H_kv):
            held = [(s, int(slot_block[r, h, s])) for s in range(S) if slot_block[r, h, s] >= 0]
            for i, (s, b) in enumerate(held):
                tbl_slot[r, h, i], tbl_block[r, h, i] = s, b
            tbl_n[r, h] = len(held)
    q = wl.attention_query(w, 1)
    out = m.oasis_sparse_decode_attn(q.to(DEV), ws_d, tbl_slot.to(DEV), tbl_block.to(DEV), tbl_n.to(DEV), ctx)
    ref, _ = oracle.attend(u16(q), o_kv, o_ctx, tbl_block.numpy(), tbl_n.numpy(), 1 / math.sqrt(w.D))
    assert_attn_close(bf16_to_f64(u16(out)), ref)
