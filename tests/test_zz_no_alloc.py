"""oasis_sparse_decode_attn_static: the attention entry point that allocates
nothing (its split-K partials live in the library's fixed device scratch).

Through the C ABI, its output must equal oasis_sparse_decode_attn's with a
caller workspace, bit for bit (the same kernels with the same split count),
and the oracle's within the attention tolerance; checked on two calls in a
row, the second with a smaller input, so the second call runs over a scratch
that still holds the first call's partials.  Sizes beyond the scratch are
refused before anything is enqueued."""
import ctypes
import math

import numpy as np
import pytest
import torch

import oracle
from helpers import assert_attn_close, bf16_to_f64, u16

pytestmark = pytest.mark.gpu

DEV = "cuda"


def oa():
    import prefetch_block_scoring_amd as m
    return m


def case(B, H_q, H_kv, NB, T, seed):
    g = torch.Generator().manual_seed(seed)
    ctx = torch.randint(16 * (NB // 2), 16 * NB + 1, (B,), generator=g, dtype=torch.int32)
    kv = torch.randn((B, H_kv, NB, 2, 16, 128), generator=g).to(torch.bfloat16)
    q = torch.randn((B, H_q, 128), generator=g).to(torch.bfloat16)
    tbl = torch.full((B, H_kv, T), -1, dtype=torch.int32)
    n = torch.zeros((B, H_kv), dtype=torch.int32)
    for r in range(B):
        nb = -(-int(ctx[r]) // 16)
        for h in range(H_kv):
            ids = torch.randperm(nb, generator=g)[:T].sort().values.to(torch.int32)
            tbl[r, h, :len(ids)] = ids
            n[r, h] = len(ids)
    return ctx, kv, q, tbl, n


def run_both(ctx, kv, q, tbl, n, n_split):
    """(static output, workspace output, lse of each) through the raw C ABI."""
    m = oa()
    L = m.library()
    B, H_q, D = q.shape
    H_kv, P = kv.shape[1], kv.shape[2]
    T = tbl.shape[2]
    d = m.dims(B, H_q, H_kv, P)
    dq, dkv, dt, dn, dc = (x.to(DEV) for x in (q, kv, tbl, n, ctx))
    sm = 1.0 / math.sqrt(D)
    out_s = torch.full((B, H_q, D), 7, dtype=torch.bfloat16, device=DEV)
    lse_s = torch.full((B, H_q), 7.0, dtype=torch.float32, device=DEV)
    out_w = torch.empty_like(out_s)
    lse_w = torch.empty_like(lse_s)
    need = m.oasis_attn_workspace_bytes(B, H_q, H_kv, T, n_split)
    assert need > 0, "the case must split, or the scratch is not used"
    assert need <= m.oasis_sparse_decode_attn_static_bytes()
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    rc = L.oasis_sparse_decode_attn_static(ctypes.byref(d), p(dq), p(dkv), P, p(dt), p(dt), p(dn), T, p(dc), sm,
                                           p(out_s), p(lse_s), n_split, stream)
    assert rc == 0, m.oasis_last_error()
    rc = L.oasis_sparse_decode_attn(ctypes.byref(d), p(dq), p(dkv), P, p(dt), p(dt), p(dn), T, p(dc), sm,
                                    p(out_w), p(lse_w), p(ws), need, n_split, stream)
    assert rc == 0, m.oasis_last_error()
    torch.cuda.synchronize()
    return out_s.cpu(), out_w.cpu(), lse_s.cpu(), lse_w.cpu()


def test_static_scratch_matches_workspace_entry_point_twice():
    # first call: 4 requests, 32 / 8 heads, 4 splits; second: smaller, 3 splits
    for (B, H_q, H_kv, NB, T, n_split, seed) in ((4, 32, 8, 40, 24, 4, 301), (2, 8, 2, 20, 9, 3, 302)):
        ctx, kv, q, tbl, n = case(B, H_q, H_kv, NB, T, seed)
        out_s, out_w, lse_s, lse_w = run_both(ctx, kv, q, tbl, n, n_split)
        assert torch.equal(out_s, out_w), f"B={B}: static and workspace outputs differ"
        assert torch.equal(lse_s, lse_w)
        ref, ref_lse = oracle.attend(u16(q), u16(kv), ctx.numpy(), tbl.numpy(), n.numpy(), 1.0 / math.sqrt(128))
        assert_attn_close(bf16_to_f64(u16(out_s)), ref)
        np.testing.assert_allclose(lse_s.numpy(), ref_lse, rtol=1e-5, atol=1e-4)


def test_static_scratch_refuses_sizes_beyond_it():
    m = oa()
    B, H_q, H_kv = 512, 64, 4
    d = m.dims(B, H_q, H_kv, 64)
    assert m.oasis_attn_workspace_bytes(B, H_q, H_kv, 128, 16) > m.oasis_sparse_decode_attn_static_bytes()
    fake = ctypes.c_void_p(0x1000)  # never dereferenced: the call fails on the host
    rc = m.library().oasis_sparse_decode_attn_static(ctypes.byref(d), fake, fake, 64, fake, fake, fake, 128, fake,
                                                     0.1, fake, None, 16, None)
    assert rc == m.OASIS_ENOSPACE
    assert "fixed scratch" in m.oasis_last_error()
