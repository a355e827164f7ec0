"""Shared helpers of the test suite (conversions and tolerance checks)."""
import numpy as np
import torch


def u16(t: torch.Tensor) -> np.ndarray:
    """bf16 tensor (any device) -> uint16 NumPy array of its bit patterns."""
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def bf16_to_f64(a: np.ndarray) -> np.ndarray:
    return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def n_blocks(ctx: int, bs: int = 16) -> int:
    return -(-int(ctx) // bs) if ctx > 0 else 0


def assert_scores_close(got: np.ndarray, ref: np.ndarray, ctx, bs=16):
    """GPU and oracle both round an fp64 sum of the same exact products to
    fp32; the sums differ only in rounding order, so they agree to one fp32
    ulp.  Entries past a request's blocks are -inf on both."""
    for r in range(ref.shape[0]):
        nb = n_blocks(ctx[r], bs)
        g = got[r, :, :nb].astype(np.float64)
        e = ref[r, :, :nb].astype(np.float64)
        ulp = np.spacing(np.abs(ref[r, :, :nb])).astype(np.float64)
        bad = np.abs(g - e) > ulp
        assert not bad.any(), f"request {r}: {bad.sum()} scores differ by more than 1 ulp"
        assert np.all(np.isneginf(got[r, :, nb:]))


def assert_selection_matches(sel_g, n_g, sel_o, n_o, scores_o, rel=1e-6):
    """Selections agree except for swaps between blocks whose oracle scores
    tie within `rel` relative."""
    assert np.array_equal(n_g, n_o)
    for idx in np.ndindex(*n_o.shape):
        k = int(n_o[idx])
        G = set(sel_g[idx][:k].tolist())
        O = set(sel_o[idx][:k].tolist())
        assert np.all(sel_g[idx][k:] == -1)
        assert sel_g[idx][:k].tolist() == sorted(G)
        if G == O:
            continue
        s = scores_o[idx]
        for a in G - O:
            for b in O - G:
                sa, sb = float(s[a]), float(s[b])
                assert abs(sa - sb) <= rel * max(abs(sa), abs(sb)), (idx, a, b, sa, sb)


def assert_attn_close(out_gpu: np.ndarray, ref: np.ndarray, atol=2e-3, rtol=1e-2):
    """bf16 output vs fp64 reference: |o - ref| <= atol + rtol * |ref|."""
    err = np.abs(out_gpu - ref)
    lim = atol + rtol * np.abs(ref)
    bad = err > lim
    assert not bad.any(), f"{bad.sum()} of {bad.size} outputs out of tolerance; worst excess {np.max(err - lim):.3g}"


def gpu_stage_state(slot_block, slot_stamp, NB):
    """Per-block stamps (-1 = not resident) from the GPU's slot arrays, in the
    oracle's layout; checks that no block is held by two slots."""
    sb = slot_block.cpu().numpy() if isinstance(slot_block, torch.Tensor) else slot_block
    st = slot_stamp.cpu().numpy() if isinstance(slot_stamp, torch.Tensor) else slot_stamp
    B, H, S = sb.shape
    stamp = np.full((B, H, NB), -1, dtype=np.int32)
    for r in range(B):
        for h in range(H):
            held = sb[r, h][sb[r, h] >= 0]
            assert len(set(held.tolist())) == len(held), "a block is held by two slots"
            for s in range(S):
                if sb[r, h, s] >= 0:
                    stamp[r, h, sb[r, h, s]] = st[r, h, s]
    return stamp


def selection_equal_pairs(sel_g, n_g, sel_o, n_o):
    """Boolean [B][H_kv]: the two selections are identical for that pair."""
    out = np.zeros(n_o.shape, dtype=bool)
    for idx in np.ndindex(*n_o.shape):
        k = int(n_o[idx])
        out[idx] = int(n_g[idx]) == k and np.array_equal(sel_g[idx][:k], sel_o[idx][:k])
    return out
