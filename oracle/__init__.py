"""CPU oracle of the lookahead block-scoring decode path (test infrastructure).

Only the tests, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline
leg may import this package.  The product path (the HIP library and its Python
binding) never imports it.  It shares no code with the HIP library: the
arithmetic lives in ``oracle.c`` (plain C, fp64, OpenMP over independent rows);
this module only marshals NumPy arrays into it.

Each wrapper names the step of the OasisKV pages (arXiv 2608.08097, paperlayer
summary, section 4 "System Design") that the C function restates.  bf16 arrays
travel as uint16 bit patterns.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from . import build as _build

_lib = None

_i32 = np.int32
_u16 = np.uint16


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        L = ctypes.CDLL(_build.LIB)
        P = ctypes.c_void_p
        I = ctypes.c_int
        L.oracle_build_summaries.argtypes = [I, I, I, I, I, P, P, P]
        L.oracle_score.argtypes = [I, I, I, I, I, I, I, P, P, P, P]
        L.oracle_select.argtypes = [I, I, I, I, P, P, I, P, P]
        L.oracle_fetch_cap_blocks.argtypes = [ctypes.c_double, I]
        L.oracle_fetch_cap_blocks.restype = I
        L.oracle_stage.argtypes = [I, I, I, I, P, P, P, I, P, I, I, I, P, P, P, P, P, P]
        L.oracle_attend.argtypes = [I, I, I, I, I, I, P, P, P, P, P, I, ctypes.c_double, P, P]
        L.oracle_append.argtypes = [I, I, I, I, I, P, P, P, P, P]
        L.oracle_append.restype = None
        L.oracle_block_mass.argtypes = [I, I, I, I, I, I, P, P, P, ctypes.c_double, P]
        L.oracle_block_mass.restype = None
        L.oracle_num_threads.argtypes = []
        L.oracle_num_threads.restype = I
        for f in (L.oracle_build_summaries, L.oracle_score, L.oracle_select, L.oracle_stage,
                  L.oracle_attend):
            f.restype = None
        _lib = L
    return _lib


def _c(a, dtype):
    a = np.ascontiguousarray(a)
    if a.dtype != dtype:
        if dtype == _u16 and a.dtype == np.int16:
            a = a.view(_u16)
        else:
            raise TypeError(f"expected {np.dtype(dtype)}, got {a.dtype}")
    return a


def _p(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def num_threads() -> int:
    """OpenMP threads the oracle's loops run on."""
    return int(lib().oracle_num_threads())


def build_summaries(kv, ctx_len, bs: int):
    """Per-block coordinate-wise min / max of the valid keys (section 4).
    kv uint16 [B][H_kv][NB_max][2][bs][D] -> uint16 [B][H_kv][NB_max][2][D];
    blocks past the context stay zero."""
    kv = _c(kv, _u16)
    ctx = _c(ctx_len, _i32)
    B, H_kv, NB, two, bs_, D = kv.shape
    assert two == 2 and bs_ == bs
    out = np.zeros((B, H_kv, NB, 2, D), dtype=_u16)
    lib().oracle_build_summaries(B, H_kv, NB, bs, D, _p(kv), _p(ctx), _p(out))
    return out


def score(q_look, kminmax, ctx_len, bs: int, H_kv: int):
    """Lookahead block scores, fp32 [B][H_kv][NB_max] (section 4; bounding-box
    reading, summed over drafts and the group's query heads, fp64 sum rounded
    once)."""
    q = _c(q_look, _u16)
    s = _c(kminmax, _u16)
    ctx = _c(ctx_len, _i32)
    B, J, H_q, D = q.shape
    NB = s.shape[2]
    assert s.shape == (B, H_kv, NB, 2, D)
    out = np.empty((B, H_kv, NB), dtype=np.float32)
    lib().oracle_score(B, J, H_q, H_kv, D, NB, bs, _p(q), _p(s), _p(ctx), _p(out))
    return out


def select(scores, ctx_len, bs: int, K_b: int):
    """Top-K_b blocks per (r, h), ascending ids, -1 padded (sections 4-5)."""
    sc = _c(scores, np.float32)
    ctx = _c(ctx_len, _i32)
    B, H_kv, NB = sc.shape
    sel = np.empty((B, H_kv, K_b), dtype=_i32)
    n = np.empty((B, H_kv), dtype=_i32)
    lib().oracle_select(B, H_kv, NB, bs, _p(sc), _p(ctx), K_b, _p(sel), _p(n))
    return sel, n


def fetch_cap_blocks(cap: float, K_b: int) -> int:
    """Blocks per KV head per layer per step for a fetch-cap fraction."""
    return int(lib().oracle_fetch_cap_blocks(float(cap), int(K_b)))


class StageState:
    """Resident set and last-selected stamps per (r, h): stamp[b] = -1 when
    block b is not resident."""

    def __init__(self, B, H_kv, NB_max):
        self.stamp = np.full((B, H_kv, NB_max), -1, dtype=_i32)
        # per (r, h), after each step: predicted blocks that were neither
        # resident nor admitted (held back by the cap)
        self.deferred = np.zeros((B, H_kv), dtype=_i32)

    def resident(self, r, h):
        return np.nonzero(self.stamp[r, h] >= 0)[0]


def stage(state: StageState, sel, n_sel, scores, ctx_len, bs: int, K_b: int, C: int, step: int):
    """One staging step (section 4: keep resident predicted blocks, admit at
    most C non-resident ones, pair them with least-recently-selected victims).
    Updates ``state`` in place (``state.deferred`` receives the predicted
    blocks held back by the cap, |P \\ R| - |A| per pair); returns (admitted,
    n_admitted, evicted, n_evicted) with admitted/evicted int32
    [B][H_kv][max(C,1)] in order."""
    sel = _c(sel, _i32)
    n_sel = _c(n_sel, _i32)
    sc = _c(scores, np.float32)
    ctx = _c(ctx_len, _i32)
    B, H_kv, NB = state.stamp.shape
    Cs = max(C, 1)
    adm = np.full((B, H_kv, Cs), -1, dtype=_i32)
    ev = np.full((B, H_kv, Cs), -1, dtype=_i32)
    na = np.zeros((B, H_kv), dtype=_i32)
    ne = np.zeros((B, H_kv), dtype=_i32)
    assert sc.shape == (B, H_kv, NB)
    lib().oracle_stage(B, H_kv, NB, bs, _p(ctx), _p(sel), _p(n_sel), sel.shape[2], _p(sc),
                       K_b, C, step, _p(state.stamp), _p(adm), _p(na), _p(ev), _p(ne), _p(state.deferred))
    return adm, na, ev, ne


def attend(q, kv, ctx_len, blocks, n_blocks, sm_scale: float):
    """Softmax attention of each query head over the listed blocks' valid
    tokens (sections 4 and 7), fp64.  Returns (out [B][H_q][D] float64,
    lse [B][H_q] float64)."""
    q = _c(q, _u16)
    kv = _c(kv, _u16)
    ctx = _c(ctx_len, _i32)
    blk = _c(blocks, _i32)
    nb = _c(n_blocks, _i32)
    B, H_q, D = q.shape
    _, H_kv, NB, two, bs, D2 = kv.shape
    assert D2 == D and two == 2 and blk.shape[:2] == (B, H_kv)
    T = blk.shape[2]
    out = np.empty((B, H_q, D), dtype=np.float64)
    lse = np.empty((B, H_q), dtype=np.float64)
    lib().oracle_attend(B, H_q, H_kv, D, NB, bs, _p(q), _p(kv), _p(ctx), _p(blk), _p(nb), T,
                        float(sm_scale), _p(out), _p(lse))
    return out, lse


def append(k_new, v_new, ctx_len, kv, kminmax, bs: int):
    """One decoded token per request (section 4: full KV off-GPU, block
    summaries in HBM): K / V written at position ctx_len[r] of every KV head,
    the block's min / max summary updated, ctx_len incremented.  Returns the
    updated copies (ctx_len, kv, kminmax); the inputs are not modified.
    k_new, v_new uint16 [B][H_kv][D]."""
    k = _c(k_new, _u16)
    v = _c(v_new, _u16)
    ctx = _c(ctx_len, _i32).copy()
    kv = _c(kv, _u16).copy()
    s = _c(kminmax, _u16).copy()
    B, H_kv, NB, two, bs_, D = kv.shape
    assert two == 2 and bs_ == bs and k.shape == (B, H_kv, D) and v.shape == (B, H_kv, D)
    assert s.shape == (B, H_kv, NB, 2, D) and ctx.shape == (B,)
    lib().oracle_append(B, H_kv, NB, bs, D, _p(k), _p(v), _p(ctx), _p(kv), _p(s))
    return ctx, kv, s


def block_mass(q, kv, ctx_len, sm_scale: float):
    """Exact attention mass per block of the query q over the whole context,
    summed over each KV head's query heads (the true next-token set of the
    lookahead-agreement analogue, section 4): fp64 [B][H_kv][NB_max].
    q uint16 [B][H_q][D], kv uint16 [B][H_kv][NB_max][2][bs][D]."""
    q = _c(q, _u16)
    kv = _c(kv, _u16)
    ctx = _c(ctx_len, _i32)
    B, H_kv, NB, two, bs, D = kv.shape
    H_q = q.shape[1]
    assert two == 2 and q.shape == (B, H_q, D) and ctx.shape == (B,)
    out = np.empty((B, H_kv, NB), dtype=np.float64)
    lib().oracle_block_mass(B, H_q, H_kv, D, NB, bs, _p(q), _p(kv), _p(ctx), float(sm_scale), _p(out))
    return out


def agreement(pred_sel, pred_n, true_sel, true_n):
    """Per (r, h): |predicted set & true set| / |true set| (1 where the true
    set is empty); [B][H_kv] fp64."""
    B, H = true_n.shape
    out = np.ones((B, H), dtype=np.float64)
    for r in range(B):
        for h in range(H):
            k = int(true_n[r, h])
            if k <= 0:
                continue
            P = set(pred_sel[r, h, :int(pred_n[r, h])].tolist())
            T = set(true_sel[r, h, :k].tolist())
            out[r, h] = len(P & T) / k
    return out
