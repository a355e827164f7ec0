"""Python binding of liboasis.so: argument marshalling only.

Each function carries the name of the C entry point it calls (include/oasis.h
documents the semantics).  Tensors supply device memory, pinned host memory
and streams; every step of the decode path runs in the library's HIP kernels.
If the library is missing the import of this module raises: there is no
fallback path.
"""
from __future__ import annotations

import ctypes
import math
import os
import weakref
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboasis.so")

OASIS_OK = 0
OASIS_EINVAL = -1
OASIS_EUNSUPPORTED = -2
OASIS_EHIP = -3
OASIS_ENOSPACE = -4
OASIS_COPY_KERNEL = 0
OASIS_COPY_DMA = 1
OASIS_COPY_MIXED = 2  # layer pipeline only: even layers DMA, odd layers gather kernel

_I32 = ctypes.c_int32
_P = ctypes.c_void_p


class OasisError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"oasis error {code}: {msg}")
        self.code = code


class oasis_dims(ctypes.Structure):
    _fields_ = [("B", _I32), ("H_q", _I32), ("H_kv", _I32), ("D", _I32), ("bs", _I32),
                ("NB_max", _I32)]


class oasis_stage_args(ctypes.Structure):
    _fields_ = [
        ("sel", _P), ("n_sel", _P), ("K_sel", _I32), ("scores", _P), ("K_b", _I32), ("C", _I32),
        ("S", _I32), ("step", _I32), ("slot_block", _P), ("slot_stamp", _P), ("ctx_len", _P),
        ("host_pool", _P), ("ws_pool", _P), ("tbl_slot", _P), ("tbl_block", _P), ("tbl_n", _P),
        ("plan", _P), ("plan_bytes", ctypes.c_size_t), ("host_plan", _P),
        ("host_plan_bytes", ctypes.c_size_t), ("stage_host", _P), ("stage_host_bytes", ctypes.c_size_t),
        ("stage_dev", _P), ("stage_dev_bytes", ctypes.c_size_t), ("host_threads", _I32),
        ("copy_mode", _I32), ("stream", _P), ("copy_stream", _P), ("wait_event", _P),
        ("done_event", _P), ("plan_event", _P), ("stats_accum", _P)]


class oasis_stage_stats(ctypes.Structure):
    _fields_ = [("admits", ctypes.c_int64), ("evictions", ctypes.c_int64), ("deferred", ctypes.c_int64),
                ("capped_pairs", ctypes.c_int64), ("bytes", ctypes.c_int64)]

    def as_dict(self) -> dict:
        return {k: int(getattr(self, k)) for k, _ in self._fields_}


class oasis_layer_buffers(ctypes.Structure):
    _fields_ = [
        ("scores", _P), ("sel", _P * 2), ("n_sel", _P * 2), ("attn_ws", _P), ("attn_ws_bytes", ctypes.c_size_t),
        ("ws_pool", _P), ("slot_block", _P), ("slot_stamp", _P), ("tbl_slot", _P * 3), ("tbl_block", _P * 3),
        ("tbl_n", _P * 3), ("plan", _P * 2), ("plan_bytes", ctypes.c_size_t), ("host_plan", _P),
        ("stage_host", _P * 2), ("stage_dev", _P), ("stage_bytes", ctypes.c_size_t)]


class oasis_pipeline_desc(ctypes.Structure):
    _fields_ = [
        ("n_layers", _I32), ("K_b", _I32), ("C", _I32), ("J", _I32), ("n_q", _I32), ("staged", _I32),
        ("copy_mode", _I32),
        ("host_threads", _I32), ("n_split", _I32), ("sm_scale", ctypes.c_float), ("pool", _P),
        ("kminmax", _P), ("ctx_len", _P), ("main_stream", _P), ("layers", ctypes.POINTER(oasis_layer_buffers)),
        ("compute_streams", _I32), ("stage_stats", _P), ("issue_threads", _I32)]


# name -> (restype, argtypes)
_SIGNATURES = {
    "oasis_version": (ctypes.c_char_p, []),
    "oasis_last_error": (ctypes.c_char_p, []),
    "oasis_fetch_cap_blocks": (_I32, [ctypes.c_double, _I32]),
    "oasis_host_alloc": (ctypes.c_int, [ctypes.c_size_t, ctypes.POINTER(ctypes.c_void_p)]),
    "oasis_host_free": (ctypes.c_int, [_P]),
    "oasis_build_summaries": (ctypes.c_int, [ctypes.POINTER(oasis_dims), _P, _P, _P, _P]),
    "oasis_score_blocks": (ctypes.c_int, [ctypes.POINTER(oasis_dims), _P, _I32, _P, _P, _P, _P]),
    "oasis_select_topk": (ctypes.c_int, [ctypes.POINTER(oasis_dims), _P, _P, _I32, _P, _P, _P]),
    "oasis_stage_plan_bytes": (ctypes.c_size_t, [ctypes.POINTER(oasis_dims), _I32]),
    "oasis_stage_buffer_bytes": (ctypes.c_size_t, [ctypes.POINTER(oasis_dims), _I32]),
    "oasis_stage_blocks": (ctypes.c_int, [ctypes.POINTER(oasis_dims), ctypes.POINTER(oasis_stage_args),
                                          ctypes.POINTER(oasis_stage_stats)]),
    "oasis_stage_read_stats": (ctypes.c_int, [ctypes.POINTER(oasis_dims), _I32, _P,
                                              ctypes.POINTER(oasis_stage_stats), _P]),
    "oasis_stage_plan": (ctypes.c_int, [ctypes.POINTER(oasis_dims), ctypes.POINTER(oasis_stage_args)]),
    "oasis_stage_copy": (ctypes.c_int, [ctypes.POINTER(oasis_dims), ctypes.POINTER(oasis_stage_args)]),
    "oasis_attn_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(oasis_dims), _I32, _I32]),
    "oasis_attn_num_splits": (_I32, [ctypes.POINTER(oasis_dims), _I32, _I32]),
    "oasis_attn_launch_shape": (ctypes.c_int, [ctypes.POINTER(oasis_dims), _I32, _I32, _I32, ctypes.POINTER(_I32),
                                               ctypes.POINTER(_I32)]),
    "oasis_sparse_decode_attn": (ctypes.c_int, [
        ctypes.POINTER(oasis_dims), _P, _P, _I32, _P, _P, _P, _I32, _P, ctypes.c_float, _P, _P, _P,
        ctypes.c_size_t, _I32, _P]),
    "oasis_sparse_decode_attn_static_bytes": (ctypes.c_size_t, []),
    "oasis_sparse_decode_attn_static": (ctypes.c_int, [
        ctypes.POINTER(oasis_dims), _P, _P, _I32, _P, _P, _P, _I32, _P, ctypes.c_float, _P, _P, _I32, _P]),
    "oasis_block_mass_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(oasis_dims)]),
    "oasis_block_attention_mass": (ctypes.c_int, [ctypes.POINTER(oasis_dims), _P, _P, _P, ctypes.c_float, _P, _P,
                                                  ctypes.c_size_t, _P]),
    "oasis_topk_overlap": (ctypes.c_int, [ctypes.POINTER(oasis_dims), _P, _P, _P, _P, _I32, _P, _P]),
    "oasis_append_kv": (ctypes.c_int, [ctypes.POINTER(oasis_dims), _P, _P, _P, _P, _P, _P, _P, _I32, _P]),
    "oasis_lookahead_attn_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(oasis_dims), _I32, _I32, _I32]),
    "oasis_lookahead_attn": (ctypes.c_int, [
        ctypes.POINTER(oasis_dims), _I32, _P, _P, _I32, _P, _P, _P, _I32, _P, ctypes.c_float, _P, _P, _P,
        ctypes.c_size_t, _I32, _P]),
    "oasis_pipeline_create": (ctypes.c_int, [ctypes.POINTER(oasis_dims), ctypes.POINTER(oasis_pipeline_desc),
                                             ctypes.POINTER(ctypes.c_void_p)]),
    "oasis_pipeline_layer_step": (ctypes.c_int, [_P, _I32, _I32, _P, _P, _P, _P]),
    "oasis_pipeline_drain": (ctypes.c_int, [_P]),
    "oasis_pipeline_stream": (ctypes.c_int, [_P, _I32, ctypes.POINTER(ctypes.c_void_p)]),
    "oasis_pipeline_issue_threads": (ctypes.c_int, [_P, ctypes.POINTER(_I32)]),
    "oasis_pipeline_timing": (ctypes.c_int, [_P, _I32, ctypes.c_uint32, _I32]),
    "oasis_pipeline_timing_read": (ctypes.c_int, [_P, _I32, ctypes.POINTER(ctypes.c_double),
                                                  ctypes.POINTER(_I32)]),
    "oasis_pipeline_timing_values": (ctypes.c_int, [_P, _I32, ctypes.POINTER(ctypes.c_float), _I32,
                                                    ctypes.POINTER(_I32)]),
    "oasis_pipeline_copy_host_seconds": (ctypes.c_int, [_P, ctypes.POINTER(ctypes.c_double),
                                                        ctypes.POINTER(_I32)]),
    "oasis_pipeline_destroy": (ctypes.c_int, [_P]),
}


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python -m prefetch_block_scoring_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in _SIGNATURES.items():
        f = getattr(L, name)
        f.restype = res
        f.argtypes = args
    return L


_lib = _load()


def library() -> ctypes.CDLL:
    return _lib


def _check(rc: int):
    if rc != OASIS_OK:
        raise OasisError(rc, _lib.oasis_last_error().decode())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(s) -> Optional[int]:
    if s is None:
        s = torch.cuda.current_stream()
    if isinstance(s, int):
        return s
    return s.cuda_stream


def _event(ev) -> Optional[int]:
    if ev is None:
        return None
    if isinstance(ev, int):
        return ev
    if not ev.cuda_event:
        ev.record()  # torch creates its event lazily on first record
    return ev.cuda_event


def _on_device(t: torch.Tensor) -> bool:
    return t.is_cuda


def _need(t: torch.Tensor, name: str, dtype, ndim: int, device: Optional[str] = "cuda", shape=None):
    """Type, rank, contiguity and device of one argument; with `shape`, its
    exact shape.  The C entry points see only pointers, so every size they
    index with is checked here before anything is enqueued."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if t.dim() != ndim:
        raise ValueError(f"{name}: expected {ndim} dims, got shape {tuple(t.shape)}")
    if shape is not None and tuple(t.shape) != tuple(int(x) for x in shape):
        raise ValueError(f"{name}: expected shape {tuple(int(x) for x in shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if device == "cuda" and not _on_device(t):
        raise ValueError(f"{name} must be a device tensor")


def _need_bytes(t: torch.Tensor, name: str, device: Optional[str] = "cuda"):
    """A workspace of any dtype: contiguous, on the device (or host)."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if device == "cuda" and not _on_device(t):
        raise ValueError(f"{name} must be a device tensor")
    if device == "host" and _on_device(t):
        raise ValueError(f"{name} must be a host tensor")


def _group(H_q: int, H_kv: int):
    if H_kv <= 0 or H_q % H_kv != 0:
        raise ValueError(f"H_q = {H_q} is not a multiple of H_kv = {H_kv}")


def dims(B, H_q, H_kv, NB_max, D=128, bs=16) -> oasis_dims:
    return oasis_dims(int(B), int(H_q), int(H_kv), int(D), int(bs), int(NB_max))


# --------------------------------------------------------------------------


def oasis_version() -> str:
    return _lib.oasis_version().decode()


def oasis_last_error() -> str:
    return _lib.oasis_last_error().decode()


def oasis_host_empty(shape, dtype=torch.bfloat16) -> torch.Tensor:
    """A CPU tensor over pinned host memory from oasis_host_alloc (freed
    with the tensor's storage).  Unlike torch's pin_memory buffers this memory
    is cacheable for the CPU, which the DMA engine's packing threads need."""
    nbytes = max(1, math.prod(shape) * torch.empty((), dtype=dtype).element_size())
    p = ctypes.c_void_p()
    _check(_lib.oasis_host_alloc(nbytes, ctypes.byref(p)))
    ptr = p.value
    buf = (ctypes.c_uint8 * nbytes).from_address(ptr)
    flat = torch.frombuffer(buf, dtype=torch.uint8)
    # free the memory when the last view of it dies
    weakref.finalize(buf, _lib.oasis_host_free, ctypes.c_void_p(ptr))
    flat._oasis_host_buffer = buf  # keep the ctypes owner alive with the tensor
    t = flat[: math.prod(shape) * torch.empty((), dtype=dtype).element_size()].view(dtype).view(shape)
    t._oasis_host_buffer = buf
    return t


def oasis_fetch_cap_blocks(cap: float, K_b: int) -> int:
    return int(_lib.oasis_fetch_cap_blocks(float(cap), int(K_b)))


def oasis_build_summaries(kv: torch.Tensor, ctx_len: torch.Tensor, kminmax=None, stream=None):
    """kv bf16 [B][H_kv][NB_max][2][bs][D] (device or pinned host) ->
    kminmax bf16 [B][H_kv][NB_max][2][D]."""
    _need(kv, "kv", torch.bfloat16, 6, device=None)
    _need(ctx_len, "ctx_len", torch.int32, 1)
    B, H_kv, NB, two, bs, D = kv.shape
    if two != 2:
        raise ValueError(f"kv: dimension 3 must be 2 (K, V), got {two}")
    _need(ctx_len, "ctx_len", torch.int32, 1, shape=(B,))
    if kminmax is None:
        kminmax = torch.empty((B, H_kv, NB, 2, D), dtype=torch.bfloat16, device=ctx_len.device)
    _need(kminmax, "kminmax", torch.bfloat16, 5, shape=(B, H_kv, NB, 2, D))
    d = dims(B, H_kv, H_kv, NB, D, bs)
    _check(_lib.oasis_build_summaries(ctypes.byref(d), _ptr(kv), _ptr(ctx_len), _ptr(kminmax),
                                      _stream(stream)))
    return kminmax


def oasis_score_blocks(q_look: torch.Tensor, kminmax: torch.Tensor, ctx_len: torch.Tensor,
                       scores=None, bs: int = 16, stream=None):
    """q_look bf16 [B][J][H_q][D], kminmax bf16 [B][H_kv][NB_max][2][D] ->
    scores fp32 [B][H_kv][NB_max]."""
    _need(q_look, "q_look", torch.bfloat16, 4)
    _need(kminmax, "kminmax", torch.bfloat16, 5)
    _need(ctx_len, "ctx_len", torch.int32, 1)
    B, J, H_q, D = q_look.shape
    H_kv, NB = kminmax.shape[1], kminmax.shape[2]
    _group(H_q, H_kv)
    _need(kminmax, "kminmax", torch.bfloat16, 5, shape=(B, H_kv, NB, 2, D))
    _need(ctx_len, "ctx_len", torch.int32, 1, shape=(B,))
    if scores is None:
        scores = torch.empty((B, H_kv, NB), dtype=torch.float32, device=q_look.device)
    _need(scores, "scores", torch.float32, 3, shape=(B, H_kv, NB))
    d = dims(B, H_q, H_kv, NB, D, bs)
    _check(_lib.oasis_score_blocks(ctypes.byref(d), _ptr(q_look), J, _ptr(kminmax), _ptr(ctx_len),
                                   _ptr(scores), _stream(stream)))
    return scores


def oasis_select_topk(scores: torch.Tensor, ctx_len: torch.Tensor, K_b: int, sel=None, n_sel=None,
                      bs: int = 16, stream=None):
    """scores fp32 [B][H_kv][NB_max] -> (sel int32 [B][H_kv][K_b], n_sel int32 [B][H_kv])."""
    _need(scores, "scores", torch.float32, 3)
    _need(ctx_len, "ctx_len", torch.int32, 1)
    B, H_kv, NB = scores.shape
    _need(ctx_len, "ctx_len", torch.int32, 1, shape=(B,))
    if sel is None:
        sel = torch.empty((B, H_kv, K_b), dtype=torch.int32, device=scores.device)
    if n_sel is None:
        n_sel = torch.empty((B, H_kv), dtype=torch.int32, device=scores.device)
    _need(sel, "sel", torch.int32, 3, shape=(B, H_kv, K_b))
    _need(n_sel, "n_sel", torch.int32, 2, shape=(B, H_kv))
    d = dims(B, H_kv, H_kv, NB, 128, bs)
    _check(_lib.oasis_select_topk(ctypes.byref(d), _ptr(scores), _ptr(ctx_len), int(K_b), _ptr(sel),
                                  _ptr(n_sel), _stream(stream)))
    return sel, n_sel


def oasis_append_kv(k_new: torch.Tensor, v_new: torch.Tensor, ctx_len: torch.Tensor, kminmax: torch.Tensor,
                    pool: torch.Tensor, ws_pool: Optional[torch.Tensor] = None,
                    slot_block: Optional[torch.Tensor] = None, stream=None):
    """One decoded token per request: k_new / v_new bf16 [B][H_kv][D] go to
    position ctx_len[r] of pool (bf16 [B][H_kv][NB_max][2][bs][D], device or
    pinned host), the block's summary in kminmax is updated, the resident
    slot (ws_pool [B][H_kv][S][2][bs][D] with slot_block [B][H_kv][S]) too;
    ctx_len is advanced in place."""
    _need(k_new, "k_new", torch.bfloat16, 3)
    _need(v_new, "v_new", torch.bfloat16, 3)
    _need(ctx_len, "ctx_len", torch.int32, 1)
    _need(kminmax, "kminmax", torch.bfloat16, 5)
    _need(pool, "pool", torch.bfloat16, 6, device=None)
    B, H_kv, NB, _, bs, D = pool.shape
    if tuple(k_new.shape) != (B, H_kv, D) or tuple(v_new.shape) != (B, H_kv, D):
        raise ValueError("k_new / v_new must be [B][H_kv][D]")
    if tuple(kminmax.shape) != (B, H_kv, NB, 2, D) or tuple(ctx_len.shape) != (B,):
        raise ValueError("kminmax / ctx_len shape mismatch")
    S = 0
    if ws_pool is not None:
        if slot_block is None:
            raise ValueError("a working set needs its slot_block table")
        S = ws_pool.shape[2] if ws_pool.dim() == 6 else 0
        _need(ws_pool, "ws_pool", torch.bfloat16, 6, shape=(B, H_kv, S, 2, bs, D))
        _need(slot_block, "slot_block", torch.int32, 3, shape=(B, H_kv, S))
    d = dims(B, H_kv, H_kv, NB, D, bs)
    _check(_lib.oasis_append_kv(ctypes.byref(d), _ptr(k_new), _ptr(v_new), _ptr(ctx_len), _ptr(kminmax),
                                _ptr(pool), _ptr(ws_pool), _ptr(slot_block), int(S), _stream(stream)))


def oasis_block_mass_workspace_bytes(B: int, H_q: int, H_kv: int, NB_max: int) -> int:
    d = dims(B, H_q, H_kv, NB_max)
    return int(_lib.oasis_block_mass_workspace_bytes(ctypes.byref(d)))


def oasis_block_attention_mass(q: torch.Tensor, kv_pool: torch.Tensor, ctx_len: torch.Tensor,
                               sm_scale: Optional[float] = None, mass=None, ws=None, stream=None):
    """q bf16 [B][H_q][D], kv_pool bf16 [B][H_kv][NB_max][2][bs][D] (device
    or pinned host) -> exact attention mass per block, fp32
    [B][H_kv][NB_max], summed over each KV head's query heads."""
    _need(q, "q", torch.bfloat16, 3)
    _need(kv_pool, "kv_pool", torch.bfloat16, 6, device=None)
    _need(ctx_len, "ctx_len", torch.int32, 1)
    B, H_q, D = q.shape
    H_kv, NB, bs = kv_pool.shape[1], kv_pool.shape[2], kv_pool.shape[4]
    _group(H_q, H_kv)
    _need(kv_pool, "kv_pool", torch.bfloat16, 6, device=None, shape=(B, H_kv, NB, 2, bs, D))
    _need(ctx_len, "ctx_len", torch.int32, 1, shape=(B,))
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(D)
    if mass is None:
        mass = torch.empty((B, H_kv, NB), dtype=torch.float32, device=q.device)
    _need(mass, "mass", torch.float32, 3, shape=(B, H_kv, NB))
    d = dims(B, H_q, H_kv, NB, D, bs)
    need = int(_lib.oasis_block_mass_workspace_bytes(ctypes.byref(d)))
    if ws is None or ws.numel() * ws.element_size() < need:
        ws = torch.empty((max(need, 1),), dtype=torch.uint8, device=q.device)
    _need_bytes(ws, "ws")
    _check(_lib.oasis_block_attention_mass(ctypes.byref(d), _ptr(q), _ptr(kv_pool), _ptr(ctx_len), float(sm_scale),
                                           _ptr(mass), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))
    return mass


def oasis_topk_overlap(sel_a: torch.Tensor, n_a: torch.Tensor, sel_b: torch.Tensor, n_b: torch.Tensor,
                       out=None, stream=None) -> torch.Tensor:
    """|A & B| per (request, KV head), int32 [B][H_kv], of two top-K lists."""
    for t, n in ((sel_a, "sel_a"), (sel_b, "sel_b")):
        _need(t, n, torch.int32, 3)
    for t, n in ((n_a, "n_a"), (n_b, "n_b")):
        _need(t, n, torch.int32, 2)
    B, H_kv, K = sel_a.shape
    _need(sel_b, "sel_b", torch.int32, 3, shape=(B, H_kv, K))
    _need(n_a, "n_a", torch.int32, 2, shape=(B, H_kv))
    _need(n_b, "n_b", torch.int32, 2, shape=(B, H_kv))
    if out is None:
        out = torch.empty((B, H_kv), dtype=torch.int32, device=sel_a.device)
    _need(out, "out", torch.int32, 2, shape=(B, H_kv))
    d = dims(B, H_kv, H_kv, 1)
    _check(_lib.oasis_topk_overlap(ctypes.byref(d), _ptr(sel_a), _ptr(n_a), _ptr(sel_b), _ptr(n_b), int(K),
                                   _ptr(out), _stream(stream)))
    return out


def oasis_stage_plan_bytes(B: int, H_kv: int, C: int) -> int:
    d = dims(B, H_kv, H_kv, 1)
    return int(_lib.oasis_stage_plan_bytes(ctypes.byref(d), int(C)))


def oasis_stage_buffer_bytes(n_blocks: int, D: int = 128, bs: int = 16) -> int:
    d = dims(1, 1, 1, 1, D, bs)
    return int(_lib.oasis_stage_buffer_bytes(ctypes.byref(d), int(n_blocks)))


def _stage_args(sel, n_sel, scores, ctx_len, K_b, C, step, slot_block, slot_stamp, host_pool, ws_pool,
                tbl_slot, tbl_block, tbl_n, plan, host_plan, stage_host, stage_dev, host_threads, copy_mode,
                stream, copy_stream, wait_event, done_event, plan_event, stats_accum=None):
    _need(sel, "sel", torch.int32, 3)
    _need(n_sel, "n_sel", torch.int32, 2)
    _need(scores, "scores", torch.float32, 3)
    _need(ctx_len, "ctx_len", torch.int32, 1)
    _need(slot_block, "slot_block", torch.int32, 3)
    _need(slot_stamp, "slot_stamp", torch.int32, 3)
    _need(host_pool, "host_pool", torch.bfloat16, 6, device=None)
    _need(ws_pool, "ws_pool", torch.bfloat16, 6)
    _need(tbl_slot, "tbl_slot", torch.int32, 3)
    _need(tbl_block, "tbl_block", torch.int32, 3)
    _need(tbl_n, "tbl_n", torch.int32, 2)
    B, H_kv, NB, two, bs, D = host_pool.shape
    if two != 2:
        raise ValueError(f"host_pool: dimension 3 must be 2 (K, V), got {two}")
    S = ws_pool.shape[2]
    K_sel = sel.shape[2]
    _need(ws_pool, "ws_pool", torch.bfloat16, 6, shape=(B, H_kv, S, 2, bs, D))
    _need(slot_block, "slot_block", torch.int32, 3, shape=(B, H_kv, S))
    _need(slot_stamp, "slot_stamp", torch.int32, 3, shape=(B, H_kv, S))
    _need(tbl_slot, "tbl_slot", torch.int32, 3, shape=(B, H_kv, K_b))
    _need(tbl_block, "tbl_block", torch.int32, 3, shape=(B, H_kv, K_b))
    _need(tbl_n, "tbl_n", torch.int32, 2, shape=(B, H_kv))
    _need(scores, "scores", torch.float32, 3, shape=(B, H_kv, NB))
    _need(sel, "sel", torch.int32, 3, shape=(B, H_kv, K_sel))
    _need(n_sel, "n_sel", torch.int32, 2, shape=(B, H_kv))
    _need(ctx_len, "ctx_len", torch.int32, 1, shape=(B,))
    _need_bytes(plan, "plan")
    if host_plan is not None:
        _need_bytes(host_plan, "host_plan", device="host")
    if stage_host is not None:
        _need_bytes(stage_host, "stage_host", device="host")
    if stage_dev is not None:
        _need_bytes(stage_dev, "stage_dev")
    if stats_accum is not None:
        _need(stats_accum, "stats_accum", torch.int64, 1, shape=(4,))
    d = dims(B, H_kv, H_kv, NB, D, bs)
    a = oasis_stage_args()
    a.sel, a.n_sel, a.K_sel, a.scores = sel.data_ptr(), n_sel.data_ptr(), K_sel, scores.data_ptr()
    a.K_b, a.C, a.S, a.step = int(K_b), int(C), int(S), int(step)
    a.slot_block, a.slot_stamp, a.ctx_len = slot_block.data_ptr(), slot_stamp.data_ptr(), ctx_len.data_ptr()
    a.host_pool, a.ws_pool = host_pool.data_ptr(), ws_pool.data_ptr()
    a.tbl_slot, a.tbl_block, a.tbl_n = tbl_slot.data_ptr(), tbl_block.data_ptr(), tbl_n.data_ptr()
    a.plan, a.plan_bytes = plan.data_ptr(), plan.numel() * plan.element_size()
    for name, t in (("host_plan", host_plan), ("stage_host", stage_host), ("stage_dev", stage_dev)):
        if t is not None:
            setattr(a, name, t.data_ptr())
            setattr(a, name + "_bytes", t.numel() * t.element_size())
    a.host_threads = int(host_threads)
    a.copy_mode = int(copy_mode)
    a.stream = _stream(stream)
    a.copy_stream = _stream(copy_stream) if copy_stream is not None else None
    a.wait_event = _event(wait_event)
    a.done_event = _event(done_event)
    a.plan_event = _event(plan_event)
    a.stats_accum = None if stats_accum is None else stats_accum.data_ptr()
    return d, a


def oasis_stage_blocks(*, sel, n_sel, scores, ctx_len, K_b: int, C: int, step: int, slot_block,
                       slot_stamp, host_pool, ws_pool, tbl_slot, tbl_block, tbl_n, plan,
                       host_plan=None, stage_host=None, stage_dev=None, host_threads: int = 0,
                       copy_mode: int = OASIS_COPY_KERNEL, stream=None, copy_stream=None, wait_event=None,
                       done_event=None, plan_event=None, stats_accum=None, want_stats: bool = False):
    """One staging step (include/oasis.h).  host_pool: pinned bf16
    [B][H_kv][NB_max][2][bs][D]; ws_pool: device bf16 [B][H_kv][S][2][bs][D];
    slot tables int32 [B][H_kv][S]; tables int32 [B][H_kv][K_b]; plan: device
    int32 of oasis_stage_plan_bytes() bytes.  The DMA engine also needs
    host_plan (pinned, as large as plan) and the staging buffers stage_host
    (pinned) and stage_dev (device).  stats_accum: optional device int64[4]
    that the step's admits, evictions, deferred admits and 1 are added to.
    With want_stats the call waits for the plan and returns the step's
    counts (oasis_stage_stats as a dict); otherwise it returns None."""
    d, a = _stage_args(sel, n_sel, scores, ctx_len, K_b, C, step, slot_block, slot_stamp, host_pool, ws_pool,
                       tbl_slot, tbl_block, tbl_n, plan, host_plan, stage_host, stage_dev, host_threads,
                       copy_mode, stream, copy_stream, wait_event, done_event, plan_event, stats_accum)
    st = oasis_stage_stats() if want_stats else None
    _check(_lib.oasis_stage_blocks(ctypes.byref(d), ctypes.byref(a), None if st is None else ctypes.byref(st)))
    return None if st is None else st.as_dict()


def oasis_stage_read_stats(plan: torch.Tensor, B: int, H_kv: int, C: int, stream=None) -> dict:
    """The counts of the staging step whose plan is in `plan` (fetch cap C):
    waits for `stream`, then reads the plan's totals."""
    _need_bytes(plan, "plan")
    d = dims(B, H_kv, H_kv, 1)
    st = oasis_stage_stats()
    _check(_lib.oasis_stage_read_stats(ctypes.byref(d), int(C), _ptr(plan), ctypes.byref(st), _stream(stream)))
    return st.as_dict()


def oasis_stage_plan(**kw):
    """The plan half of oasis_stage_blocks (same keyword arguments); never blocks."""
    d, a = _stage_args(**_stage_kw(kw))
    _check(_lib.oasis_stage_plan(ctypes.byref(d), ctypes.byref(a)))


def oasis_stage_copy(**kw):
    """The copy half of oasis_stage_blocks (same keyword arguments)."""
    d, a = _stage_args(**_stage_kw(kw))
    _check(_lib.oasis_stage_copy(ctypes.byref(d), ctypes.byref(a)))


def _stage_kw(kw):
    full = dict(host_plan=None, stage_host=None, stage_dev=None, host_threads=0, copy_mode=OASIS_COPY_KERNEL,
                stream=None, copy_stream=None, wait_event=None, done_event=None, plan_event=None,
                stats_accum=None)
    full.update(kw)
    return full


def oasis_attn_workspace_bytes(B: int, H_q: int, H_kv: int, T: int, n_split: int = 0) -> int:
    d = dims(B, H_q, H_kv, 1)
    return int(_lib.oasis_attn_workspace_bytes(ctypes.byref(d), int(T), int(n_split)))


def oasis_attn_num_splits(B: int, H_q: int, H_kv: int, T: int, n_split: int = 0) -> int:
    d = dims(B, H_q, H_kv, 1)
    return int(_lib.oasis_attn_num_splits(ctypes.byref(d), int(T), int(n_split)))


def oasis_attn_launch_shape(B: int, H_q: int, H_kv: int, n_q: int, T: int, n_split: int = 0):
    """(splits, waves per workgroup) of an attention launch with n_q queries per request."""
    d = dims(B, H_q, H_kv, 1)
    sp, wv = _I32(), _I32()
    _check(_lib.oasis_attn_launch_shape(ctypes.byref(d), int(n_q), int(T), int(n_split), ctypes.byref(sp),
                                        ctypes.byref(wv)))
    return sp.value, wv.value


def oasis_sparse_decode_attn(q: torch.Tensor, kv_pool: torch.Tensor, tbl_slot: torch.Tensor,
                             tbl_block: torch.Tensor, tbl_n: torch.Tensor, ctx_len: torch.Tensor,
                             sm_scale: Optional[float] = None, out=None, lse=None, ws=None,
                             n_split: int = 0, want_lse: bool = False, stream=None):
    """q bf16 [B][H_q][D], kv_pool bf16 [B][H_kv][P][2][bs][D], tables int32
    [B][H_kv][T] and [B][H_kv] -> out bf16 [B][H_q][D] (and lse fp32 [B][H_q])."""
    _need(q, "q", torch.bfloat16, 3)
    _need(kv_pool, "kv_pool", torch.bfloat16, 6)
    _need(tbl_slot, "tbl_slot", torch.int32, 3)
    _need(tbl_block, "tbl_block", torch.int32, 3)
    _need(tbl_n, "tbl_n", torch.int32, 2)
    _need(ctx_len, "ctx_len", torch.int32, 1)
    B, H_q, D = q.shape
    H_kv, P, bs = kv_pool.shape[1], kv_pool.shape[2], kv_pool.shape[4]
    _group(H_q, H_kv)
    _need(kv_pool, "kv_pool", torch.bfloat16, 6, shape=(B, H_kv, P, 2, bs, D))
    T = tbl_slot.shape[2]
    _need(tbl_slot, "tbl_slot", torch.int32, 3, shape=(B, H_kv, T))
    _need(tbl_block, "tbl_block", torch.int32, 3, shape=(B, H_kv, T))
    _need(tbl_n, "tbl_n", torch.int32, 2, shape=(B, H_kv))
    _need(ctx_len, "ctx_len", torch.int32, 1, shape=(B,))
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty((B, H_q, D), dtype=torch.bfloat16, device=q.device)
    _need(out, "out", torch.bfloat16, 3, shape=(B, H_q, D))
    if lse is None and want_lse:
        lse = torch.empty((B, H_q), dtype=torch.float32, device=q.device)
    if lse is not None:
        _need(lse, "lse", torch.float32, 2, shape=(B, H_q))
    d = dims(B, H_q, H_kv, max(P, 1), D, bs)
    need = int(_lib.oasis_attn_workspace_bytes(ctypes.byref(d), T, int(n_split)))
    if need and (ws is None or ws.numel() * ws.element_size() < need):
        ws = torch.empty((need,), dtype=torch.uint8, device=q.device)
    if ws is not None:
        _need_bytes(ws, "ws")
    _check(_lib.oasis_sparse_decode_attn(
        ctypes.byref(d), _ptr(q), _ptr(kv_pool), int(P), _ptr(tbl_slot), _ptr(tbl_block), _ptr(tbl_n),
        int(T), _ptr(ctx_len), float(sm_scale), _ptr(out), _ptr(lse), _ptr(ws),
        0 if ws is None else ws.numel() * ws.element_size(), int(n_split), _stream(stream)))
    return (out, lse) if want_lse or lse is not None else out


def oasis_sparse_decode_attn_static_bytes() -> int:
    """Bytes of the fixed split-K scratch of oasis_sparse_decode_attn_static."""
    return int(_lib.oasis_sparse_decode_attn_static_bytes())


def oasis_sparse_decode_attn_static(q: torch.Tensor, kv_pool: torch.Tensor, tbl_slot: torch.Tensor,
                                    tbl_block: torch.Tensor, tbl_n: torch.Tensor, ctx_len: torch.Tensor,
                                    sm_scale: Optional[float] = None, out=None, lse=None, n_split: int = 0,
                                    want_lse: bool = False, stream=None):
    """oasis_sparse_decode_attn without a workspace: the split-K partials go
    to the library's fixed device scratch, so the call allocates nothing
    (pass `out` / `lse` to allocate nothing here either).  Calls that overlap
    on one device race on that scratch."""
    _need(q, "q", torch.bfloat16, 3)
    _need(kv_pool, "kv_pool", torch.bfloat16, 6)
    _need(tbl_slot, "tbl_slot", torch.int32, 3)
    _need(tbl_block, "tbl_block", torch.int32, 3)
    _need(tbl_n, "tbl_n", torch.int32, 2)
    _need(ctx_len, "ctx_len", torch.int32, 1)
    B, H_q, D = q.shape
    H_kv, P, bs = kv_pool.shape[1], kv_pool.shape[2], kv_pool.shape[4]
    _group(H_q, H_kv)
    _need(kv_pool, "kv_pool", torch.bfloat16, 6, shape=(B, H_kv, P, 2, bs, D))
    T = tbl_slot.shape[2]
    _need(tbl_slot, "tbl_slot", torch.int32, 3, shape=(B, H_kv, T))
    _need(tbl_block, "tbl_block", torch.int32, 3, shape=(B, H_kv, T))
    _need(tbl_n, "tbl_n", torch.int32, 2, shape=(B, H_kv))
    _need(ctx_len, "ctx_len", torch.int32, 1, shape=(B,))
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty((B, H_q, D), dtype=torch.bfloat16, device=q.device)
    _need(out, "out", torch.bfloat16, 3, shape=(B, H_q, D))
    if lse is None and want_lse:
        lse = torch.empty((B, H_q), dtype=torch.float32, device=q.device)
    if lse is not None:
        _need(lse, "lse", torch.float32, 2, shape=(B, H_q))
    d = dims(B, H_q, H_kv, max(P, 1), D, bs)
    _check(_lib.oasis_sparse_decode_attn_static(
        ctypes.byref(d), _ptr(q), _ptr(kv_pool), int(P), _ptr(tbl_slot), _ptr(tbl_block), _ptr(tbl_n),
        int(T), _ptr(ctx_len), float(sm_scale), _ptr(out), _ptr(lse), int(n_split), _stream(stream)))
    return (out, lse) if want_lse or lse is not None else out


def oasis_lookahead_attn_workspace_bytes(B: int, H_q: int, H_kv: int, n_q: int, T: int, n_split: int = 0) -> int:
    d = dims(B, H_q, H_kv, 1)
    return int(_lib.oasis_lookahead_attn_workspace_bytes(ctypes.byref(d), int(n_q), int(T), int(n_split)))


def oasis_lookahead_attn(q: torch.Tensor, kv_pool: torch.Tensor, tbl_slot: torch.Tensor, tbl_block: torch.Tensor,
                         tbl_n: torch.Tensor, ctx_len: torch.Tensor, sm_scale: Optional[float] = None, out=None,
                         lse=None, ws=None, n_split: int = 0, want_lse: bool = False, stream=None):
    """q bf16 [B][n_q][H_q][D] (the normal query and the drafts), kv_pool bf16
    [B][H_kv][P][2][bs][D], tables int32 [B][H_kv][T] and [B][H_kv] ->
    out bf16 [B][n_q][H_q][D] (and lse fp32 [B][n_q][H_q])."""
    _need(q, "q", torch.bfloat16, 4)
    _need(kv_pool, "kv_pool", torch.bfloat16, 6)
    _need(tbl_slot, "tbl_slot", torch.int32, 3)
    _need(tbl_block, "tbl_block", torch.int32, 3)
    _need(tbl_n, "tbl_n", torch.int32, 2)
    _need(ctx_len, "ctx_len", torch.int32, 1)
    B, n_q, H_q, D = q.shape
    H_kv, P, bs = kv_pool.shape[1], kv_pool.shape[2], kv_pool.shape[4]
    _group(H_q, H_kv)
    _need(kv_pool, "kv_pool", torch.bfloat16, 6, shape=(B, H_kv, P, 2, bs, D))
    T = tbl_slot.shape[2]
    _need(tbl_slot, "tbl_slot", torch.int32, 3, shape=(B, H_kv, T))
    _need(tbl_block, "tbl_block", torch.int32, 3, shape=(B, H_kv, T))
    _need(tbl_n, "tbl_n", torch.int32, 2, shape=(B, H_kv))
    _need(ctx_len, "ctx_len", torch.int32, 1, shape=(B,))
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty((B, n_q, H_q, D), dtype=torch.bfloat16, device=q.device)
    _need(out, "out", torch.bfloat16, 4, shape=(B, n_q, H_q, D))
    if lse is None and want_lse:
        lse = torch.empty((B, n_q, H_q), dtype=torch.float32, device=q.device)
    if lse is not None:
        _need(lse, "lse", torch.float32, 3, shape=(B, n_q, H_q))
    d = dims(B, H_q, H_kv, max(P, 1), D, bs)
    need = int(_lib.oasis_lookahead_attn_workspace_bytes(ctypes.byref(d), int(n_q), T, int(n_split)))
    if need and (ws is None or ws.numel() * ws.element_size() < need):
        ws = torch.empty((need,), dtype=torch.uint8, device=q.device)
    if ws is not None:
        _need_bytes(ws, "ws")
    _check(_lib.oasis_lookahead_attn(
        ctypes.byref(d), int(n_q), _ptr(q), _ptr(kv_pool), int(P), _ptr(tbl_slot), _ptr(tbl_block), _ptr(tbl_n),
        int(T), _ptr(ctx_len), float(sm_scale), _ptr(out), _ptr(lse), _ptr(ws),
        0 if ws is None else ws.numel() * ws.element_size(), int(n_split), _stream(stream)))
    return (out, lse) if want_lse or lse is not None else out


# -------------------------------------------------------------------------- layer pipeline


def oasis_pipeline_create(d: oasis_dims, desc: oasis_pipeline_desc) -> int:
    """Creates a native layer pipeline (include/oasis.h); returns its handle."""
    h = ctypes.c_void_p()
    _check(_lib.oasis_pipeline_create(ctypes.byref(d), ctypes.byref(desc), ctypes.byref(h)))
    return h.value


def oasis_pipeline_layer_step(h: int, layer: int, step: int, q_look: torch.Tensor,
                              q_attn: Optional[torch.Tensor], out: Optional[torch.Tensor],
                              lse: Optional[torch.Tensor] = None):
    """One layer-step: q_look bf16 [B][J][H_q][D], q_attn bf16 [B][n_q][H_q][D]
    (or [B][H_q][D] when n_q = 1; unused at step 0), out bf16 of q_attn's
    shape, lse fp32 [B][n_q][H_q] or None."""
    _need(q_look, "q_look", torch.bfloat16, 4)
    if q_attn is not None:
        _need(q_attn, "q_attn", torch.bfloat16, q_attn.dim())
    _check(_lib.oasis_pipeline_layer_step(h, int(layer), int(step), q_look.data_ptr(),
                                          None if q_attn is None else q_attn.data_ptr(),
                                          None if out is None else out.data_ptr(),
                                          None if lse is None else lse.data_ptr()))


def oasis_pipeline_drain(h: int):
    _check(_lib.oasis_pipeline_drain(h))


def oasis_pipeline_stream(h: int, which: int) -> Optional[int]:
    s = ctypes.c_void_p()
    _check(_lib.oasis_pipeline_stream(h, int(which), ctypes.byref(s)))
    return s.value


def oasis_pipeline_issue_threads(h: int) -> bool:
    """Whether the pipeline's chain and copies are enqueued by issue threads."""
    on = _I32()
    _check(_lib.oasis_pipeline_issue_threads(h, ctypes.byref(on)))
    return bool(on.value)


def oasis_pipeline_timing(h: int, capacity: int, kinds: int = 0xF, every: int = 1):
    _check(_lib.oasis_pipeline_timing(h, int(capacity), int(kinds), int(every)))


def oasis_pipeline_timing_read(h: int, kind: int):
    """(total milliseconds, count) of the timed launches of one kind."""
    ms, n = ctypes.c_double(), _I32()
    _check(_lib.oasis_pipeline_timing_read(h, int(kind), ctypes.byref(ms), ctypes.byref(n)))
    return ms.value, n.value


def oasis_pipeline_timing_values(h: int, kind: int, capacity: int):
    """Milliseconds of each timed launch of one kind, in launch order (at
    most `capacity` of them)."""
    buf = (ctypes.c_float * max(int(capacity), 1))()
    n = _I32()
    _check(_lib.oasis_pipeline_timing_values(h, int(kind), buf, int(capacity), ctypes.byref(n)))
    return [buf[i] for i in range(min(n.value, int(capacity)))]


def oasis_pipeline_copy_host_seconds(h: int):
    sec, n = ctypes.c_double(), _I32()
    _check(_lib.oasis_pipeline_copy_host_seconds(h, ctypes.byref(sec), ctypes.byref(n)))
    return sec.value, n.value


def oasis_pipeline_destroy(h: Optional[int]):
    if h:
        _check(_lib.oasis_pipeline_destroy(h))
