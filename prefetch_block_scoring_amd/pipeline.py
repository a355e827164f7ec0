"""Per-layer decode chain overlapped across layers and decode steps.

OasisKV (arXiv 2608.08097), paperlayer summary, section 4.  Prediction,
selection and the copy of the admitted blocks for a layer run off the
critical path, so that several layers and decode steps are in flight at once;
a layer's attention is held back only until its own working set has been
copied.  The library's native pipeline (oasis_pipeline_* in include/oasis.h)
lays that out on one GPU's streams:

  main stream     attention of (layer l, step t), after the transfer of
                  (l, t - 1) only
  compute stream  scores and top-K of (l, t), then the staging plan of (l, t)
                  (one stream when nothing is staged; two by layer parity for
                  a staged step that the link does not bind; otherwise the
                  main stream itself, behind each attention;
                  `compute_streams` overrides)
  copy streams    the copies of (l, t) (gather kernels, on two streams by
                  layer parity when the chain is on the main stream, or DMA
                  copy + scatter, or, mixed, DMA for even layers and gathers
                  for odd layers)

With compute streams of its own, the chain and the copies of a layer-step
are enqueued by the pipeline's two issue threads, which make the chain's
cross-stream waits on the host, and the calling thread enqueues only the
attention (`issue_threads`; without staging the calling thread then waits
on the host for the selection its attention reads).

`LayerPipeline` allocates the per-layer buffers the native pipeline works in
(three attention tables, two selections and two plan buffers per layer, the
working sets) and issues one native call per layer-step.  Workloads without
staging (K/V fully in HBM) run the same chain without the copy stream: the
attention of step t reads the full pool through the selection of step t - 1.

Argument marshalling only: every step runs in the library.
"""
from __future__ import annotations

import ctypes
import math
from typing import Optional

import torch

from . import binding as oa

TIMING_KINDS = {"attn": 0, "score": 1, "topk": 2, "plan": 3}


class _Layer:
    def __init__(self, B, H_q, H_kv, NB, K_b, C, staged, copy_mode, ws_bytes, dev, D=128, bs=16, n_q=1):
        i32 = torch.int32
        self.scores = torch.empty((B, H_kv, NB), dtype=torch.float32, device=dev)
        self.sel = [torch.empty((B, H_kv, K_b), dtype=i32, device=dev) for _ in range(2)]
        self.n_sel = [torch.empty((B, H_kv), dtype=i32, device=dev) for _ in range(2)]
        # attention output: [B][H_q][D], or [B][n_q][H_q][D] for look-ahead attention
        qs = (B, H_q) if n_q == 1 else (B, n_q, H_q)
        self.out = torch.empty(qs + (D,), dtype=torch.bfloat16, device=dev)
        self.lse = torch.empty(qs, dtype=torch.float32, device=dev)
        self.attn_ws = torch.empty((max(ws_bytes, 1),), dtype=torch.uint8, device=dev)
        self.ws_pool = self.slot_block = self.slot_stamp = None
        self.tbls, self.plans, self.host_plan, self.stage_host, self.stage_dev = [], [], None, [None, None], None
        if staged:
            S = K_b + C
            self.ws_pool = torch.empty((B, H_kv, S, 2, bs, D), dtype=torch.bfloat16, device=dev)
            self.slot_block = torch.full((B, H_kv, S), -1, dtype=i32, device=dev)
            self.slot_stamp = torch.full_like(self.slot_block, -1)
            self.tbls = [(torch.empty((B, H_kv, K_b), dtype=i32, device=dev),
                          torch.empty((B, H_kv, K_b), dtype=i32, device=dev),
                          torch.zeros((B, H_kv), dtype=i32, device=dev)) for _ in range(3)]
            n_plan = oa.oasis_stage_plan_bytes(B, H_kv, K_b) // 4
            self.plans = [torch.empty(n_plan, dtype=i32, device=dev) for _ in range(2)]
            if copy_mode in (oa.OASIS_COPY_DMA, oa.OASIS_COPY_MIXED):
                self.host_plan = oa.oasis_host_empty((n_plan,), i32)
                sbytes = oa.oasis_stage_buffer_bytes(B * H_kv * max(C, 1))
                self.stage_host = [oa.oasis_host_empty((sbytes,), torch.uint8) for _ in range(2)]
                self.stage_dev = torch.empty(sbytes, dtype=torch.uint8, device=dev)

    def buffers(self) -> oa.oasis_layer_buffers:
        b = oa.oasis_layer_buffers()
        p = lambda t: None if t is None else t.data_ptr()
        b.scores = p(self.scores)
        for k in range(2):
            b.sel[k], b.n_sel[k] = p(self.sel[k]), p(self.n_sel[k])
        b.attn_ws, b.attn_ws_bytes = p(self.attn_ws), self.attn_ws.numel()
        if self.ws_pool is not None:
            b.ws_pool, b.slot_block, b.slot_stamp = p(self.ws_pool), p(self.slot_block), p(self.slot_stamp)
            for k in range(3):
                b.tbl_slot[k], b.tbl_block[k], b.tbl_n[k] = (p(x) for x in self.tbls[k])
            for k in range(2):
                b.plan[k] = p(self.plans[k])
            b.plan_bytes = self.plans[0].numel() * 4
            if self.host_plan is not None:
                b.host_plan, b.stage_dev = p(self.host_plan), p(self.stage_dev)
                for k in range(2):
                    b.stage_host[k] = p(self.stage_host[k])
                b.stage_bytes = min(self.stage_dev.numel(), self.stage_host[0].numel())
        return b


class LayerPipeline:
    """Runs `n_layers` layers of the decode path over one batch.

    pool:  bf16 [B][H_kv][NB_max][2][bs][D]; pinned host (oasis_host_empty)
           when staged, else device memory.
    summ:  the pool's block summaries (oasis_build_summaries), device.
    ctx:   int32 [B] context lengths, device.
    n_q:   attention queries per request; 1 + J runs look-ahead attention of
           the normal and the draft queries (q_attn [B][n_q][H_q][D]).
    The attention runs on the stream current at construction (`main`); the
    compute and copy streams belong to the native pipeline.  Step 0 of every
    layer is the uncapped initial fill (staged workloads).  The caller keeps
    the query tensors it passes alive until their work has completed.
    """

    def __init__(self, *, pool, summ, ctx, H_q: int, K_b: int, C: int, n_layers: int, staged: bool,
                 copy_mode: int = oa.OASIS_COPY_KERNEL, host_threads: int = 8, n_split: int = 0, J: int = 1,
                 n_q: int = 1, compute_streams: int = 0, issue_threads: int = 0):
        B, H_kv, NB, _, bs, D = pool.shape
        if tuple(summ.shape) != (B, H_kv, NB, 2, D) or summ.dtype != torch.bfloat16 or not summ.is_cuda:
            raise ValueError(f"summ: expected bf16 device [B][H_kv][NB_max][2][D] = {(B, H_kv, NB, 2, D)}, "
                             f"got {summ.dtype} {tuple(summ.shape)}")
        if tuple(ctx.shape) != (B,) or ctx.dtype != torch.int32 or not ctx.is_cuda:
            raise ValueError(f"ctx: expected int32 device [B] = ({B},), got {ctx.dtype} {tuple(ctx.shape)}")
        if H_q % H_kv != 0:
            raise ValueError(f"H_q = {H_q} is not a multiple of H_kv = {H_kv}")
        self.B, self.H_q, self.H_kv, self.NB, self.K_b, self.C = B, H_q, H_kv, NB, K_b, C
        self.block_bytes = 2 * bs * D * pool.element_size()  # K and V of one block
        self.pool, self.summ, self.ctx = pool, summ, ctx
        self.staged, self.copy_mode = staged, copy_mode
        self.L, self.J, self.n_q = n_layers, J, n_q
        dev = ctx.device
        ws = oa.oasis_lookahead_attn_workspace_bytes(B, H_q, H_kv, n_q, K_b, n_split)
        self.layers = [_Layer(B, H_q, H_kv, NB, K_b, C, staged, copy_mode, ws, dev, D, bs, n_q)
                       for _ in range(n_layers)]
        self.main = torch.cuda.current_stream()
        # admits, evictions, deferred admits and staging steps of every layer,
        # added by the plan kernels on the device
        self.stats = torch.zeros(4, dtype=torch.int64, device=dev)
        bufs = (oa.oasis_layer_buffers * n_layers)(*[ly.buffers() for ly in self.layers])
        desc = oa.oasis_pipeline_desc(
            n_layers=n_layers, K_b=K_b, C=C if staged else 0, J=J, n_q=n_q, staged=int(staged),
            copy_mode=copy_mode,
            host_threads=host_threads, n_split=n_split, sm_scale=1.0 / math.sqrt(D), pool=pool.data_ptr(),
            kminmax=summ.data_ptr(), ctx_len=ctx.data_ptr(), main_stream=self.main.cuda_stream,
            layers=ctypes.cast(bufs, ctypes.POINTER(oa.oasis_layer_buffers)), compute_streams=compute_streams,
            issue_threads=issue_threads,
            stage_stats=self.stats.data_ptr() if staged else None)
        self._h = oa.oasis_pipeline_create(oa.dims(B, H_q, H_kv, NB, D, bs), desc)
        c1 = oa.oasis_pipeline_stream(self._h, 1)
        odd = oa.oasis_pipeline_stream(self._h, 4)
        # -1: the chain shares the main stream (whose handle is NULL when it
        # is the default stream)
        on_main = c1 == self.main.cuda_stream or not c1
        self.comp = self.main if on_main else torch.cuda.ExternalStream(c1)
        self._comp_odd = torch.cuda.ExternalStream(odd) if odd else self.comp
        self.compute_streams = -1 if on_main else (2 if odd else 1)
        # whether worker threads enqueue the chain and the copies
        self.issue_threads = oa.oasis_pipeline_issue_threads(self._h)
        self.copy = [torch.cuda.ExternalStream(c) for c in
                     (oa.oasis_pipeline_stream(self._h, k) for k in (2, 3)) if c]

    def layer_step(self, l: int, t: int, q_look: torch.Tensor, q_attn: Optional[torch.Tensor]):
        """Enqueue layer l's work of decode step t: the attention of step t
        (query q_attn, over the working set staged at step t - 1; skipped at
        t = 0) and the prediction and staging for step t + 1 from the
        lookahead queries q_look.  The attention output lands in
        `self.layers[l].out` / `.lse` once the main stream reaches it."""
        D = self.layers[l].out.shape[-1]
        if tuple(q_look.shape) != (self.B, self.J, self.H_q, D):
            raise ValueError(f"q_look shape {tuple(q_look.shape)}: expected [B][J = {self.J}][H_q][D]")
        if t >= 1 and (q_attn is None or q_attn.numel() != self.B * self.n_q * self.H_q * D
                       or q_attn.dtype != torch.bfloat16 or not q_attn.is_cuda or not q_attn.is_contiguous()):
            raise ValueError(f"q_attn: expected contiguous bf16 device [B][n_q = {self.n_q}][H_q][D], got "
                             f"{None if q_attn is None else (q_attn.dtype, tuple(q_attn.shape))}")
        ly = self.layers[l]
        oa.oasis_pipeline_layer_step(self._h, l, t, q_look, q_attn if t >= 1 else None, ly.out, ly.lse)

    def comp_stream(self, l: int):
        """The compute stream that runs layer l's scores, top-K and plan."""
        return self._comp_odd if l & 1 else self.comp

    def admitted(self, l: int, t: int) -> torch.Tensor:
        """Device scalar: total admits of layer l's staging at step t (valid
        once the plan of that step has run and until step t + 2 plans)."""
        ly = self.layers[l]
        row = 4 + 2 * max(self.K_b if t == 0 else self.C, 1)
        return ly.plans[t % 2][self.B * self.H_kv * row]

    def reset_stage_stats(self):
        """Clears the staging counters; call it with no layer-step in flight
        (it synchronises the device, so the clear is done before any later
        plan kernel adds to them)."""
        self.stats.zero_()
        torch.cuda.synchronize(self.stats.device)

    def stage_stats(self) -> dict:
        """Admits, evictions, deferred admits and staging steps summed over
        every layer since the last reset (synchronises the device)."""
        torch.cuda.synchronize(self.stats.device)
        a, e, d, n = (int(x) for x in self.stats.cpu().tolist())
        return {"admits": a, "evictions": e, "deferred": d, "steps": n,
                "bytes": a * self.block_bytes}

    def table(self, l: int, t: int):
        """(slot, block, n) tables that the attention of step t reads."""
        return self.layers[l].tbls[t % 3]

    def enable_timing(self, capacity: int, kinds=("attn", "score", "topk", "plan"), every: int = 1):
        """Time up to `capacity` launches of each of `kinds` (attn, score,
        topk, plan), one in every `every` of them, with events bound to
        their kernels; clears earlier totals."""
        oa.oasis_pipeline_timing(self._h, capacity, sum(1 << TIMING_KINDS[k] for k in kinds), every)

    def timing(self, kind: str):
        """(average microseconds, count) of the timed launches of `kind`."""
        ms, n = oa.oasis_pipeline_timing_read(self._h, TIMING_KINDS[kind])
        return (ms * 1e3 / n if n else 0.0), n

    def timing_values(self, kind: str, capacity: int):
        """Microseconds of each timed launch of `kind`, in launch order."""
        return [ms * 1e3 for ms in oa.oasis_pipeline_timing_values(self._h, TIMING_KINDS[kind], capacity)]

    def copy_host_seconds(self):
        """(host seconds in the copy half of staging, calls) since timing
        was last enabled."""
        return oa.oasis_pipeline_copy_host_seconds(self._h)

    def drain(self):
        """Returns once the worker threads have enqueued every layer-step
        submitted so far (no device synchronisation)."""
        oa.oasis_pipeline_drain(self._h)

    def close(self):
        if self._h:
            oa.oasis_pipeline_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
