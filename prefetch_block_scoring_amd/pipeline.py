"""Per-layer decode chain overlapped across layers and decode steps.

The OasisKV pages (arXiv 2608.08097, paperlayer summary, section 4) run, per
layer, a background chain of top-K prediction, KV selection and KV transfer,
with independent workers overlapped across layers and decode steps; the
foreground waits only for the relevant layer's transfer before that layer's
next-step attention.  `LayerPipeline` schedules the library's calls that way
on one GPU:

  main stream     attention of (layer l, step t), after the transfer of
                  (l, t - 1) only
  compute stream  scores and top-K of (l, t), then the staging plan of (l, t)
  copy stream     the copies of (l, t) (gather kernel, or DMA copy + scatter)

Per layer the buffers rotate so that the compute stream can run ahead: three
attention tables (step t attends table t % 3, the plan of step t writes
(t + 1) % 3) and two plan workspaces.  The plan of step t therefore waits for
the attention of step t - 2 (the last reader of its table) and for the copies
of step t - 2 (the last reader of its plan), and the copies of step t wait
for the attention of step t - 1 (whose slots they may refill).  The copy half
of a staging step blocks its thread with the DMA engine, so it runs on one
worker thread, in submission order.

Workloads without staging (K/V fully in HBM) run the same chain without the
copy stream: the attention of step t reads the full pool through the
selection of step t - 1.

Argument marshalling and scheduling only: every step runs in the library.
"""
from __future__ import annotations

import concurrent.futures
import time
from typing import Callable, Optional

import torch

from . import binding as oa


class _Layer:
    def __init__(self, B, H_q, H_kv, NB, K_b, C, staged, copy_mode, dev, D=128, bs=16):
        i32 = torch.int32
        self.scores = torch.empty((B, H_kv, NB), dtype=torch.float32, device=dev)
        self.sel = [torch.empty((B, H_kv, K_b), dtype=i32, device=dev) for _ in range(2)]
        self.n_sel = [torch.empty((B, H_kv), dtype=i32, device=dev) for _ in range(2)]
        self.out = torch.empty((B, H_q, D), dtype=torch.bfloat16, device=dev)
        self.lse = torch.empty((B, H_q), dtype=torch.float32, device=dev)
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
            if copy_mode == oa.OASIS_COPY_DMA:
                self.host_plan = oa.oasis_host_empty((n_plan,), i32)
                sbytes = oa.oasis_stage_buffer_bytes(B * H_kv * max(C, 1))
                self.stage_host = [oa.oasis_host_empty((sbytes,), torch.uint8) for _ in range(2)]
                self.stage_dev = torch.empty(sbytes, dtype=torch.uint8, device=dev)
            else:
                self.host_plan, self.stage_host, self.stage_dev = None, [None, None], None


class LayerPipeline:
    """Runs `n_layers` layers of the decode path over one batch.

    pool:  bf16 [B][H_kv][NB_max][2][bs][D]; pinned host (oasis_host_empty)
           when staged, else device memory.
    summ:  the pool's block summaries (oasis_build_summaries), device.
    ctx:   int32 [B] context lengths, device.
    Step 0 of every layer is the uncapped initial fill (staged workloads).
    """

    def __init__(self, *, pool, summ, ctx, H_q: int, K_b: int, C: int, n_layers: int, staged: bool,
                 copy_mode: int = oa.OASIS_COPY_KERNEL, host_threads: int = 8, n_split: int = 0,
                 timer: Optional[Callable] = None):
        B, H_kv, NB, _, bs, D = pool.shape
        self.B, self.H_q, self.H_kv, self.NB, self.K_b, self.C = B, H_q, H_kv, NB, K_b, C
        self.pool, self.summ, self.ctx = pool, summ, ctx
        self.staged, self.copy_mode, self.host_threads, self.n_split = staged, copy_mode, host_threads, n_split
        self.L = n_layers
        dev = ctx.device
        self.layers = [_Layer(B, H_q, H_kv, NB, K_b, C, staged, copy_mode, dev, D, bs) for _ in range(n_layers)]
        self.main = torch.cuda.current_stream()
        self.comp = torch.cuda.Stream()
        self.copy = torch.cuda.Stream() if staged else None
        ws = oa.oasis_attn_workspace_bytes(B, H_q, H_kv, K_b, n_split)
        self.attn_ws = [torch.empty((max(ws, 1),), dtype=torch.uint8, device=dev) for _ in range(n_layers)]
        self.events = {}
        self.pending = {}
        self.stager = concurrent.futures.ThreadPoolExecutor(max_workers=1) if staged else None
        self.timer = timer or (lambda name, stream, fn: fn())
        self.copy_host_s = []

    # ------------------------------------------------------------ helpers

    def _ev(self, kind, l, t):
        key = (kind, l, t)
        e = self.events.get(key)
        if e is None:
            e = self.events[key] = torch.cuda.Event()
        return e

    def _forget(self, l, t):
        for kind in ("attn", "stage", "plan", "sel"):
            self.events.pop((kind, l, t), None)

    def _stage_kw(self, l, t):
        ly = self.layers[l]
        j = t % 2
        tb = ly.tbls[(t + 1) % 3]
        return dict(
            sel=ly.sel[j], n_sel=ly.n_sel[j], scores=ly.scores, ctx_len=self.ctx, K_b=self.K_b,
            C=self.K_b if t == 0 else self.C, step=t, slot_block=ly.slot_block, slot_stamp=ly.slot_stamp,
            host_pool=self.pool, ws_pool=ly.ws_pool, tbl_slot=tb[0], tbl_block=tb[1], tbl_n=tb[2],
            plan=ly.plans[j], host_plan=ly.host_plan, stage_host=ly.stage_host[j], stage_dev=ly.stage_dev,
            host_threads=self.host_threads, copy_mode=self.copy_mode, stream=self.comp,
            copy_stream=self.copy, done_event=self._ev("stage", l, t), plan_event=self._ev("plan", l, t),
            wait_event=self._ev("attn", l, t - 1) if t >= 2 else None)

    def _copy(self, kw):
        h0 = time.perf_counter()
        oa.oasis_stage_copy(**kw)
        self.copy_host_s.append(time.perf_counter() - h0)

    # ------------------------------------------------------------ one layer-step

    def layer_step(self, l: int, t: int, q_look: torch.Tensor, q_attn: Optional[torch.Tensor]):
        """Enqueue layer l's work of decode step t: the attention of step t
        (query q_attn, over the working set staged at step t - 1; skipped at
        t = 0) and the prediction and staging for step t + 1 from the
        lookahead queries q_look.  The attention output lands in
        `self.layers[l].out` / `.lse` once the main stream reaches it."""
        ly = self.layers[l]
        main, comp = self.main, self.comp
        j = t % 2
        if t >= 1:
            if self.staged:
                self.pending.pop((l, t - 1)).result()        # its done event is recorded
                tb = ly.tbls[t % 3]
                main.wait_event(self._ev("stage", l, t - 1))
                self.timer("attn", main, lambda: oa.oasis_sparse_decode_attn(
                    q_attn, ly.ws_pool, tb[0], tb[1], tb[2], self.ctx, out=ly.out, lse=ly.lse,
                    ws=self.attn_ws[l], n_split=self.n_split, stream=main))
            else:
                jp = (t - 1) % 2
                main.wait_event(self._ev("sel", l, t - 1))
                self.timer("attn", main, lambda: oa.oasis_sparse_decode_attn(
                    q_attn, self.pool, ly.sel[jp], ly.sel[jp], ly.n_sel[jp], self.ctx, out=ly.out,
                    lse=ly.lse, ws=self.attn_ws[l], n_split=self.n_split, stream=main))
            self._ev("attn", l, t).record(main)
        with torch.cuda.stream(comp):
            self.timer("score", comp, lambda: oa.oasis_score_blocks(q_look, self.summ, self.ctx,
                                                                    scores=ly.scores, stream=comp))
            if t >= 2:
                # sel[j] (no staging) and table (t + 1) % 3 were last read by
                # the attention of step t - 2 ... t - 1
                comp.wait_event(self._ev("attn", l, t - 1 if not self.staged else t - 2))
            self.timer("topk", comp, lambda: oa.oasis_select_topk(ly.scores, self.ctx, self.K_b, sel=ly.sel[j],
                                                                  n_sel=ly.n_sel[j], stream=comp))
            if not self.staged:
                self._ev("sel", l, t).record(comp)
            else:
                if t >= 2:
                    comp.wait_event(self._ev("stage", l, t - 2))   # plan[j] was read by those copies
                kw = self._stage_kw(l, t)
                self.timer("plan", comp, lambda: oa.oasis_stage_plan(**kw))
        if self.staged:
            self.pending[(l, t)] = self.stager.submit(self._copy, kw)
        if t >= 3:
            self._forget(l, t - 3)

    def admitted(self, l: int, t: int) -> torch.Tensor:
        """Device scalar: total admits of layer l's staging at step t (valid
        once the plan of that step has run and until step t + 2 plans)."""
        ly = self.layers[l]
        row = 4 + 2 * max(self.K_b if t == 0 else self.C, 1)
        return ly.plans[t % 2][self.B * self.H_kv * row]

    def table(self, l: int, t: int):
        """(slot, block, n) tables that the attention of step t reads."""
        return self.layers[l].tbls[t % 3]

    def drain(self):
        for f in list(self.pending.values()):
            f.result()

    def close(self):
        self.drain()
        if self.stager is not None:
            self.stager.shutdown()
