"""Seeded synthetic workloads for the lookahead block-scoring decode path.

This module only draws random inputs: lookahead (draft) queries, the attention
query, a paged K/V pool with a planted importance structure, context lengths,
and, for unit tests of single calls, stand-alone score rows, predicted-set
sequences and attention tables.  It holds no step of the method (no summaries,
no scoring, no selection, no staging rule, no attention); both the HIP path and
the CPU oracle receive what it draws.

Shapes follow the OasisKV pages (arXiv 2608.08097, "OasisKV: Scaling In-Decode
KV Cache Beyond HBM with Lookahead Sparse Prefetching"): Qwen3-8B-shaped GQA
layers at 16K context with a 2048-token budget (paperlayer summary, section 5),
a 32B-class GQA layer of 256 KiB KV per token over 64 layers (section 2), a
reasoning workload with several draft queries, and a 0.05 fetch cap (section 5,
"Eviction Strategy").  The pages measure on LongBench v2, AIME, GPQA and GSM8K;
none of those suites is used here: these seeded synthetic inputs stand in for
their shapes.

Layouts (row-major, bf16 unless noted):
  q_look  [B][J][H_q][D]              lookahead queries
  q       [B][H_q][D]                 attention query
  kv      [B][H_kv][NB_max][2][bs][D] paged pool; index 0 = K, 1 = V, so one
                                      block of one KV head is contiguous
  ctx_len int32 [B]

Every tensor comes from its own torch.Generator seeded from (workload seed,
purpose, request), so values do not depend on generation order or chunking.
The CPU and CUDA generators give different streams: a test draws once, on one
device, and hands copies to both sides.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, replace
from typing import Optional, Tuple, Union

import torch

# token value written into K and V positions past a request's context: large
# enough that any unmasked use of a padding token shows up in parity tests
PAD_VALUE = 64.0

_PURPOSE = {"ctx": 1, "qbase": 2, "kv": 3, "plant": 4, "drift": 5, "qstep": 6,
            "scores": 7, "sets": 8, "table": 9, "attnq": 10, "truenext": 11}


@dataclass(frozen=True)
class Workload:
    """One synthetic decode layer.

    ctx is either a fixed context length or an inclusive (lo, hi) range drawn
    uniformly per request.  structure is one of:
      "planted": `planted` blocks per (request, KV head) get every key shifted
                 by 2 * qbar, the mean lookahead query of that KV head's group;
      "drift":   keys carry a rotating direction; the lookahead turns by a
                 fixed angle per step so that about `drift` of the budget
                 changes per step;
      "zipf":    keys get 2 * qbar * rank^(-zipf_s) over a random rank order;
      "none":    plain N(0, 1).
    """
    name: str
    B: int
    H_q: int
    H_kv: int
    D: int = 128
    bs: int = 16
    ctx: Union[int, Tuple[int, int]] = 16384
    budget: int = 2048
    J: int = 1
    cap: Optional[float] = None        # fetch-cap fraction; None = full KV in HBM
    steps: int = 1
    structure: str = "planted"
    planted: int = 0
    drift: float = 0.05
    drift_amp: float = 8.0
    zipf_s: float = 1.1
    seed: int = 0

    @property
    def G(self) -> int:
        return self.H_q // self.H_kv

    @property
    def ctx_max(self) -> int:
        return self.ctx if isinstance(self.ctx, int) else self.ctx[1]

    @property
    def NB_max(self) -> int:
        return -(-self.ctx_max // self.bs)

    @property
    def K_b(self) -> int:
        return self.budget // self.bs

    @property
    def staged(self) -> bool:
        return self.cap is not None

    def shrink(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS = {
    # 8 query / 2 KV heads, one request of 4096 tokens, 512-token budget
    "parity_8q2kv_4k": Workload(
        "parity_8q2kv_4k", B=1, H_q=8, H_kv=2, ctx=4096, budget=512, J=1,
        structure="planted", planted=8, seed=1001),
    # Qwen3-8B-shaped layer, KV fully in HBM
    "qwen3_8b_16k_b32_hbm": Workload(
        "qwen3_8b_16k_b32_hbm", B=32, H_q=32, H_kv=8, ctx=16384, budget=2048,
        J=1, structure="planted", planted=51, seed=1002),
    # Qwen3-8B-shaped layer, KV pool in pinned host memory, 64 staged steps
    "qwen3_8b_16k_b128_staged": Workload(
        "qwen3_8b_16k_b128_staged", B=128, H_q=32, H_kv=8, ctx=16384,
        budget=2048, J=1, cap=0.05, steps=64, structure="drift", seed=1003),
    # long-reasoning layer: 32K context, 4 draft queries summed
    "reasoning_32k_b64_j4": Workload(
        "reasoning_32k_b64_j4", B=64, H_q=32, H_kv=8, ctx=32768, budget=2048,
        J=4, structure="zipf", seed=1004),
    # 32B-class GQA layer, ragged contexts, pinned host pool
    "gqa32b_ragged_b16_staged": Workload(
        "gqa32b_ragged_b16_staged", B=16, H_q=64, H_kv=8, ctx=(8192, 65536),
        budget=2048, J=1, cap=0.05, steps=64, structure="drift", seed=1005),
}


def generator(w: Workload, purpose: str, index: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed((w.seed * 1000003 + _PURPOSE[purpose] * 7919 + index) & 0x7FFFFFFFFFFF)
    return g


def _randn(shape, gen, device, scale=1.0):
    return torch.randn(shape, generator=gen, device=device, dtype=torch.float32) * scale


def context_lengths(w: Workload) -> torch.Tensor:
    """int32 [B] on the CPU."""
    if isinstance(w.ctx, int):
        return torch.full((w.B,), w.ctx, dtype=torch.int32)
    lo, hi = w.ctx
    g = generator(w, "ctx", 0, "cpu")
    return torch.randint(lo, hi + 1, (w.B,), generator=g, dtype=torch.int32)


def fetch_cap_fraction(w: Workload) -> Optional[float]:
    return w.cap


def _qbase(w: Workload, device) -> torch.Tensor:
    """fp32 [B][J][H_q][D]: the N(0,1) part of the lookahead queries."""
    out = torch.empty((w.B, w.J, w.H_q, w.D), dtype=torch.float32, device=device)
    for r in range(w.B):
        out[r] = _randn((w.J, w.H_q, w.D), generator(w, "qbase", r, device), device)
    return out


def _drift_frame(w: Workload, r: int, device):
    """Per KV head of request r: orthonormal (a, b) [H_kv][D] and a start angle."""
    g = generator(w, "drift", r, device)
    a = _randn((w.H_kv, w.D), g, device)
    b = _randn((w.H_kv, w.D), g, device)
    a = a / a.norm(dim=1, keepdim=True)
    b = b - (b * a).sum(dim=1, keepdim=True) * a
    b = b / b.norm(dim=1, keepdim=True)
    theta0 = torch.rand((w.H_kv,), generator=g, device=device) * (2 * math.pi)
    return a, b, theta0


def _drift_step_angle(w: Workload, n_b: int) -> float:
    # turning by this angle moves a K_b-wide arc of the block circle by
    # drift * K_b blocks
    return 2 * math.pi * w.drift * min(w.K_b, n_b) / n_b


def lookahead_f32(w: Workload, step: int, device="cpu") -> torch.Tensor:
    """fp32 [B][J][H_q][D] lookahead queries of decode step `step` (before the
    bf16 rounding)."""
    q = _qbase(w, device)
    if w.structure == "drift":
        ctx = context_lengths(w)
        for r in range(w.B):
            n_b = -(-int(ctx[r]) // w.bs)
            a, b, th0 = _drift_frame(w, r, device)
            th = th0 + step * _drift_step_angle(w, n_b)                      # [H_kv]
            d = w.drift_amp * (torch.cos(th)[:, None] * a + torch.sin(th)[:, None] * b)
            q[r] += d.repeat_interleave(w.G, dim=0)[None, :, :]
    elif step != 0:
        # stationary structures: later steps redraw a small perturbation so
        # that every step's input differs
        for r in range(w.B):
            q[r] += _randn((w.J, w.H_q, w.D), generator(w, "qstep", r * 65536 + step, device),
                           device, 0.05)
    return q


def lookahead(w: Workload, step: int = 0, device="cpu") -> torch.Tensor:
    """bf16 [B][J][H_q][D] lookahead (draft) queries for decode step `step`."""
    return lookahead_f32(w, step, device).to(torch.bfloat16)


def attention_query(w: Workload, step: int = 0, device="cpu") -> torch.Tensor:
    """bf16 [B][H_q][D].  The pages predict one step ahead; the synthetic
    drafter is taken as exact, so the query attended at step s is the first
    lookahead query drawn at step s - 1 (at step 0, that of step 0)."""
    return lookahead(w, max(step - 1, 0), device)[:, 0].contiguous()


def true_next_query(w: Workload, step: int, sigma: float, device="cpu") -> torch.Tensor:
    """bf16 [B][H_q][D]: the query the next token really has, for the
    lookahead-agreement analogue: the first draft of `step` plus seeded
    N(0, sigma^2) noise per coordinate (the draft queries are N(0, 1) plus
    the workload's structure), so sigma = 0 is a perfect drafter."""
    q = lookahead_f32(w, step, device)[:, 0]
    if sigma > 0:
        g = generator(w, "truenext", step, device)
        q = q + _randn(tuple(q.shape), g, device, sigma)
    return q.to(torch.bfloat16).contiguous()


def _qbar(w: Workload, device) -> torch.Tensor:
    """fp32 [B][H_kv][D]: mean over drafts and the group's query heads of the
    step-0 lookahead queries (after bf16 rounding)."""
    q = lookahead(w, 0, device).float()                                    # [B][J][H_q][D]
    return q.view(w.B, w.J, w.H_kv, w.G, w.D).mean(dim=(1, 3))


def _plant_picks(w: Workload, n_b: int, gp: torch.Generator, device):
    return [torch.randperm(n_b, generator=gp, device=device)[: w.planted] for _ in range(w.H_kv)]


def planted_blocks(w: Workload):
    """The planted block ids of a "planted" workload: list over requests of
    lists over KV heads of sorted int lists (CPU draws, matching kv_pool on
    the CPU)."""
    ctx = context_lengths(w)
    out = []
    for r in range(w.B):
        n_b = -(-int(ctx[r]) // w.bs)
        gp = generator(w, "plant", r, "cpu")
        out.append([sorted(p.tolist()) for p in _plant_picks(w, n_b, gp, "cpu")])
    return out


def kv_pool(w: Workload, device="cpu", out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """bf16 [B][H_kv][NB_max][2][bs][D] paged K/V pool with the workload's
    planted structure.  Positions at or past a request's context hold
    PAD_VALUE.  If `out` is given (any device, e.g. pinned host memory) the
    pool is generated request by request on `device` and copied into it."""
    ctx = context_lengths(w)
    NB, bs, D = w.NB_max, w.bs, w.D
    shape = (w.B, w.H_kv, NB, 2, bs, D)
    if out is None:
        out = torch.empty(shape, dtype=torch.bfloat16, device=device)
    assert tuple(out.shape) == shape and out.dtype == torch.bfloat16
    qbar = _qbar(w, device) if w.structure in ("planted", "zipf") else None
    tok = torch.arange(NB * bs, device=device).view(NB, bs)
    for r in range(w.B):
        n_ctx = int(ctx[r])
        n_b = -(-n_ctx // bs)
        kv = _randn((w.H_kv, NB, 2, bs, D), generator(w, "kv", r, device), device)
        k = kv[:, :, 0]                                                     # [H_kv][NB][bs][D]
        gp = generator(w, "plant", r, device)
        if w.structure == "planted" and w.planted > 0:
            for h, pick in enumerate(_plant_picks(w, n_b, gp, device)):
                k[h, pick] += 2.0 * qbar[r, h]
        elif w.structure == "zipf":
            for h in range(w.H_kv):
                rank = torch.randperm(n_b, generator=gp, device=device).float() + 1.0
                k[h, :n_b] += (2.0 * rank.pow(-w.zipf_s))[:, None, None] * qbar[r, h]
        elif w.structure == "drift":
            a, b, _ = _drift_frame(w, r, device)
            for h in range(w.H_kv):
                perm = torch.randperm(n_b, generator=gp, device=device).float()
                phi = 2 * math.pi * perm / n_b                              # [n_b]
                shift = w.drift_amp * (torch.cos(phi)[:, None] * a[h] + torch.sin(phi)[:, None] * b[h])
                k[h, :n_b] += shift[:, None, :]
        pad = (tok >= n_ctx)                                                # [NB][bs]
        kv.masked_fill_(pad[None, :, None, :, None], PAD_VALUE)
        out[r].copy_(kv.to(torch.bfloat16))
    return out


# ---------------------------------------------------------------------------
# stand-alone inputs for single-call unit tests


def random_scores(w: Workload, tie_levels: int = 0, device="cpu") -> torch.Tensor:
    """fp32 [B][H_kv][NB_max].  With tie_levels > 0 the values are drawn from
    that many distinct levels, so equal scores are common."""
    g = generator(w, "scores", 0, device)
    if tie_levels > 0:
        s = torch.randint(0, tie_levels, (w.B, w.H_kv, w.NB_max), generator=g, device=device)
        return (s.float() - tie_levels / 2) * 0.25
    return _randn((w.B, w.H_kv, w.NB_max), g, device, 100.0)


def predicted_set_sequence(w: Workload, steps: int, turnover: int, seed_index: int = 0):
    """A sequence of predicted sets for the staging rule, per (r, h): a list
    over steps of int32 [B][H_kv][K_b] (ascending ids, -1 padded) and n_sel
    [B][H_kv], plus fp32 scores [steps][B][H_kv][NB_max].  Each step replaces
    `turnover` members of the previous set with random non-members.  All on
    the CPU."""
    g = generator(w, "sets", seed_index, "cpu")
    ctx = context_lengths(w)
    K = w.K_b
    sels, nsels, scores = [], [], []
    cur = []
    for r in range(w.B):
        n_b = -(-int(ctx[r]) // w.bs)
        row = []
        for h in range(w.H_kv):
            k = min(K, n_b)
            row.append(torch.randperm(n_b, generator=g)[:k].tolist())
        cur.append(row)
    for s in range(steps):
        sel = torch.full((w.B, w.H_kv, K), -1, dtype=torch.int32)
        ns = torch.zeros((w.B, w.H_kv), dtype=torch.int32)
        for r in range(w.B):
            n_b = -(-int(ctx[r]) // w.bs)
            for h in range(w.H_kv):
                members = cur[r][h]
                if s > 0 and turnover > 0 and len(members) < n_b:
                    outside = [b for b in torch.randperm(n_b, generator=g).tolist()
                               if b not in set(members)]
                    t = min(turnover, len(outside), len(members))
                    drop = set(torch.randperm(len(members), generator=g)[:t].tolist())
                    members = [m for i, m in enumerate(members) if i not in drop] + outside[:t]
                    cur[r][h] = members
                srt = sorted(members)
                sel[r, h, : len(srt)] = torch.tensor(srt, dtype=torch.int32)
                ns[r, h] = len(srt)
        sc = torch.randn((w.B, w.H_kv, w.NB_max), generator=g) * 100.0
        # a few exact ties among the scores
        sc = torch.round(sc * 4) / 4
        sels.append(sel)
        nsels.append(ns)
        scores.append(sc)
    return sels, nsels, torch.stack(scores)


def random_table(w: Workload, n_entries: int, device="cpu", seed_index: int = 0):
    """A random resident set per (r, h): int32 block ids [B][H_kv][T] (T =
    n_entries, -1 padded, unordered) and counts [B][H_kv]; each row holds
    min(n_entries, n_b) distinct blocks, the request's last block always
    included when it is partial."""
    g = generator(w, "table", seed_index, "cpu")
    ctx = context_lengths(w)
    T = n_entries
    tbl = torch.full((w.B, w.H_kv, T), -1, dtype=torch.int32)
    n = torch.zeros((w.B, w.H_kv), dtype=torch.int32)
    for r in range(w.B):
        n_ctx = int(ctx[r])
        n_b = -(-n_ctx // w.bs)
        for h in range(w.H_kv):
            k = min(T, n_b)
            pick = torch.randperm(n_b, generator=g)[:k]
            if n_ctx % w.bs and not bool((pick == n_b - 1).any()) and k > 0:
                pick[0] = n_b - 1
            tbl[r, h, :k] = pick.to(torch.int32)
            n[r, h] = k
    return tbl.to(device), n.to(device)
