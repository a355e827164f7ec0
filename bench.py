#!/usr/bin/env python3
"""Decode-layer benchmark of the lookahead block-scoring path on one MI355X.

One step = one decode layer-step of the whole path over the batch: block
scores from the lookahead queries, top-K under the KV budget, staging of the
newly selected blocks (fetch-capped, from the pinned host pool into the HBM
working set) and sparse GQA decode attention over the working set.  Staging of
step s overlaps the attention of step s; the attention of step s + 1 waits only
for that staging (the per-layer ordering of the OasisKV pages, arXiv
2608.08097, paperlayer summary, section 4).

The default workload is the Qwen3-8B-shaped layer (32 query / 8 KV heads,
head dim 128, 16-token blocks) at batch 128 and 16K context, 2048-token budget,
fetch cap 0.05, K/V pool in pinned host memory.  Inputs are seeded synthetic
data (workloads.py), generated on the GPU and resident before timing.

Prints one JSON line: tokens/s per layer-step (whole job), the attention
kernel's HBM roofline (algorithmic bytes / measured launch time), the staging
traffic against the PCIe link, and the CPU oracle timed on the host cores.
"""
import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "sparse decode tokens/s per layer-step at 16K ctx, batch 128; HBM GB/s % peak"
HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, vendor figure
PCIE_PEAK_GBS = 64.0         # PCIe Gen5 x16, nominal per direction


def parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=64)
    p.add_argument("--warmup", type=int, default=4)
    p.add_argument("--workload", default="qwen3_8b_16k_b128_staged")
    p.add_argument("--copy-mode", choices=["kernel", "dma"], default="kernel")
    p.add_argument("--same-stream-copies", action="store_true",
                   help="run staging copies on the compute stream instead of a copy stream")
    p.add_argument("--n-split", type=int, default=0)
    p.add_argument("--cpu-seconds", type=float, default=10.0,
                   help="approximate CPU time budget of the oracle baseline")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--check", action="store_true",
                   help="after timing, compare sampled requests of the last step against the oracle")
    return p.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print(f"bench.py: this build measures one GPU only (asked for --gpus {args.gpus}); "
              "the path shards by request and KV head with no exchange, see DESIGN.md", file=sys.stderr)
        sys.exit(2)

    import torch
    import prefetch_block_scoring_amd as oa
    import workloads as wl

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = wl.WORKLOADS[args.workload]
    B, H_q, H_kv, D, bs, K_b, NB = w.B, w.H_q, w.H_kv, w.D, w.bs, w.K_b, w.NB_max
    staged = w.staged
    C = oa.oasis_fetch_cap_blocks(w.cap, K_b) if staged else 0
    S = K_b + C
    copy_mode = oa.OASIS_COPY_DMA if args.copy_mode == "dma" else oa.OASIS_COPY_KERNEL
    total_steps = 1 + args.warmup + args.steps          # step 0 = initial fill
    t_setup = time.perf_counter()

    ctx_cpu = wl.context_lengths(w)
    ctx = ctx_cpu.to(dev)
    log(f"workload {w.name}: B={B} H_q={H_q} H_kv={H_kv} NB_max={NB} K_b={K_b} C={C} staged={staged}")
    if staged:
        pool = torch.empty((B, H_kv, NB, 2, bs, D), dtype=torch.bfloat16, pin_memory=True)
        wl.kv_pool(w, device=dev, out=pool)
    else:
        pool = wl.kv_pool(w, device=dev)
    summ = oa.oasis_build_summaries(pool, ctx)
    q_look = [wl.lookahead(w, s, dev) for s in range(total_steps)]
    q_attn = [q_look[max(s - 1, 0)][:, 0].contiguous() for s in range(total_steps)]
    torch.cuda.synchronize()
    log(f"inputs ready in {time.perf_counter() - t_setup:.1f}s")

    main_s = torch.cuda.current_stream()
    comp_s = torch.cuda.Stream()
    copy_s = None if (args.same_stream_copies or not staged) else torch.cuda.Stream()

    scores = torch.empty((B, H_kv, NB), dtype=torch.float32, device=dev)
    sel = [torch.empty((B, H_kv, K_b), dtype=torch.int32, device=dev) for _ in range(2)]
    n_sel = [torch.empty((B, H_kv), dtype=torch.int32, device=dev) for _ in range(2)]
    out = torch.empty((B, H_q, D), dtype=torch.bfloat16, device=dev)
    if staged:
        ws_pool = torch.empty((B, H_kv, S, 2, bs, D), dtype=torch.bfloat16, device=dev)
        slot_block = torch.full((B, H_kv, S), -1, dtype=torch.int32, device=dev)
        slot_stamp = torch.full_like(slot_block, -1)
        tbls = [(torch.empty((B, H_kv, K_b), dtype=torch.int32, device=dev),
                 torch.empty((B, H_kv, K_b), dtype=torch.int32, device=dev),
                 torch.zeros((B, H_kv), dtype=torch.int32, device=dev)) for _ in range(2)]
        # two plans: the copies of step s still read theirs while step s + 1 plans
        plans = [torch.empty(oa.oasis_stage_plan_bytes(B, H_kv, K_b) // 4, dtype=torch.int32, device=dev)
                 for _ in range(2)]
        host_plan = torch.empty(plans[0].numel(), dtype=torch.int32).pin_memory() if copy_mode else None
        admitted = torch.zeros((), dtype=torch.int64, device=dev)
        T, P = K_b, S
        attn_pool = ws_pool
    else:
        T, P = K_b, NB
        attn_pool = pool
    splits = oa.oasis_attn_num_splits(B, H_q, H_kv, T, args.n_split)
    ws_bytes = oa.oasis_attn_workspace_bytes(B, H_q, H_kv, T, args.n_split)
    attn_ws = torch.empty((max(ws_bytes, 1),), dtype=torch.uint8, device=dev)

    def ev(timing=False):
        return torch.cuda.Event(enable_timing=timing)

    attn_done = [ev() for _ in range(total_steps)]
    stage_done = [ev() for _ in range(total_steps)]
    sel_done = [ev() for _ in range(total_steps)]
    timers = {k: [] for k in ("attn", "score", "topk", "stage")}

    def timed(name, stream, fn, on):
        if not on:
            fn()
            return
        a, b = ev(True), ev(True)
        a.record(stream)
        fn()
        b.record(stream)
        timers[name].append((a, b))

    def attend(s, on):
        if staged:
            t = tbls[s % 2]
            main_s.wait_event(stage_done[s - 1])
            timed("attn", main_s, lambda: oa.oasis_sparse_decode_attn(
                q_attn[s], attn_pool, t[0], t[1], t[2], ctx, out=out, ws=attn_ws, n_split=args.n_split,
                stream=main_s), on)
        else:
            j = (s - 1) % 2
            main_s.wait_event(sel_done[s - 1])
            timed("attn", main_s, lambda: oa.oasis_sparse_decode_attn(
                q_attn[s], attn_pool, sel[j], sel[j], n_sel[j], ctx, out=out, ws=attn_ws,
                n_split=args.n_split, stream=main_s), on)
        attn_done[s].record(main_s)

    def predict_and_stage(s, on):
        j = s % 2
        with torch.cuda.stream(comp_s):
            timed("score", comp_s, lambda: oa.oasis_score_blocks(q_look[s], summ, ctx, scores=scores,
                                                                 stream=comp_s), on)
            if s >= 2:
                # sel[j] / tables[(s+1)%2] were last read by the attention of step s-1
                comp_s.wait_event(attn_done[s - 1])
            timed("topk", comp_s, lambda: oa.oasis_select_topk(scores, ctx, K_b, sel=sel[j], n_sel=n_sel[j],
                                                               stream=comp_s), on)
            if staged:
                t = tbls[(s + 1) % 2]
                timed("stage", comp_s, lambda: oa.oasis_stage_blocks(
                    sel=sel[j], n_sel=n_sel[j], scores=scores, ctx_len=ctx, K_b=K_b,
                    C=K_b if s == 0 else C, step=s, slot_block=slot_block, slot_stamp=slot_stamp,
                    host_pool=pool, ws_pool=ws_pool, tbl_slot=t[0], tbl_block=t[1], tbl_n=t[2],
                    plan=plans[j], host_plan=host_plan, copy_mode=copy_mode, stream=comp_s,
                    copy_stream=copy_s, done_event=stage_done[s]), on)
                if on:
                    row = 2 + 2 * max(C, 1)
                    admitted.add_(plans[j][: B * H_kv * row].view(B * H_kv, row)[:, 0].sum())
            else:
                sel_done[s].record(comp_s)

    def step(s, on):
        if s >= 1:
            attend(s, on)        # enqueue first: a blocking DMA-mode stage must not delay it
        predict_and_stage(s, on)

    # initial fill (step 0) and warm-up
    for s in range(0, 1 + args.warmup):
        step(s, False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(1 + args.warmup, total_steps):
        step(s, True)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed / args.steps * 1e3
    value = B * args.steps / elapsed

    def avg_us(name):
        xs = timers[name]
        return sum(a.elapsed_time(b) for a, b in xs) / max(len(xs), 1) * 1e3

    # algorithmic bytes per launch
    if staged:
        tn = tbls[(total_steps - 1) % 2][2]
    else:
        tn = n_sel[(total_steps - 2) % 2]
    n_entries = int(tn.sum())
    attn_bytes = (n_entries * 2 * bs * D * 2 + 2 * B * H_q * D * 2 + B * H_kv * T * 8 + B * H_kv * 4 + B * 4)
    n_blocks_total = int(sum(-(-int(c) // bs) for c in ctx_cpu)) * H_kv
    score_bytes = n_blocks_total * 2 * D * 2 + B * H_kv * NB * 4 + q_look[0].numel() * 2 + B * 4
    topk_bytes = n_blocks_total * 4 + B * H_kv * (K_b + 1) * 4 + B * 4
    kern = {}
    for name, nbytes in (("attn", attn_bytes), ("score", score_bytes), ("topk", topk_bytes)):
        us = avg_us(name)
        kern[name] = {"avg_us": round(us, 2), "bytes": nbytes,
                      "GBps": round(nbytes / (us * 1e-6) / 1e9, 1) if us > 0 else None}
    h2d = None
    if staged:
        kern["stage"] = {"avg_us": round(avg_us("stage"), 2),
                         "note": "plan kernel" + (" and gather kernel" if copy_s is None and copy_mode == 0 else
                                                  "; copies run on the copy engine / copy stream")}
        adm = int(admitted) / args.steps
        h2d_bytes = adm * 2 * bs * D * 2
        # reference: one large pinned host -> device copy
        big = torch.empty(256 << 20, dtype=torch.uint8, pin_memory=True)
        dst = torch.empty_like(big, device=dev)
        dst.copy_(big, non_blocking=True)
        a, b = ev(True), ev(True)
        a.record()
        for _ in range(4):
            dst.copy_(big, non_blocking=True)
        b.record()
        torch.cuda.synchronize()
        memcpy_gbs = 4 * big.numel() / (a.elapsed_time(b) * 1e-3) / 1e9
        step_gbs = h2d_bytes / (ms_per_step * 1e-3) / 1e9
        h2d = {"bytes_per_step": int(h2d_bytes), "blocks_per_step": round(adm, 1),
               "GBps_over_step": round(step_gbs, 2), "pcie_nominal_GBps": PCIE_PEAK_GBS,
               "frac_of_nominal": round(step_gbs / PCIE_PEAK_GBS, 3),
               "pinned_memcpy_GBps": round(memcpy_gbs, 2),
               "frac_of_memcpy": round(step_gbs / memcpy_gbs, 3),
               "copy_engine": args.copy_mode, "drift_frac": round(adm / (B * H_kv) / K_b, 4)}
        del big, dst

    a_us = kern["attn"]["avg_us"]
    achieved = attn_bytes / (a_us * 1e-6) / 1e9
    roofline = {"kernel": "sparse_attn", "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                "bytes_per_launch": attn_bytes, "avg_launch_us": a_us}
    hbm_us = sum(kern[k]["avg_us"] for k in ("attn", "score", "topk"))
    hbm_bytes = attn_bytes + score_bytes + topk_bytes
    kern["hbm_kernels_total"] = {"avg_us": round(hbm_us, 2), "bytes": hbm_bytes,
                                 "GBps": round(hbm_bytes / (hbm_us * 1e-6) / 1e9, 1),
                                 "frac_of_peak": round(hbm_bytes / (hbm_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}

    if args.check:
        check_against_oracle(w, pool, ctx_cpu, q_look, q_attn, out, tbls if staged else None, total_steps)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, pool, ctx_cpu, q_look, args.cpu_seconds, C)

    line = {
        "metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": B, "context": w.ctx, "heads_q": H_q, "heads_kv": H_kv,
                   "head_dim": D, "block_tokens": bs, "kv_budget_tokens": w.budget, "lookahead_queries": w.J,
                   "fetch_cap": w.cap, "fetch_cap_blocks": C, "slots": S if staged else None,
                   "kv_location": "pinned host pool + HBM working set" if staged else "HBM",
                   "copy_engine": args.copy_mode if staged else None, "attn_splits": splits},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "h2d": h2d,
        "kernels": kern,
    }
    print(json.dumps(line), flush=True)


def cpu_baseline(w, pool, ctx_cpu, q_look, seconds, C):
    """The CPU oracle, unchanged, on the same inputs: full-batch decode
    layer-steps (score, select, staging bookkeeping, attention over the
    selected resident blocks read from the host pool) until about `seconds`
    of work are done."""
    import numpy as np
    import torch
    import oracle

    log("cpu baseline: building summaries (untimed)")
    kv_np = pool.view(torch.int16).cpu().numpy().view(np.uint16) if pool.is_cuda else \
        pool.view(torch.int16).numpy().view(np.uint16)
    ctx = ctx_cpu.numpy()
    summ = oracle.build_summaries(kv_np, ctx, w.bs)
    st = oracle.StageState(w.B, w.H_kv, w.NB_max)
    sm = 1.0 / math.sqrt(w.D)
    n_steps, t_total = 0, 0.0
    s = 0
    while True:
        ql = q_look[s % len(q_look)].cpu().view(torch.int16).numpy().view(np.uint16)
        qa = q_look[max(s - 1, 0) % len(q_look)][:, 0].contiguous().cpu().view(torch.int16).numpy().view(np.uint16)
        t0 = time.perf_counter()
        sc = oracle.score(ql, summ, ctx, w.bs, w.H_kv)
        sel, n = oracle.select(sc, ctx, w.bs, w.K_b)
        if w.staged:
            oracle.stage(st, sel, n, sc, ctx, w.bs, w.K_b, w.K_b if s == 0 else C, s)
            blocks = np.full((w.B, w.H_kv, w.K_b), -1, dtype=np.int32)
            nb = np.zeros((w.B, w.H_kv), dtype=np.int32)
            for r in range(w.B):
                for h in range(w.H_kv):
                    res = st.resident(r, h)
                    blocks[r, h, :len(res)] = res
                    nb[r, h] = len(res)
        else:
            blocks, nb = sel, n
        oracle.attend(qa, kv_np, ctx, blocks, nb, sm)
        dt = time.perf_counter() - t0
        n_steps += 1
        t_total += dt
        s += 1
        log(f"cpu baseline: step {n_steps} took {dt:.2f}s")
        if t_total >= seconds or n_steps >= 64:
            break
    return {"value": round(w.B * n_steps / t_total, 2), "unit": "tokens/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": f"{n_steps} full-batch layer-steps (B={w.B}) of score+select+"
                      f"{'stage bookkeeping+' if w.staged else ''}attend, fp64 C oracle, "
                      f"{t_total:.1f}s of CPU time",
            "cpu_model": _cpu_model()}


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def check_against_oracle(w, pool, ctx_cpu, q_look, q_attn, out, tbls, total_steps):
    """Sampled parity at full size: requests 0 and B-1 of the last step."""
    import numpy as np
    import torch
    import oracle
    log("check: comparing sampled requests against the oracle")
    s = total_steps - 1
    rs = sorted({0, w.B - 1})
    u16 = lambda t: t.contiguous().cpu().view(torch.int16).numpy().view(np.uint16)
    kv = u16(pool[rs])
    ctx = ctx_cpu.numpy()[rs]
    if tbls is not None:
        t = tbls[s % 2]
        blocks = t[1].cpu().numpy()[rs]
        n = t[2].cpu().numpy()[rs]
    else:
        raise SystemExit("--check covers staged workloads")
    ref, _ = oracle.attend(u16(q_attn[s][rs]), kv, ctx, blocks, n, 1 / math.sqrt(w.D))
    got = (u16(out[rs]).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    bad = np.abs(got - ref) > 2e-3 + 1e-2 * np.abs(ref)
    log(f"check: {bad.sum()} of {bad.size} outputs out of tolerance")
    if bad.any():
        raise SystemExit("check failed")


if __name__ == "__main__":
    main()
