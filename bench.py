#!/usr/bin/env python3
"""Decode-layer benchmark of the lookahead block-scoring path on one MI355X.

One layer-step = one pass of the whole path over the batch for one layer:
block scores from that layer's lookahead queries, top-K under the KV budget,
staging of the newly selected blocks (fetch-capped, from the pinned host pool
into the layer's HBM working set) and sparse GQA decode attention over the
working set.  OasisKV (arXiv 2608.08097, paperlayer summary, section 4) keeps
prediction, selection and copies off the attention's critical path with
several layers in flight; the benchmark keeps `--layers` layers in flight
(default 4): each decode step issues the layers in order, a layer's staging
overlaps the other layers' work, and its attention at the next step waits
only on its own copies.

Workload (default): the Qwen3-8B-shaped layer (32 query / 8 KV heads, head dim
128, 16-token blocks) at batch 128 and 16K context, 2048-token budget, fetch
cap 0.05, K/V pool in pinned host memory (one pool shared read-only by the
layers, each layer with its own working set, slot table and lookahead phase).
Inputs are seeded synthetic data (workloads.py), generated on the GPU and
resident before timing.

Prints one JSON line: tokens/s per layer-step (whole job), the attention
kernel's HBM roofline (algorithmic bytes / measured launch time), the staging
traffic against the PCIe link, and the CPU oracle timed on the host cores.
"""
import argparse
import concurrent.futures
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
    p.add_argument("--steps", type=int, default=64, help="timed decode steps")
    p.add_argument("--warmup", type=int, default=4)
    p.add_argument("--layers", type=int, default=4, help="layers in flight")
    p.add_argument("--workload", default="qwen3_8b_16k_b128_staged")
    p.add_argument("--copy-mode", choices=["kernel", "dma", "mixed"], default="kernel")
    p.add_argument("--host-threads", type=int, default=8, help="packing threads of the DMA copy engine")
    p.add_argument("--n-split", type=int, default=0)
    p.add_argument("--compute-streams", type=int, default=0, choices=[-1, 0, 1, 2],
                   help="streams for scores, top-K and plan (0 = the library's automatic choice, "
                        "-1 = the main stream, after each layer's attention)")
    p.add_argument("--issue-threads", type=int, default=0, choices=[-1, 0, 1],
                   help="worker threads that enqueue each layer-step's chain and copies (0 = the library's "
                        "automatic choice, 1 = on, -1 = off: the calling thread enqueues everything)")
    p.add_argument("--joint", action="store_true",
                   help="look-ahead attention: the normal query and the step's J draft queries attend together")
    p.add_argument("--attn-sweep", action="store_true",
                   help="also time look-ahead attention alone for every supported number of queries per request")
    p.add_argument("--agreement", action="store_true",
                   help="instead of the throughput run: the lookahead-agreement analogue (top-K overlap of the "
                        "draft-based selection with the next query's exact attention top-K, against drafting noise)")
    p.add_argument("--kernel-timing", default="attn", choices=["all", "attn"],
                   help="launches of the timed steps that get timing events (a start event recorded on the "
                        "stream, which holds it ~3 us, and a stop event bound to the last kernel); the others "
                        "are timed in an extra pass afterwards")
    p.add_argument("--timing-every", type=int, default=1,
                   help="time one launch in every N of each timed kind during the timed steps (a timed launch's "
                        "start event holds its queue ~3 us)")
    p.add_argument("--cap", type=float, default=None,
                   help="override the staged workload's fetch cap (fraction of the budget; >= 1 = fetch-all)")
    p.add_argument("--drift", type=float, default=None,
                   help="override the drift workload's per-step turnover (fraction of the budget)")
    p.add_argument("--cpu-seconds", type=float, default=10.0,
                   help="approximate CPU time budget of the oracle baseline")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--check", action="store_true",
                   help="after timing, compare sampled requests of the last step against the oracle")
    p.add_argument("--summarize-profile", nargs="+", metavar="DIR",
                   help="summarize rocprofv3 CSV output directories (kernel stats, FETCH_SIZE and "
                        "WRITE_SIZE runs) instead of benchmarking")
    p.add_argument("--command", default="", help="with --summarize-profile: the profiled command line")
    p.add_argument("--bench-log", default=None,
                   help="with --summarize-profile: the profiled bench run's output (stderr and the JSON line); "
                        "splits the attention launches of the kernel trace by phase")
    return p.parse_args()


def percentiles(values):
    """p10 / p50 / p90 of a list of microsecond figures (linear
    interpolation between order statistics)."""
    if not values:
        return {}
    import numpy as np
    p10, p50, p90 = np.percentile(np.asarray(values, dtype=np.float64), [10, 50, 90])
    return {"p10_us": round(float(p10), 2), "p50_us": round(float(p50), 2), "p90_us": round(float(p90), 2),
            "n": len(values)}


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


ROTATION_BYTES = 1 << 30     # bytes a rotation of alone launches cycles through


def rotation_count(nbytes, most=64):
    """Input copies for launches timed alone: at least three, and enough that
    one round through them reads ROTATION_BYTES (four times the 256 MB
    Infinity Cache), so a launch never re-reads what the last ones cached."""
    return int(min(most, max(3, -(-ROTATION_BYTES // max(int(nbytes), 1)))))


def time_rotated(torch, fns, n, label=None):
    """Mean microseconds per launch of n launches cycling through fns (one
    launch per input copy), after one untimed round.  The launches run back
    to back on the GPU: before the first, the stream is kept busy with fills
    of a scratch buffer for longer than the host takes to enqueue all n, so
    the figure is the kernels' own time and not the binding's per-call host
    cost (which exceeds a 30 us kernel's).  A measurement in which the host
    had not enqueued the last launch by the time the GPU finished the fills
    (a pause of the host thread, seen up to ~36 ms) is taken again, up to
    three times.  With a label, the number of launches made (untimed rounds
    and every attempt) is logged, so that a kernel trace can be split."""
    import gc
    for f in fns:
        f()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for f in fns:
        f()
    host_s = (time.perf_counter() - t0) / len(fns)
    torch.cuda.synchronize()
    hold = torch.empty(64 << 20, dtype=torch.int32, device="cuda")  # 256 MiB: one fill takes ~40 us
    n_fill = int(math.ceil((2.0 * n * host_s + 500e-6) / 40e-6))
    h, a, b = (torch.cuda.Event(enable_timing=True) for _ in range(3))
    made = 2 * len(fns)
    for attempt in range(3):
        gc_on = gc.isenabled()
        gc.disable()
        t0 = time.perf_counter()
        h.record()
        for _ in range(n_fill):
            hold.fill_(1)
        a.record()
        for i in range(n):
            fns[i % len(fns)]()
        enqueue_ms = (time.perf_counter() - t0) * 1e3
        made += n
        b.record()
        if gc_on:
            gc.enable()
        torch.cuda.synchronize()
        if enqueue_ms < h.elapsed_time(a):
            break
        log(f"alone launches: the host fell behind the GPU (enqueue {enqueue_ms:.2f} ms, fills "
            f"{h.elapsed_time(a):.2f} ms); measuring again")
    del hold
    if label:
        log(f"{label} alone launches made: {made}")
    return a.elapsed_time(b) / n * 1e3


def alone_entry(nbytes, us, n_rot, how):
    gbs = nbytes / (us * 1e-6) / 1e9
    return {"avg_us": round(us, 2), "bytes": int(nbytes), "GBps": round(gbs, 1),
            "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4), "rotation": n_rot,
            "note": f"alone on the GPU after the timed steps; consecutive launches cycle through {n_rot} {how}"}


def numa_placement(host_tensor, samples=256):
    """NUMA node of the GPU (sysfs, from its PCI address) and the nodes that
    hold a sample of a pinned host buffer's pages (move_pages with no target
    nodes reports where each page lives)."""
    import ctypes
    import torch
    out = {"gpu_node": None, "pool_pages": None}
    try:
        p = torch.cuda.get_device_properties(torch.cuda.current_device())
        addr = f"{p.pci_domain_id:04x}:{p.pci_bus_id:02x}:{p.pci_device_id:02x}.0"
        with open(f"/sys/bus/pci/devices/{addr}/numa_node") as f:
            out["gpu_node"] = int(f.read().strip())
        out["gpu_pci"] = addr
    except (AttributeError, OSError, ValueError):
        pass
    try:
        libc = ctypes.CDLL(None, use_errno=True)
        page = os.sysconf("SC_PAGE_SIZE")
        base = host_tensor.data_ptr()
        nbytes = host_tensor.numel() * host_tensor.element_size()
        step = max(page, (nbytes // samples) // page * page)
        addrs = [(base + i * step) // page * page for i in range(samples) if i * step < nbytes]
        pages = (ctypes.c_void_p * len(addrs))(*addrs)
        status = (ctypes.c_int * len(addrs))()
        SYS_move_pages = 279  # x86_64
        rc = libc.syscall(SYS_move_pages, 0, ctypes.c_ulong(len(addrs)), pages, None, status, 0)
        if rc == 0:
            counts = {}
            for v in status:
                key = str(v) if v >= 0 else f"err{-v}"
                counts[key] = counts.get(key, 0) + 1
            out["pool_pages"] = counts
        else:
            out["pool_pages"] = f"move_pages errno {ctypes.get_errno()}"
    except (OSError, AttributeError) as e:
        out["pool_pages"] = f"unavailable: {e}"
    return out


KERNEL_SOURCES = {"attn_kernel": "attn.hip", "score_kernel": "score.hip", "topk_kernel": "topk.hip",
                  "stage_gather_kernel": "stage.hip", "stage_plan_kernel": "stage.hip"}
CALIB_BYTES = 256 << 20
READ_REF_BYTES = 512 << 20


def _source_hash(name):
    import hashlib
    path = os.path.join(ROOT, "prefetch_block_scoring_amd", "csrc", name)
    return hashlib.sha256(open(path, "rb").read()).hexdigest()[:16]


def _short(name):
    import re
    m = re.search(r"oasis::\(anonymous namespace\)::([A-Za-z_0-9]+(<[^>]*>)?)", name)
    if m:
        return m.group(1)
    return name.split("(")[0][-60:]


def _attention_phases(trace_path, bench_log):
    """Mean duration of the attention launches of each bench phase, from a
    rocprofv3 kernel trace and the bench run's log (its launch counts per
    phase and its JSON line); the attention kernel runs once per layer-step
    and once per alone launch, in that order."""
    import csv
    phases, line = None, None
    for ln in open(bench_log):
        if "attention launches: " in ln:
            phases = json.loads(ln.split("attention launches: ", 1)[1])
        elif "attention alone launches made: " in ln and phases is not None:
            # the alone leg measured again (a host that fell behind the GPU)
            phases["alone"] = int(ln.split("attention alone launches made: ", 1)[1])
        elif ln.startswith("{"):
            line = json.loads(ln)
    if phases is None:
        return []
    all_rows = list(csv.DictReader(open(trace_path)))
    by_start = lambda r: int(r["Start_Timestamp"])
    rows = sorted((r for r in all_rows if "attn_kernel" in r["Kernel_Name"]), key=by_start)
    comb = sorted((r for r in all_rows if "attn_combine_kernel" in r["Kernel_Name"]), key=by_start)
    dur = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in rows]
    out = [f"attention launches by bench phase ({os.path.basename(trace_path)}, {len(dur)} launches):"]
    expect = sum(phases.values())
    if len(dur) != expect:
        out.append(f"  launch count {len(dur)} differs from the bench's {expect}: not split")
        return out
    # with split-K, each launch is the attention kernel and then its combine
    # kernel; the HIP events bracket both, so the span (attention start to
    # combine end) is what they compare with
    span = None
    if comb and len(comb) == len(rows):
        out.append("  each launch: attention kernel + combine kernel (split-K); span = attention start to "
                   "combine end")
        span = [(int(c["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r, c in zip(rows, comb)]
    i = 0
    res = {}
    for name in ("warmup", "timed", "extra", "alone"):
        n = phases[name]
        if n:
            seg = dur[i:i + n]
            res[name] = sum(seg) / n
            txt = f"  {name:7s} {n:5d} launches  mean {res[name]:9.2f} us  min {min(seg):9.2f}  max {max(seg):9.2f}"
            if span:
                res[name] = sum(span[i:i + n]) / n
                txt += f"  span mean {res[name]:9.2f} us"
            out.append(txt)
        i += n
    if line and "timed" in res:
        b = line["roofline"]["avg_launch_us"]
        out.append(f"  bench line (HIP events on the attention's stream, timed steps): {b:.2f} us; "
                   f"trace {'span' if span else 'mean'} / events = {res['timed'] / b:.3f}")
    return out


RDREQ_SIZES = (("TCC_EA0_RDREQ_32B_sum", 32), ("TCC_EA0_RDREQ_64B_sum", 64), ("TCC_EA0_RDREQ_128B_sum", 128))


def request_bytes(vals):
    """HBM bytes of one dispatch from the L2's request counters: read
    requests by size (32, 64 and 128 bytes), write requests as 64 bytes
    (TCC_EA0_WRREQ_64B) or 32 bytes (the rest); None for a side not
    counted."""
    rd = None
    if all(k in vals for k, _ in RDREQ_SIZES):
        rd = sum(vals[k] * n for k, n in RDREQ_SIZES)
    wr = None
    if "TCC_EA0_WRREQ_sum" in vals and "TCC_EA0_WRREQ_64B_sum" in vals:
        w64 = vals["TCC_EA0_WRREQ_64B_sum"]
        wr = 64 * w64 + 32 * (vals["TCC_EA0_WRREQ_sum"] - w64)
    return rd, wr


def _derived(v):
    """Ratios of one dispatch's counters that need no clock or unit count:
    the L2 hit fraction, and the shares of the waves' lifetime spent waiting
    on an outstanding access (SQ_WAIT_INST_ANY) and issuing vector ALU work
    (SQ_ACTIVE_INST_VALU), both counted in the same 4-cycle units as
    SQ_WAVE_CYCLES."""
    parts = []
    if "TCC_HIT_sum" in v and "TCC_MISS_sum" in v and v["TCC_HIT_sum"] + v["TCC_MISS_sum"] > 0:
        parts.append(f"L2 hit {v['TCC_HIT_sum'] / (v['TCC_HIT_sum'] + v['TCC_MISS_sum']):.3f}")
    if v.get("SQ_WAVE_CYCLES"):
        for c, label in (("SQ_WAIT_INST_ANY", "waiting"), ("SQ_ACTIVE_INST_VALU", "issuing VALU")):
            if c in v:
                parts.append(f"{label} {v[c] / v['SQ_WAVE_CYCLES']:.3f} of wave time")
    if "OccupancyPercent" in v:
        parts.append(f"occupancy {v['OccupancyPercent']:.1f}% of 32 waves per CU")
    return ("  [" + ", ".join(parts) + "]") if parts else ""


def _raw_counters(rows, fname, machine):
    """Counters other than FETCH_SIZE / WRITE_SIZE, per dispatch of each of
    the library's kernels and of the plain copy / reduction kernels, in
    dispatch order; read and write request counters also as bytes
    (request_bytes), and per kernel the mean over its dispatches."""
    out = [f"counters ({fname}), the first three dispatches of each of the library's kernels and of "
           f"the plain copy / reduction kernels' large dispatches (the calibration copy, the read "
           f"reference), then the mean over all of them:"]
    per = {}
    lib = set()  # short names of the library's kernels
    for r in rows:
        name = r["Kernel_Name"]
        if "oasis" not in name and "copy" not in name.lower() and "reduce" not in name.lower():
            continue
        key = (_short(name), int(r["Dispatch_Id"]))
        if "oasis" in name:
            lib.add(key[0])
        per.setdefault(key, {})[r["Counter_Name"]] = float(r["Counter_Value"])
    for key in [k for k in per if k[0] not in lib]:
        v = per[key]
        rd, wr = request_bytes(v)
        # a large transfer by whichever counter this pass holds: bytes, L2
        # misses (128 B lines), or a long-lived grid
        big = ((rd or 0) >= 100e6 or (wr or 0) >= 100e6 or v.get("TCC_MISS_sum", 0) >= 1e6
               or v.get("SQ_WAVE_CYCLES", 0) >= 1e7)
        if not big:
            del per[key]
    means = {}
    shown = {}
    for (k, disp), vals in sorted(per.items(), key=lambda kv: kv[0][1]):
        for c, v in vals.items():
            means.setdefault(k, {}).setdefault(c, []).append(v)
        shown[k] = shown.get(k, 0) + 1
        if shown[k] > 3:  # the first three dispatches of each kernel; all of them enter the mean
            continue
        txt = "  ".join(f"{c} {v:.0f}" for c, v in sorted(vals.items()))
        rd, wr = request_bytes(vals)
        if rd is not None:
            txt += f"  -> read {rd / 1e6:.2f} MB"
        if wr is not None:
            txt += f"  -> written {wr / 1e6:.2f} MB"
        out.append(f"  {k[:40]:40s} dispatch {disp:6d}  {txt}")
    out.append("  mean per dispatch:")
    for k, cs in means.items():
        avg = {c: sum(v) / len(v) for c, v in cs.items()}
        rd, wr = request_bytes(avg)
        txt = "  ".join(f"{c} {v:.0f}" for c, v in sorted(avg.items()))
        out.append(f"  {k[:40]:40s} ({len(next(iter(cs.values())))} dispatches)  {txt}"
                   + (f"  -> read {rd / 1e6:.2f} MB" if rd is not None else "")
                   + (f"  -> written {wr / 1e6:.2f} MB" if wr is not None else "")
                   + _derived(avg))
        if k in lib:
            m = machine.setdefault(k, {})
            if rd is not None:
                m["read_bytes"] = rd
            if wr is not None:
                m["write_bytes"] = wr
    return out


def summarize_profile(dirs, command, bench_log=None):
    """Reduce rocprofv3 CSV output to a short text summary: per-kernel call
    counts and durations, and, from FETCH_SIZE / WRITE_SIZE runs, HBM bytes
    per dispatch scaled by what the same counters read for the plain
    CALIB_BYTES device copy that bench.py runs after its timed steps."""
    import csv
    import glob
    import statistics
    out = [f"command: {command}"] if command else []
    machine = {}
    for d in dirs:
        for path in sorted(glob.glob(os.path.join(d, "**", "*kernel_stats.csv"), recursive=True)):
            rows = list(csv.DictReader(open(path)))
            out.append(f"kernel stats ({os.path.basename(path)}):")
            out.append(f"  {'kernel':40s} {'calls':>6s} {'avg_us':>10s} {'min_us':>10s} {'max_us':>10s}")
            for r in rows:
                n = _short(r["Name"])
                if "oasis" not in r["Name"] and float(r.get("Percentage", 0) or 0) < 1.0:
                    continue
                out.append(f"  {n:40s} {r['Calls']:>6s} {float(r['AverageNs']) / 1e3:10.2f} "
                           f"{float(r['MinNs']) / 1e3:10.2f} {float(r['MaxNs']) / 1e3:10.2f}")
                if "oasis" in r["Name"]:
                    machine.setdefault(_short(r["Name"]), {})["avg_us"] = float(r["AverageNs"]) / 1e3
        if bench_log:
            for path in sorted(glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True)):
                out.extend(_attention_phases(path, bench_log))
        for path in sorted(glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)):
            rows = list(csv.DictReader(open(path)))
            if not rows:
                continue
            counters = sorted({r["Counter_Name"] for r in rows})
            if counters not in (["FETCH_SIZE"], ["WRITE_SIZE"]):
                out.extend(_raw_counters(rows, os.path.basename(path), machine))
                continue
            counter = counters[0]
            per = {}
            for r in rows:
                per.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
            copies = [(max(v), k) for k, v in per.items() if "copy" in k.lower()]
            calib_kib = max(copies)[0] if copies else None
            factor = calib_kib / (CALIB_BYTES / 1024) if calib_kib else None
            out.append(f"{counter} ({os.path.basename(path)}): calibration copy of {CALIB_BYTES >> 20} MiB reads "
                       f"{calib_kib} KiB -> scale {factor}")
            for k, v in per.items():
                if "oasis" not in k:
                    continue
                kib = statistics.mean(v)
                byt = kib * 1024 / factor if factor else None
                out.append(f"  {_short(k):40s} dispatches {len(v):4d} mean {kib:12.1f} KiB -> "
                           f"{byt / 1e6 if byt else float('nan'):10.2f} MB per dispatch (calibrated)")
                machine.setdefault(_short(k), {})[counter] = byt
    if bench_log:
        for ln in open(bench_log):
            if ln.startswith("{"):
                h2d = json.loads(ln).get("h2d")
                if h2d:
                    out.append(f"bench line: admitted blocks per layer-step over the timed steps "
                               f"{h2d['blocks_per_layer_step']}, {h2d['bytes_per_layer_step'] / 1e6:.2f} MB")
    for k, v in machine.items():
        for src_key, fname in KERNEL_SOURCES.items():
            if k.endswith(src_key) or src_key in k:
                v["source"] = fname
                v["source_sha256_16"] = _source_hash(fname)
    out.append("machine-readable: " + json.dumps(machine, sort_keys=True))
    print("\n".join(out))


def profiled_traffic(kernel_key, profile_file):
    """HBM bytes per dispatch of a kernel (read plus written, from the L2's
    request-size counters) from a committed profile summary, or None when the
    summary is missing or the kernel's source has changed since the counters
    were taken."""
    path = os.path.join(ROOT, "profiles", profile_file)
    try:
        for line in open(path):
            if line.startswith("machine-readable: "):
                data = json.loads(line[len("machine-readable: "):])
                break
        else:
            return None
    except OSError:
        return None
    for k, v in data.items():
        if kernel_key in k and "read_bytes" in v and "write_bytes" in v:
            if v.get("source_sha256_16") != _source_hash(KERNEL_SOURCES[kernel_key]):
                return None
            return int(v["read_bytes"] + v["write_bytes"])
    return None


def main():
    args = parse()
    if args.summarize_profile:
        summarize_profile(args.summarize_profile, args.command, args.bench_log)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print(f"bench.py: measures one GPU only (asked for --gpus {args.gpus}); "
              "the path shards by request and KV head with no exchange between GPUs", file=sys.stderr)
        sys.exit(2)

    if args.agreement:
        agreement_run(args)
        return

    import torch
    import prefetch_block_scoring_amd as oa
    import workloads as wl

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = wl.WORKLOADS[args.workload]
    if args.cap is not None:
        if not w.staged:
            raise SystemExit(f"--cap: workload {w.name} keeps its K/V in HBM")
        w = w.shrink(cap=args.cap)
    if args.drift is not None:
        if w.structure != "drift":
            raise SystemExit(f"--drift: workload {w.name} has no drift structure")
        w = w.shrink(drift=args.drift)
    B, H_q, H_kv, D, bs, K_b, NB = w.B, w.H_q, w.H_kv, w.D, w.bs, w.K_b, w.NB_max
    staged = w.staged
    L = max(1, args.layers)
    C = oa.oasis_fetch_cap_blocks(w.cap, K_b) if staged else 0
    S = K_b + C
    copy_mode = {"kernel": oa.OASIS_COPY_KERNEL, "dma": oa.OASIS_COPY_DMA, "mixed": oa.OASIS_COPY_MIXED}[args.copy_mode]
    n_steps = 1 + args.warmup + args.steps              # step 0 = initial fill
    n_extra = min(args.steps, 16)                       # per-kernel timing pass after the timed steps
    n_total = n_steps + n_extra
    t_setup = time.perf_counter()

    ctx_cpu = wl.context_lengths(w)
    ctx = ctx_cpu.to(dev)
    log(f"workload {w.name}: B={B} H_q={H_q} H_kv={H_kv} NB_max={NB} K_b={K_b} C={C} staged={staged} "
        f"layers={L} copy={args.copy_mode}")
    if staged:
        pool = oa.oasis_host_empty((B, H_kv, NB, 2, bs, D), torch.bfloat16)
        wl.kv_pool(w, device=dev, out=pool)
    else:
        pool = wl.kv_pool(w, device=dev)
    summ = oa.oasis_build_summaries(pool, ctx)
    # layer l at step t uses the lookahead of drift step t + 3 l (its own phase)
    n_look = n_total + 3 * (L - 1)
    q_look = [wl.lookahead(w, s, dev) for s in range(n_look)]
    q_attn = [q_look[max(s - 1, 0)][:, 0].contiguous() for s in range(n_look)]
    n_q = 1 + w.J if args.joint else 1
    if n_q * (H_q // H_kv) > 16:
        raise SystemExit(f"--joint: {n_q} queries x {H_q // H_kv} heads per KV head = {n_q * (H_q // H_kv)} "
                         "columns; look-ahead attention supports at most 16")
    if args.joint:
        # the normal query, then the draft queries that score this step's blocks
        q_attn = [torch.cat([q_attn[s][:, None], q_look[s]], dim=1).contiguous() for s in range(n_look)]
    torch.cuda.synchronize()
    log(f"inputs ready in {time.perf_counter() - t_setup:.1f}s")

    from prefetch_block_scoring_amd.pipeline import LayerPipeline
    pipe = LayerPipeline(pool=pool, summ=summ, ctx=ctx, H_q=H_q, K_b=K_b, C=C, n_layers=L, staged=staged,
                         copy_mode=copy_mode, host_threads=args.host_threads, n_split=args.n_split, J=w.J,
                         n_q=n_q, compute_streams=args.compute_streams, issue_threads=args.issue_threads)
    T = K_b
    splits, attn_waves = oa.oasis_attn_launch_shape(B, H_q, H_kv, n_q, T, args.n_split)

    def run(t0, t1, step_events=None):
        for t in range(t0, t1):
            for l in range(L):
                s = t + 3 * l
                pipe.layer_step(l, t, q_look[s], q_attn[s])
            if step_events is not None:
                # the main stream passes the step's last attention
                ev = torch.cuda.Event(enable_timing=True)
                ev.record(pipe.main)
                step_events.append(ev)

    # initial fill (step 0) and warm-up
    run(0, 1 + args.warmup)
    pipe.drain()
    torch.cuda.synchronize()
    # the staging counters (admits, evictions, deferred admits, steps) that
    # the plan kernels add up on the device: cleared now, read after the
    # timed steps, so the H2D bytes are those of the timed steps themselves
    if staged:
        pipe.reset_stage_stats()
    # timing events around the attention launches of the timed steps, on
    # their own stream (the roofline's live figure); other kinds only with
    # --kernel-timing all
    all_kinds = ("attn", "score", "topk", "plan") if staged else ("attn", "score", "topk")
    timed_kinds = all_kinds if args.kernel_timing == "all" else ("attn",)
    every = max(1, args.timing_every)
    n_timed = -(-args.steps * L // every)
    pipe.enable_timing(n_timed, timed_kinds, every=every)
    step_events = []
    # Python's garbage collector stays off over the timed steps: a collection
    # pauses the issuing thread for tens of ms, which a caller in C++ would
    # not see
    import gc
    gc.collect()
    gc.disable()
    cpu0 = time.process_time()
    t0 = time.perf_counter()
    run(1 + args.warmup, n_steps, step_events=step_events)
    issued = time.perf_counter() - t0
    pipe.drain()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    gc.enable()
    host_cores = (time.process_time() - cpu0) / elapsed  # CPU time of all the process's threads / wall
    timed_stats = pipe.stage_stats() if staged else None
    layer_steps = args.steps * L
    ms_per_step = elapsed / layer_steps * 1e3
    value = B * layer_steps / elapsed

    def read_us(name, n_expect):
        us, n = pipe.timing(name)
        if n != n_expect:
            raise SystemExit(f"timing of {name}: {n} launches recorded, {n_expect} expected")
        return us

    live = {k: read_us(k, n_timed) for k in timed_kinds}
    live_note = "live, timed steps" + (f", one launch in {every}" if every > 1 else "")
    # distributions: each timed launch, and each decode step (intervals
    # between the main stream's passes of consecutive steps), per layer-step
    spread = {k: pipe.timing_values(k, n_timed) for k in timed_kinds}
    step_us = [step_events[i - 1].elapsed_time(step_events[i]) * 1e3 / L for i in range(1, len(step_events))]
    copy_s, copy_n = pipe.copy_host_seconds()
    # the kinds not timed above: an extra pass of n_extra steps with events on
    # every launch, after the timed steps
    extra = {}
    if len(timed_kinds) < len(all_kinds):
        pipe.enable_timing(n_extra * L, all_kinds)
        run(n_steps, n_total)
        pipe.drain()
        torch.cuda.synchronize()
        extra = {k: read_us(k, n_extra * L) for k in all_kinds if k not in timed_kinds}
        spread.update({k: pipe.timing_values(k, n_extra * L) for k in extra})
    t_last = n_total - 1

    def avg_us(name):
        return live[name] if name in live else extra[name]

    # algorithmic bytes per launch
    if staged:
        tn = pipe.table(0, t_last)[2]
    else:
        tn = pipe.layers[0].n_sel[(t_last - 1) % 2]
    n_entries = int(tn.sum())
    attn_bytes = (n_entries * 2 * bs * D * 2 + 2 * n_q * B * H_q * D * 2 + B * H_kv * T * 8 + B * H_kv * 4
                  + B * 4)
    n_blocks_total = int(sum(-(-int(c) // bs) for c in ctx_cpu)) * H_kv
    score_bytes = n_blocks_total * 2 * D * 2 + B * H_kv * NB * 4 + q_look[0].numel() * 2 + B * 4
    topk_bytes = n_blocks_total * 4 + B * H_kv * (K_b + 1) * 4 + B * 4
    kern = {}
    for name, nbytes in (("attn", attn_bytes), ("score", score_bytes), ("topk", topk_bytes)):
        us = avg_us(name)
        kern[name] = {"avg_us": round(us, 2), "bytes": nbytes,
                      "GBps": round(nbytes / (us * 1e-6) / 1e9, 1) if us > 0 else None,
                      "timed": live_note if name in live else f"extra pass of {n_extra} steps",
                      **percentiles(spread.get(name, []))}
    h2d = None
    if staged:
        kern["plan"] = {"avg_us": round(avg_us("plan"), 2), "note": "plan and prefix kernels",
                        "timed": live_note if "plan" in live else f"extra pass of {n_extra} steps",
                        **percentiles(spread.get("plan", []))}
        kern["copy_host"] = {"avg_us": round(copy_s / max(copy_n, 1) * 1e6, 2),
                              "note": ("host time of a staging call: plan read-back and packing up to the "
                                       "copy's enqueue") if copy_mode != oa.OASIS_COPY_KERNEL
                              else "host time of a staging call (enqueue only)"}
        if timed_stats["steps"] != args.steps * L:
            raise SystemExit(f"staging counters saw {timed_stats['steps']} steps, {args.steps * L} expected")
        adm = timed_stats["admits"] / (args.steps * L)
        h2d_bytes = adm * 2 * bs * D * 2
        # reference: one large pinned host -> device copy
        big = oa.oasis_host_empty((256 << 20,), torch.uint8)
        dst = torch.empty_like(big, device=dev)
        dst.copy_(big, non_blocking=True)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(4):
            dst.copy_(big, non_blocking=True)
        b.record()
        torch.cuda.synchronize()
        memcpy_gbs = 4 * big.numel() / (a.elapsed_time(b) * 1e-3) / 1e9
        step_gbs = h2d_bytes / (ms_per_step * 1e-3) / 1e9
        h2d = {"bytes_per_layer_step": int(h2d_bytes), "blocks_per_layer_step": round(adm, 1),
               "GBps": round(step_gbs, 2), "pcie_nominal_GBps": PCIE_PEAK_GBS,
               "frac_of_nominal": round(step_gbs / PCIE_PEAK_GBS, 3),
               "pinned_memcpy_GBps": round(memcpy_gbs, 2),
               "frac_of_memcpy": round(step_gbs / memcpy_gbs, 3),
               "copy_engine": args.copy_mode, "drift_frac": round(adm / (B * H_kv) / K_b, 4),
               "deferred_per_layer_step": round(timed_stats["deferred"] / (args.steps * L), 1),
               "evictions_per_layer_step": round(timed_stats["evictions"] / (args.steps * L), 1),
               "counted": f"device counters of the plan kernels over the {args.steps * L} timed layer-steps",
               "numa": numa_placement(pool)}
        del big, dst

    # The same launches alone on the GPU (nothing else in flight): each
    # kernel's own rate, beside its rate while sharing the GPU with the
    # pipeline above.  Consecutive launches read different copies of their
    # input (rotation), at least 1 GiB apart in total, so no launch finds its
    # bytes in the 256 MB Infinity Cache that the previous one filled.
    q4 = q_attn[t_last].view(B, n_q, H_q, D)
    out_alone = torch.empty_like(q4)
    attn_ws = pipe.layers[0].attn_ws
    if staged:
        tb = pipe.table(0, t_last)
        wsp = pipe.layers[0].ws_pool
        n_rot = rotation_count(attn_bytes)
        rot_inputs = [wsp] + [wsp.clone() for _ in range(n_rot - 1)]

        def attn_call(q_, p_, o_, w_):
            return oa.oasis_lookahead_attn(q_, p_, tb[0], tb[1], tb[2], ctx, out=o_, ws=w_, n_split=args.n_split)
        rot_how = "copies of the working set"
    else:
        jp = (t_last - 1) % 2
        sel, ns = pipe.layers[0].sel[jp], pipe.layers[0].n_sel[jp]
        # the same number of blocks per (r, h), shifted by k * K_b blocks
        # (mod the request's blocks): other blocks of the same pool
        nbl = ((ctx + bs - 1) // bs).clamp(min=1).view(B, 1, 1)
        n_rot = min(rotation_count(attn_bytes), max(1, NB // K_b))
        rot_inputs = [sel] + [torch.where(sel >= 0, (sel + k * K_b) % nbl, sel).to(torch.int32).contiguous()
                              for k in range(1, n_rot)]

        def attn_call(q_, t_, o_, w_):
            return oa.oasis_lookahead_attn(q_, pool, t_, t_, ns, ctx, out=o_, ws=w_, n_split=args.n_split)
        rot_how = "tables shifted to other blocks of the pool"
    attn_fns = [lambda r_=r_: attn_call(q4, r_, out_alone, attn_ws) for r_ in rot_inputs]
    # attention launches of each phase in launch order, so that a profiled
    # run's kernel trace can be split the same way (--summarize-profile)
    n_alone = max(20, len(attn_fns))
    log("attention launches: " + json.dumps({"warmup": args.warmup * L, "timed": args.steps * L,
                                             "extra": n_extra * L if extra else 0,
                                             "alone": 2 * len(attn_fns) + n_alone}))
    alone_us = time_rotated(torch, attn_fns, n_alone, label="attention")
    kern["attn_alone"] = alone_entry(attn_bytes, alone_us, len(attn_fns), rot_how)
    del attn_fns
    if not args.attn_sweep:
        del rot_inputs

    # scores alone, over rotated copies of the summaries
    sc_out = pipe.layers[0].scores
    n_rot = rotation_count(score_bytes)
    summs = [summ] + [summ.clone() for _ in range(n_rot - 1)]
    ql0 = q_look[t_last]
    score_fns = [lambda sm_=sm_: oa.oasis_score_blocks(ql0, sm_, ctx, scores=sc_out) for sm_ in summs]
    kern["score_alone"] = alone_entry(score_bytes, time_rotated(torch, score_fns, max(20, n_rot)), n_rot,
                                      "copies of the block summaries")
    del score_fns, summs
    # top-K alone, over rotated copies of the scores
    n_rot = rotation_count(topk_bytes)
    scs = [sc_out] + [sc_out.clone() for _ in range(n_rot - 1)]
    sel_o, n_o = pipe.layers[0].sel[0], pipe.layers[0].n_sel[0]
    topk_fns = [lambda x=x: oa.oasis_select_topk(x, ctx, K_b, sel=sel_o, n_sel=n_o) for x in scs]
    kern["topk_alone"] = alone_entry(topk_bytes, time_rotated(torch, topk_fns, max(20, n_rot)), n_rot,
                                     "copies of the scores")
    del topk_fns, scs
    torch.cuda.empty_cache()

    if args.attn_sweep:
        # look-ahead attention alone over the same blocks for n_q = 1, 2, ...
        # query vectors per request (K / V read once for all of them), over
        # the attention alone leg's rotation of inputs
        sweep = {}
        gq = torch.Generator(device=dev).manual_seed(17)
        for nq in range(1, 16 // (H_q // H_kv) + 1):
            qs = torch.randn((B, nq, H_q, D), generator=gq, device=dev).to(torch.bfloat16)
            o_s = torch.empty_like(qs)
            ws_s = torch.empty((max(oa.oasis_lookahead_attn_workspace_bytes(B, H_q, H_kv, nq, T, args.n_split), 1),),
                               dtype=torch.uint8, device=dev)
            fns = [lambda r_=r_: attn_call(qs, r_, o_s, ws_s) for r_ in rot_inputs]
            us = time_rotated(torch, fns, max(20, len(fns)))
            kv_b = attn_bytes - 2 * n_q * B * H_q * D * 2
            sweep[str(nq)] = {"columns": nq * (H_q // H_kv), "avg_us": round(us, 2),
                              "kv_GBps": round(kv_b / (us * 1e-6) / 1e9, 1)}
        kern["lookahead_attn_alone"] = sweep
        del rot_inputs

    a_us = kern["attn"]["avg_us"]
    achieved = attn_bytes / (a_us * 1e-6) / 1e9
    roofline = {"kernel": "sparse_attn", "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": profiled_traffic("attn_kernel", f"traffic_{w.name}.txt"),
                "bytes_per_launch": attn_bytes, "avg_launch_us": a_us}
    hbm_us = sum(kern[k]["avg_us"] for k in ("attn", "score", "topk"))
    hbm_bytes = attn_bytes + score_bytes + topk_bytes
    kern["hbm_kernels_total"] = {"avg_us": round(hbm_us, 2), "bytes": hbm_bytes,
                                 "GBps": round(hbm_bytes / (hbm_us * 1e-6) / 1e9, 1),
                                 "frac_of_peak": round(hbm_bytes / (hbm_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}

    # a plain 256 MiB device copy after the timed steps: the reference that
    # hardware traffic counters of a profiled run are checked against
    calib_src = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
    calib_dst = torch.empty_like(calib_src)
    calib_dst.copy_(calib_src)
    torch.cuda.synchronize()
    del calib_src, calib_dst
    # a plain streaming read for comparison: torch's sum over 512 MiB of
    # int64 (its fastest reduction here, 5.8 TB/s against 3.8 for float32
    # and 0.85 for int32), four copies in rotation: what the HBM kernels
    # above are up against on this GPU
    reads = [torch.ones(READ_REF_BYTES // 8, dtype=torch.int64, device=dev) for _ in range(4)]
    read_us = time_rotated(torch, [lambda x=x: x.sum() for x in reads], 16)
    kern["hbm_read_reference"] = {
        "avg_us": round(read_us, 2), "bytes": READ_REF_BYTES,
        "GBps": round(READ_REF_BYTES / (read_us * 1e-6) / 1e9, 1),
        "frac_of_peak": round(READ_REF_BYTES / (read_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
        "note": "torch sum over 512 MiB of int64, 4 copies in rotation: a plain streaming read"}
    del reads
    torch.cuda.empty_cache()

    if args.check:
        check_against_oracle(w, pool, ctx_cpu, q_attn, pipe, n_total)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, pool, ctx_cpu, q_look, args.cpu_seconds, C)
    pipe.close()

    line = {
        "metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": B, "context": w.ctx, "heads_q": H_q, "heads_kv": H_kv,
                   "head_dim": D, "block_tokens": bs, "kv_budget_tokens": w.budget, "lookahead_queries": w.J,
                   "fetch_cap": w.cap, "fetch_cap_blocks": C, "slots": S if staged else None,
                   "drift": w.drift if w.structure == "drift" else None,
                   "attention_queries": n_q,
                   "layers_in_flight": L, "step_unit": "layer-step",
                   "kv_location": "pinned host pool + HBM working set" if staged else "HBM",
                   "copy_engine": args.copy_mode if staged else None,
                   "host_threads": args.host_threads if staged and copy_mode != oa.OASIS_COPY_KERNEL else None,
                   "attn_splits": splits, "attn_waves": attn_waves, "compute_streams": pipe.compute_streams,
                   "issue_threads": pipe.issue_threads,
                   "copy_streams": len(pipe.copy) if staged else None},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "h2d": h2d,
        "kernels": kern,
        "host_issue_ms_per_step": round(issued / layer_steps * 1e3, 4),
        "host_cores_busy": round(host_cores, 2),
        "layer_step_us": {**percentiles(step_us), "note": "per decode step of the timed region (main-stream "
                          "events between consecutive steps) / layers in flight"},
    }
    print(json.dumps(line), flush=True)


def agreement_run(args):
    """The synthetic analogue of the pages' lookahead agreement (section 4:
    the draft-based top-K agrees with the true next token's top-K set).  Per
    step s: the predicted set is the top-K of the block scores of the drafts
    of step s; the true set is the top-K by the exact attention mass, over
    the whole context, of the next token's query, taken as the first draft
    plus N(0, sigma^2) noise per coordinate (sigma = 0: a perfect drafter,
    so only the summary bound differs from exact attention).  Agreement is
    |predicted & true| / |true|, averaged over requests, KV heads and steps.
    `agreement_same_rule` takes the other reading of the true set: the same
    block-score top-K applied to the next token's query, which isolates the
    drafts' error from the summary bound's."""
    import torch
    import prefetch_block_scoring_amd as oa
    import workloads as wl

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = wl.WORKLOADS[args.workload]
    if args.drift is not None:
        w = w.shrink(drift=args.drift)
    B, H_q, H_kv, D, bs, K_b, NB = w.B, w.H_q, w.H_kv, w.D, w.bs, w.K_b, w.NB_max
    ctx_cpu = wl.context_lengths(w)
    ctx = ctx_cpu.to(dev)
    if w.staged:   # the host pool of a staged workload is read over PCIe here
        pool = oa.oasis_host_empty((B, H_kv, NB, 2, bs, D), torch.bfloat16)
        wl.kv_pool(w, device=dev, out=pool)
    else:
        pool = wl.kv_pool(w, device=dev)
    summ = oa.oasis_build_summaries(pool, ctx)
    sm = 1.0 / math.sqrt(D)
    sigmas = [0.0, 0.1, 0.25, 0.5, 1.0]
    steps = list(range(1, 1 + max(1, min(args.steps, 8))))
    ws = torch.empty((oa.oasis_block_mass_workspace_bytes(B, H_q, H_kv, NB),), dtype=torch.uint8, device=dev)
    mass = torch.empty((B, H_kv, NB), dtype=torch.float32, device=dev)
    per_sigma = {str(sg): [] for sg in sigmas}
    same_rule = {str(sg): [] for sg in sigmas}
    kept = {}
    for s in steps:
        sc = oa.oasis_score_blocks(wl.lookahead(w, s, dev), summ, ctx)
        psel, pn = oa.oasis_select_topk(sc, ctx, K_b)
        for sg in sigmas:
            q = wl.true_next_query(w, s, sg, dev)
            oa.oasis_block_attention_mass(q, pool, ctx, sm_scale=sm, mass=mass, ws=ws)
            tsel, tn = oa.oasis_select_topk(mass, ctx, K_b)
            ov = oa.oasis_topk_overlap(psel, pn, tsel, tn)
            per_sigma[str(sg)].append(float((ov.float() / tn.clamp(min=1).float()).mean()))
            # the other reading of the true set: the same block-score rule
            # applied to the next token's query instead of the drafts
            ssel, sn = oa.oasis_select_topk(oa.oasis_score_blocks(q[:, None].contiguous(), summ, ctx), ctx, K_b)
            ov2 = oa.oasis_topk_overlap(psel, pn, ssel, sn)
            same_rule[str(sg)].append(float((ov2.float() / sn.clamp(min=1).float()).mean()))
            if s == steps[0]:
                kept[str(sg)] = (q, psel[:1].cpu(), pn[:1].cpu(), ov[:1].cpu())
    # the mass kernel alone (the dense pass over every valid key)
    q0 = kept["0.0"][0]
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(5):
        oa.oasis_block_attention_mass(q0, pool, ctx, sm_scale=sm, mass=mass, ws=ws)
    b.record()
    torch.cuda.synchronize()
    us = a.elapsed_time(b) / 5 * 1e3
    n_keys = int(sum(int(c) for c in ctx_cpu)) * H_kv
    k_bytes = n_keys * D * 2
    result = {
        "metric": "lookahead top-K agreement (synthetic analogue)",
        "workload": w.name, "batch": B, "lookahead_queries": w.J, "kv_budget_tokens": w.budget,
        "steps": len(steps), "structure": w.structure,
        "agreement": {sg: round(sum(v) / len(v), 5) for sg, v in per_sigma.items()},
        "agreement_same_rule": {sg: round(sum(v) / len(v), 5) for sg, v in same_rule.items()},
        "mass_kernel": {"avg_us": round(us, 1), "key_bytes": k_bytes,
                        "GBps": round(k_bytes / (us * 1e-6) / 1e9, 1),
                        "read_from": "pinned host pool over PCIe" if w.staged else "HBM"},
    }
    if args.check:
        # request 0 of the first step against the oracle: mass, true set and
        # overlap (the predicted set is the GPU's, checked elsewhere)
        import numpy as np
        import oracle
        u16 = lambda x: x.contiguous().cpu().view(torch.int16).numpy().view(np.uint16)
        kv0 = u16(pool[:1])
        bad = 0
        for sg, (q, ps, pn0, ov0) in kept.items():
            ref = oracle.block_mass(u16(q[:1]), kv0, ctx_cpu.numpy()[:1], sm)
            tsel, tn = oracle.select(ref.astype(np.float32), ctx_cpu.numpy()[:1], bs, K_b)
            agree = oracle.agreement(ps.numpy(), pn0.numpy(), tsel, tn)
            got = ov0.numpy() / np.maximum(tn, 1)
            bad += int(np.sum(np.abs(got - agree) > 1.5 / K_b))   # one tie swap allowed
        result["oracle_check"] = {"request": 0, "sigmas": len(kept), "pairs_off": bad}
        if bad:
            print(json.dumps(result), flush=True)
            raise SystemExit("agreement check failed")
    print(json.dumps(result), flush=True)


def cpu_baseline(w, pool, ctx_cpu, q_look, seconds, C):
    """The CPU oracle, unchanged, on the same inputs: full-batch layer-steps
    (score, select, staging bookkeeping and a host copy of the admitted
    blocks into a staging buffer, attention over the resident blocks read
    from the host pool) until about `seconds` of work are done."""
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
    # host staging buffer for the admitted blocks of one step (as many as the
    # uncapped first step admits)
    stage_buf = np.empty((w.B * w.H_kv * w.K_b,) + kv_np.shape[3:], dtype=np.uint16) if w.staged else None
    n_steps, t_total, copied = 0, 0.0, 0
    s = 0
    while True:
        ql = q_look[s % len(q_look)].cpu().view(torch.int16).numpy().view(np.uint16)
        qa = q_look[max(s - 1, 0) % len(q_look)][:, 0].contiguous().cpu().view(torch.int16).numpy().view(np.uint16)
        t0 = time.perf_counter()
        sc = oracle.score(ql, summ, ctx, w.bs, w.H_kv)
        sel, n = oracle.select(sc, ctx, w.bs, w.K_b)
        if w.staged:
            adm, na, _, _ = oracle.stage(st, sel, n, sc, ctx, w.bs, w.K_b, w.K_b if s == 0 else C, s)
            # the admitted blocks, copied out of the host pool in (r, h, admission) order
            rr, hh, kk = np.nonzero(np.arange(adm.shape[2])[None, None, :] < na[:, :, None])
            stage_buf[:len(rr)] = kv_np[rr, hh, adm[rr, hh, kk]]
            copied += len(rr)
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
        if t_total >= seconds or n_steps >= 100000:
            break
    log(f"cpu baseline: {n_steps} layer-steps in {t_total:.1f}s")
    return {"value": round(w.B * n_steps / t_total, 2), "unit": "tokens/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": f"{n_steps} full-batch layer-steps (B={w.B}) of score+select+"
                      f"{'stage bookkeeping+host copy of the admitted blocks+' if w.staged else ''}attend, "
                      f"fp64 C oracle, {t_total:.1f}s of CPU time"
                      + (f"; {copied} blocks copied ({copied * 2 * w.bs * w.D * 2 / 1e6:.1f} MB)" if w.staged
                         else ""),
            "threads": oracle.num_threads(), "nproc": os.cpu_count(),
            "cpu_model": _cpu_model()}


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def check_against_oracle(w, pool, ctx_cpu, q_attn, pipe, n_steps):
    """Sampled parity at full size: requests 0 and B-1 of every layer's last
    step, against the oracle's attention over the same resident blocks, each
    attention query on its own (the staging itself is checked against the
    oracle in the test suite)."""
    import numpy as np
    import torch
    import oracle
    log("check: comparing sampled requests against the oracle")
    if not w.staged:
        raise SystemExit("--check covers staged workloads")
    t = n_steps - 1
    rs = sorted({0, w.B - 1})
    u16 = lambda x: x.contiguous().cpu().view(torch.int16).numpy().view(np.uint16)
    kv = u16(pool[rs])
    ctx = ctx_cpu.numpy()[rs]
    bad_total, n_total = 0, 0
    for l in range(pipe.L):
        tb = pipe.table(l, t)
        blocks = tb[1].cpu().numpy()[rs]
        n = tb[2].cpu().numpy()[rs]
        qa = q_attn[t + 3 * l][rs]
        got = (u16(pipe.layers[l].out[rs]).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        if qa.dim() == 3:          # one query per request
            qa, got = qa[:, None], got[:, None]
        for qi in range(qa.shape[1]):  # look-ahead attention: each query on its own
            ref, _ = oracle.attend(u16(qa[:, qi]), kv, ctx, blocks, n, 1 / math.sqrt(w.D))
            bad = np.abs(got[:, qi] - ref) > 2e-3 + 1e-2 * np.abs(ref)
            bad_total += int(bad.sum())
            n_total += bad.size
        # the resident blocks themselves: every slot holds its block's bytes
        ly = pipe.layers[l]
        ws = ly.ws_pool
        for i, r in enumerate(rs):
            slots = tb[0][r].cpu().numpy()
            for h in range(w.H_kv):
                for e in range(int(n[i, h])):
                    if not torch.equal(ws[r, h, int(slots[h, e])].cpu(), pool[r, h, int(blocks[i, h, e])]):
                        bad_total += 1
    log(f"check: {bad_total} of {n_total} outputs (and resident blocks) out of tolerance")
    if bad_total:
        raise SystemExit("check failed")


if __name__ == "__main__":
    main()
