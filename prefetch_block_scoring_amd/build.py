"""Build liboasis.so (HIP, gfx950) in-tree.

    python prefetch_block_scoring_amd/build.py

(run it as a file: importing the package loads the library this builds)

Every HIP source is compiled with packed-fp32 instructions disabled
(``-Xclang -target-feature -Xclang -packed-fp32-ops``): the kernels are written
with scalar fp32 arithmetic only.
"""
import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "liboasis.so")
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    return "hipcc"


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def build(verbose: bool = False) -> str:
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)
    flags = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wall", "-Wno-unused-function", "-I", INCLUDE, "-I", CSRC]
    objs = []
    procs = []
    for src in sources():
        obj = os.path.join(objdir, os.path.basename(src) + ".o")
        cmd = [hipcc()] + flags + ["-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((subprocess.Popen(cmd), src))
        objs.append(obj)
    failed = [src for p, src in procs if p.wait() != 0]
    if failed:
        raise RuntimeError(f"hipcc failed for {failed}")
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


def resource_usage(names=("score.hip", "attn.hip", "topk.hip", "stage.hip")) -> str:
    """The compiler's register, LDS, scratch and occupancy figures of each
    kernel in the named sources (device pass only, nothing is written)."""
    flags = ["-O3", "-std=c++17", f"--offload-arch={ARCH}", "--cuda-device-only",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Rpass-analysis=kernel-resource-usage", "-I", INCLUDE, "-I", CSRC, "-o", os.devnull, "-c"]
    import re
    keys = (("TotalSGPRs", "sgpr"), ("VGPRs", "vgpr"), ("AGPRs", "agpr"), ("ScratchSize [bytes/lane]", "scratch"),
            ("Occupancy [waves/SIMD]", "waves/SIMD"), ("SGPRs Spill", "sgpr spill"),
            ("VGPRs Spill", "vgpr spill"), ("LDS Size [bytes/block]", "LDS bytes"))
    out = [f"{'source':11s} {'kernel':34s} " + " ".join(f"{lab:>10s}" for _, lab in keys)]
    for name in names:
        r = subprocess.run([hipcc()] + flags + [os.path.join(CSRC, name)], capture_output=True, text=True)
        kern, vals = None, {}
        for line in r.stderr.splitlines() + ["remark: Function Name: <end>"]:
            if "remark:" not in line:
                continue
            body = line.split("remark:", 1)[1].split(" [-Rpass")[0].strip()
            field, _, value = body.partition(": ")
            if field == "Function Name":
                if kern is not None:
                    m = re.search(r"\d([a-z][a-z0-9_]*_kernel)((?:I|)(?:Li\d+E)+)?", kern)
                    args = re.findall(r"Li(\d+)E", m.group(2) or "") if m else []
                    label = (m.group(1) + (f"<{', '.join(args)}>" if args else "")) if m else kern
                    out.append(f"{name:11s} {label:34s} " + " ".join(f"{vals.get(k, '-'):>10s}" for k, _ in keys))
                kern, vals = value, {}
            else:
                vals[field] = value
    return "\n".join(out)


if __name__ == "__main__":
    if "--resource-usage" in sys.argv:
        print(resource_usage())
    else:
        build(verbose="-q" not in sys.argv)
