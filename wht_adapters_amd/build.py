"""Build libwhtq.so for gfx950 in-tree with hipcc.

Each translation unit under csrc/ is compiled to an object in parallel,
then linked into wht_adapters_amd/libwhtq.so.  Run as
``python -m wht_adapters_amd.build`` or through __graft_entry__.build().
"""
import concurrent.futures as cf
import glob
import os
import subprocess
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT_DIR = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libwhtq.so")
ARCH = os.environ.get("WHTQ_ARCH", "gfx950")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "-std=c++17", "-O3", "-fPIC", f"--offload-arch={ARCH}",
    # keep packed-fp32 VALU forms out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


# per-source extra flags: the matrix-core quantiser keeps its MFMA
# accumulators in ordinary VGPRs (the VALU stages read them directly, and the
# AGPR form would add a copy per value and cost occupancy)
EXTRA = {f"rq_fwd_b{b}.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"] for b in (2, 3, 4)}


def _compile(src):
    obj = os.path.join(OUT_DIR, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, *EXTRA.get(os.path.basename(src), []), "-c", src, "-o", obj]
    t0 = time.time()
    p = subprocess.run(cmd, capture_output=True, text=True)
    if p.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{p.stderr[-8000:]}")
    return obj, time.time() - t0


def build(verbose=True, jobs=None):
    os.makedirs(OUT_DIR, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    jobs = jobs or min(len(srcs), max(1, (os.cpu_count() or 4)))
    with cf.ThreadPoolExecutor(jobs) as ex:
        results = list(ex.map(_compile, srcs))
    if verbose:
        for (obj, dt) in results:
            print(f"  compiled {os.path.basename(obj)} in {dt:.1f}s", flush=True)
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + [o for o, _ in results]
    p = subprocess.run(cmd, capture_output=True, text=True)
    if p.returncode != 0:
        raise RuntimeError(f"link failed:\n{p.stderr[-8000:]}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"  linked {LIB}", flush=True)
    return LIB


if __name__ == "__main__":
    build()
    sys.exit(0)
