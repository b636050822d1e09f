"""Build libk3dec.so (HIP for gfx950) in-tree with hipcc.

    python -m moe_router_topk_amd.build          # compile
    python -m moe_router_topk_amd.build --usage  # also print per-kernel VGPR/LDS use

Each source compiles to its own object (in parallel, under _build/), then
hipcc links them; no kernel calls device code of another file.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libk3dec.so")
SOURCES = ["api.cpp", "dense.hip", "experts.hip", "moe_b1.hip", "noalloc.hip", "prefetch.hip",
           "skinny.hip"]
ARCH = os.environ.get("K3_OFFLOAD_ARCH", "gfx950")

HIPCC_FLAGS = [
    "-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC", "-Wall",
    # keep hand-written float code off the packed fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]
NOISE = "is not a recognized feature for this target"


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    path = os.path.join(rocm, "bin", "hipcc")
    return path if os.path.exists(path) else "hipcc"


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(ln for ln in res.stderr.splitlines() if NOISE not in ln)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{' '.join(cmd)}\n{err}")
    return err


def build(usage: bool = False, verbose: bool = False) -> str:
    """Compile every source and link libk3dec.so (always recompiles)."""
    os.makedirs(OBJ, exist_ok=True)
    tag = "%d" % os.getpid()
    objs = [os.path.join(OBJ, os.path.splitext(s)[0] + f".{tag}.o") for s in SOURCES]
    extra = ["-Rpass-analysis=kernel-resource-usage"] if usage else []
    cmds = [[hipcc(), *HIPCC_FLAGS, *extra, "-c", "-o", o, os.path.join(CSRC, s)]
            for s, o in zip(SOURCES, objs)]
    jobs = max(1, min(len(cmds), int(os.environ.get("MAX_JOBS", "8"))))
    try:
        with ThreadPoolExecutor(jobs) as ex:
            errs = list(ex.map(_run, cmds))
        tmp = LIB + ".tmp" + tag
        errs.append(_run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-o", tmp, *objs]))
    finally:
        for o in objs:
            if os.path.exists(o):
                os.remove(o)
    if verbose or usage:
        sys.stderr.write("\n".join(e for e in errs if e) + "\n")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(usage="--usage" in sys.argv, verbose="-v" in sys.argv))
