"""Build libqgemv.so in-tree with hipcc for gfx950.

Every HIP translation unit is compiled with packed FP32 instructions switched
off (``-Xclang -target-feature -Xclang -packed-fp32-ops``); hipcc's host pass
warns that it does not know the feature, which is harmless.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
# qgemv.hip: chain kernel, small kernels and the C ABI; gemv_op*.hip: one
# fused-transform variant of the GEMV kernel each (all formats and team shapes),
# compiled in parallel and linked into one library.
SOURCES = ["qgemv.hip"] + [f"gemv_op{i}.hip" for i in range(7)] + ["gemv_batch.hip", "gemv_mfma.hip"]
HEADERS = ["qgemv_impl.h"]
INC = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libqgemv.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-result",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # the first three kernel arguments of every kernel arrive in scalar
    # registers (the GEMV kernels' leading x, nb and tile count)
    "-mllvm", "-amdgpu-kernarg-preload-count=3",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cand = os.path.join(rocm, "bin", "hipcc")
    return cand if os.path.exists(cand) else "hipcc"


def source_paths():
    """Every file the kernels are built from (hashed by bench.py to tie HBM
    counter summaries to the code they were taken on)."""
    return [os.path.join(CSRC, f) for f in SOURCES + HEADERS]


def build(verbose: bool = False) -> str:
    """Compile csrc/*.hip (in parallel) and link libqgemv.so (always recompiles)."""
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    procs = []
    for s in SOURCES:
        obj = os.path.join(objdir, s.replace(".hip", ".o"))
        log = obj + ".log"
        cmd = [hipcc(), *HIPCC_FLAGS, f"-I{INC}", "-c", os.path.join(CSRC, s), "-o", obj]
        if verbose:
            print(" ".join(cmd), file=sys.stderr)
        with open(log, "w") as lf:  # a file, not a pipe: a full pipe would stall the compiler
            procs.append((s, obj, log, subprocess.Popen(cmd, stdout=lf, stderr=subprocess.STDOUT)))
    objs = []
    for s, obj, log, pr in procs:
        pr.wait()
        if pr.returncode != 0:
            raise RuntimeError(f"hipcc failed on {s} ({pr.returncode}):\n{open(log).read()[-6000:]}")
        objs.append(obj)
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed ({r.returncode}):\n{r.stderr[-6000:]}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
