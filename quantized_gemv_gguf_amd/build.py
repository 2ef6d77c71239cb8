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
SRC = os.path.join(HERE, "csrc", "qgemv.hip")
INC = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libqgemv.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    "-Wno-unused-result",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cand = os.path.join(rocm, "bin", "hipcc")
    return cand if os.path.exists(cand) else "hipcc"


def build(verbose: bool = False) -> str:
    """Compile csrc/qgemv.hip into libqgemv.so (always recompiles)."""
    tmp = LIB + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, f"-I{INC}", SRC, "-o", tmp]
    if verbose:
        print(" ".join(cmd), file=sys.stderr)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{r.stderr[-6000:]}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
