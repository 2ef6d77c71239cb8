"""CPU: bench.py's command line.  More than one GPU is refused with a message
before anything touches a device, and the workload list parses."""
from __future__ import annotations

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          timeout=120, cwd=ROOT)


def test_more_than_one_gpu_is_refused():
    for n in ("2", "8"):
        r = _run("--gpus", n)
        assert r.returncode == 2
        assert "runs on one GPU" in r.stderr and r.stdout == ""


def test_help_lists_the_workloads():
    r = _run("--help")
    assert r.returncode == 0
    for w in ("q4_0_4096", "moe_mxfp4", "ffn_streamed", "q4_k_m_dense20b", "dense20b_batch", "--eager"):
        assert w in r.stdout
