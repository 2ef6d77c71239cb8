"""GPU determinism across processes (I4): the SHA-256 of each workload's
outputs is the same in this process and in two fresh ones, and does not depend
on block_rows (Q4_0 4096 x 4096 at block_rows 0 and 512; four MXFP4 MoE tokens
at 0 and 128; two tokens of a two-layer dense pass)."""
from __future__ import annotations

import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))


def test_hashes_agree_across_processes(dev):
    import determinism_worker
    mine = determinism_worker.hashes()
    assert mine["q4_0_4096_B0"] == mine["q4_0_4096_B512"]
    assert mine["moe_4tok_B0"] == mine["moe_4tok_B128"]
    for run in range(2):
        print(f"determinism: fresh process {run}", flush=True)
        r = subprocess.run([sys.executable, "-u", os.path.join(HERE, "determinism_worker.py")],
                           capture_output=True, text=True, timeout=110)
        assert r.returncode == 0, r.stderr[-2000:]
        other = json.loads(r.stdout.strip().splitlines()[-1])
        assert other == mine, (run, other, mine)
