"""Computes SHA-256 hashes of GPU outputs for a few workloads and prints them
as one JSON line.  Run by tests/test_gpu_determinism.py in fresh processes,
and imported by it to compute the same hashes in its own process: every run
must print the same hashes (a row's bits depend only on its bytes, x, the
format and k -- not on the process, the launch or the block size)."""
from __future__ import annotations

import hashlib
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import quantized_gemv_gguf_amd as q  # noqa: E402
import synth  # noqa: E402


def _sha(t) -> str:
    return hashlib.sha256(t.detach().contiguous().cpu().numpy().tobytes()).hexdigest()


def hashes() -> dict:
    import torch
    dev = torch.device("cuda:0")
    f32 = dict(dtype=torch.float32, device=dev)
    out = {}
    # Q4_0 4096 x 4096 at block_rows 0 and 512
    rows = k = 4096
    w = torch.from_numpy(synth.blocks(q.Q4_0, rows, k, synth.seed_of(2, 0))).to(dev)
    x = torch.from_numpy(synth.x_vec(k, synth.seed_of(2, 9))).to(dev)
    for B in (0, 512):
        y = torch.empty(rows, **f32)
        q.qgemv_rows(q.Matrix(w, q.Q4_0, rows, k), 0, rows, x, y, B)
        out[f"q4_0_4096_B{B}"] = _sha(y)
    # MXFP4 experts: 4 tokens, gate/up pairs, down, combine, block_rows 0 and 128
    E, o, k = 128, 2880, 2880
    mats = [q.Matrix(torch.from_numpy(synth.blocks(q.MXFP4, E * o, k, synth.seed_of(4, t))).to(dev), q.MXFP4,
                     E * o, k) for t in range(3)]
    ids = synth.expert_ids(E, 4, 4, synth.seed_of(4, 8))
    wts = torch.from_numpy(synth.router_weights(4, 4, synth.seed_of(4, 9))).to(dev)
    for B in (0, 128):
        ys = []
        for t in range(4):
            xt = torch.from_numpy(synth.x_vec(k, synth.seed_of(4, 100 + t))).to(dev)
            h, ye, yt = torch.empty(4 * o, **f32), torch.empty(4 * o, **f32), torch.empty(o, **f32)
            q.qgemv_expert_swiglu(mats[0], mats[1], E, ids[t], xt, 0, h, block_rows=B)
            q.qgemv_expert_windows([mats[2]], E, ids[t], h, o, ye, B)
            q.qgemv_combine(ye, o, 4, wts[t], o, yt)
            ys.append(yt)
        out[f"moe_4tok_B{B}"] = _sha(torch.stack(ys))
    # two layers of the dense pass as fused launches, two tokens
    H, F = 6144, 24576
    shapes = synth.dense_layer_shapes(H, F)
    ws = [[torch.from_numpy(synth.blocks(q.Q8_0, r, kk, synth.seed_of(5, 4 * l + m))).to(dev)
           for m, (_, r, kk) in enumerate(shapes)] for l in range(2)]
    d = torch.from_numpy(synth.x_vec(H, synth.seed_of(5, 999))).to(dev)
    qkv, ov, a = torch.empty(3 * H, **f32), torch.empty(H, **f32), torch.empty(F, **f32)
    for _ in range(2):
        for l in range(2):
            M = [q.Matrix(ws[l][m], q.Q8_0, r, kk) for m, (_, r, kk) in enumerate(shapes)]
            q.qgemv_rows_op(M[0], 0, 3 * H, d, qkv, q.IN_RMS, 1e-6)
            q.qgemv_rows_op(M[1], 0, H, qkv[2 * H:], ov, q.IN_RMS, 1e-6)
            q.qgemv_rows_op(M[2], 0, F, ov, a, q.IN_RMS, 1e-6, q.OUT_GELU)
            q.qgemv_rows_op(M[3], 0, H, a, d, q.IN_RMS, 1e-6)
    out["dense_2L_2tok"] = _sha(d)
    torch.cuda.synchronize()
    return out


if __name__ == "__main__":
    print(json.dumps(hashes()), flush=True)
