"""GPU parity for the paired gate/up grid (qgemv_rows_swiglu,
qgemv_expert_swiglu): h = silu(gate . x') * (up . x') must have the bits of
the separate GEMVs followed by qgemv_silu_mul, and those GEMVs pass the
oracle's gates."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import quantized_gemv_gguf_amd as q
import synth
from gates import bits_equal, check

pytestmark = pytest.mark.gpu


def dput(a, dev):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def sync():
    import torch
    torch.cuda.synchronize()


# (format, rows, k): teams of 1, 2, 3 and 12 waves, two columns per lane
SHAPES = [(q.Q8_0, 301, 96), (q.Q8_0, 1100, 4096), (q.Q4_0, 257, 4096), (q.MXFP4, 200, 2880),
          (q.Q4_K, 130, 6144), (q.Q6_K, 71, 24576), (q.Q8_0, 65, 24576), (q.Q8_0, 33, 32768)]


def separate(dev, G, U, r0, r1, x, in_rms):
    import torch
    f32 = dict(dtype=torch.float32, device=dev)
    xd = dput(x, dev)
    if in_rms:
        t = torch.empty(x.size, **f32)
        q.qgemv_rms_carry(xd, t, 1e-6, False)
        xd = t
    g, u, h = (torch.empty(r1 - r0, **f32) for _ in range(3))
    q.qgemv_rows(G, r0, r1, xd, g)
    q.qgemv_rows(U, r0, r1, xd, u)
    q.qgemv_silu_mul(g, u, h)
    sync()
    return g.cpu().numpy(), u.cpu().numpy(), h.cpu().numpy()


@pytest.mark.parametrize("fmt,rows,k", SHAPES)
def test_rows_swiglu_equals_separate(dev, fmt, rows, k):
    import torch
    wg = synth.blocks(fmt, rows, k, synth.seed_of(12, 10 * fmt))
    wu = synth.blocks(fmt, rows, k, synth.seed_of(12, 10 * fmt + 1))
    G, U = q.Matrix(dput(wg, dev), fmt, rows, k), q.Matrix(dput(wu, dev), fmt, rows, k)
    x = (2.0 * synth.x_vec(k, synth.seed_of(12, 50))).astype(np.float32)
    for in_rms in (False, True):
        for r0, r1, B in [(0, rows, 0), (0, rows, 1), (3, rows - 2, 7), (rows // 2, rows // 2 + 1, 0), (5, rows, 64)]:
            g, u, ref = separate(dev, G, U, r0, r1, x, in_rms)
            hb = torch.full((r1 - r0 + 4,), float("nan"), dtype=torch.float32, device=dev)
            q.qgemv_rows_swiglu(G, U, r0, r1, dput(x, dev), hb[2:2 + r1 - r0], q.IN_RMS if in_rms else q.IN_X,
                                1e-6, block_rows=B)
            sync()
            got = hb.cpu().numpy()
            assert np.isnan(got[:2]).all() and np.isnan(got[-2:]).all(), "write outside the window"
            assert bits_equal(got[2:2 + r1 - r0], ref), f"rms {in_rms} rows {r0}:{r1} B={B}"
    g, u, _ = separate(dev, G, U, 0, rows, x, False)
    for w, y in ((wg, g), (wu, u)):
        r, a = oracle.gemv_rows(fmt, w, rows, k, x)
        check(y, r, a, what="gate/up")


@pytest.mark.parametrize("fmt,E,out,k", [(q.MXFP4, 128, 2880, 2880), (q.Q4_K, 16, 512, 1024),
                                         (q.Q8_0, 8, 300, 4096)])
def test_expert_swiglu_equals_separate(dev, fmt, E, out, k):
    import torch
    wg = synth.blocks(fmt, E * out, k, synth.seed_of(12, 20 + fmt))
    wu = synth.blocks(fmt, E * out, k, synth.seed_of(12, 30 + fmt))
    G, U = q.Matrix(dput(wg, dev), fmt, E * out, k), q.Matrix(dput(wu, dev), fmt, E * out, k)
    ids = [1, E // 2, E - 1, 3]
    ns = len(ids)
    f32 = dict(dtype=torch.float32, device=dev)
    for x_stride in (0, k):
        xs = np.stack([synth.x_vec(k, synth.seed_of(12, 60 + s)) for s in range(ns)]).reshape(-1)
        xd = dput(xs, dev)
        gu = torch.empty(2 * ns * out, **f32)
        ref = torch.empty(ns * out, **f32)
        q.qgemv_expert_windows([G, U], E, ids, xd, x_stride, gu)
        q.qgemv_silu_mul(gu[:ns * out], gu[ns * out:], ref)
        for B in (0, 100):
            h = torch.full((ns * out,), float("nan"), **f32)
            q.qgemv_expert_swiglu(G, U, E, ids, xd, x_stride, h, block_rows=B)
            sync()
            assert bits_equal(h.cpu().numpy(), ref.cpu().numpy()), f"x_stride {x_stride} B {B}"
