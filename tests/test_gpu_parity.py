"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Bars: dequantized weights bit-exact; y within the gates of tests/gates.py
(1e-4 against the fp64 oracle); outputs bit-identical across block sizes,
windows, grids and repeats.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import quantized_gemv_gguf_amd as q
import synth
from gates import bits_equal, check

pytestmark = pytest.mark.gpu

FMTS = [q.Q8_0, q.Q4_0, q.MXFP4]


def dput(a, dev):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def nan_f32(n, dev):
    import torch
    return torch.full((n,), float("nan"), dtype=torch.float32, device=dev)


def run_rows(dev, fmt, w, rows, k, x, r0=0, r1=None, block_rows=0, pad=0):
    """GPU y for rows [r0, r1) with `pad` NaN sentinels on each side."""
    import torch
    r1 = rows if r1 is None else r1
    wd, xd = dput(w, dev), dput(x, dev)
    buf = nan_f32(r1 - r0 + 2 * pad, dev)
    y = buf[pad:pad + (r1 - r0)]
    q.qgemv_rows(q.Matrix(wd, fmt, rows, k), r0, r1, xd, y, block_rows)
    torch.cuda.synchronize()
    out = buf.cpu().numpy()
    if pad:
        assert np.isnan(out[:pad]).all() and np.isnan(out[-pad:]).all(), "write outside the window"
    return out[pad:pad + (r1 - r0)]


# --- decode: bit-exact -------------------------------------------------------------

@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("kind", ["config", "all_bytes"])
def test_dequant_bit_exact(dev, fmt, kind):
    import torch
    rows, k = 96, 2048
    if kind == "config":
        w = synth.blocks(fmt, rows, k, seed=11 + fmt)
    else:  # every byte uniform: NaN/inf/subnormal scales and every code
        w = synth.random_bytes(fmt, rows, k, seed=21 + fmt)
    wd = dput(w, dev)
    out = torch.empty(rows * k, dtype=torch.float32, device=dev)
    q.qgemv_dequant_rows(q.Matrix(wd, fmt, rows, k), 0, rows, out)
    torch.cuda.synchronize()
    ref = oracle.dequant_rows(fmt, w, rows, k)
    assert bits_equal(out.cpu().numpy().reshape(rows, k), ref)


@pytest.mark.parametrize("fmt", FMTS)
def test_dequant_window_offsets(dev, fmt):
    import torch
    rows, k = 40, 96
    w = synth.random_bytes(fmt, rows, k, seed=31)
    wd = dput(w, dev)
    for r0, r1 in [(0, 1), (3, 17), (39, 40), (5, 5)]:
        out = torch.full(((r1 - r0) * k + 8,), float("nan"), dtype=torch.float32, device=dev)
        q.qgemv_dequant_rows(q.Matrix(wd, fmt, rows, k), r0, r1, out)
        torch.cuda.synchronize()
        o = out.cpu().numpy()
        assert bits_equal(o[:(r1 - r0) * k].reshape(r1 - r0, k), oracle.dequant_rows(fmt, w, rows, k, r0, r1))
        assert np.isnan(o[(r1 - r0) * k:]).all()


# --- GEMV values ----------------------------------------------------------------------

def test_config1_q8_0_256x1024(dev):
    rows, k = 256, 1024
    w = synth.blocks(q.Q8_0, rows, k, synth.seed_of(1, 0))
    x = synth.x_vec(k, synth.seed_of(1, 9))
    y = run_rows(dev, q.Q8_0, w, rows, k, x, pad=4)
    ref, a = oracle.gemv_rows(q.Q8_0, w, rows, k, x)
    check(y, ref, a, what="cfg1")


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("k", [32, 96, 1024, 2880, 4096, 6144, 11008, 24576])
def test_gemv_shapes(dev, fmt, k):
    rows = 301 if k <= 6144 else 83  # ragged row counts, several tiles and teams
    w = synth.blocks(fmt, rows, k, seed=1000 + k + fmt)
    x = synth.x_vec(k, seed=2000 + k)
    y = run_rows(dev, fmt, w, rows, k, x, pad=3)
    ref, a = oracle.gemv_rows(fmt, w, rows, k, x)
    check(y, ref, a, what=f"fmt{fmt} k{k}")


@pytest.mark.parametrize("fmt", FMTS)
def test_gemv_special_inputs(dev, fmt):
    """x = unit vector gives column i of dec(W) exactly; x = 0 gives zeros."""
    rows, k = 64, 256
    w = synth.blocks(fmt, rows, k, seed=77)
    dec = oracle.dequant_rows(fmt, w, rows, k)
    for i in [0, 31, 32, 200, 255]:
        x = np.zeros(k, np.float32)
        x[i] = 1.0
        y = run_rows(dev, fmt, w, rows, k, x)
        assert np.array_equal(y, dec[:, i]), f"column {i}"
    y = run_rows(dev, fmt, w, rows, k, np.zeros(k, np.float32))
    assert np.all(y == 0)


def test_config2_q4_0_4096(dev):
    rows, k = 4096, 4096
    w = synth.blocks(q.Q4_0, rows, k, synth.seed_of(2, 0))
    x = synth.x_vec(k, synth.seed_of(2, 9))
    y0 = run_rows(dev, q.Q4_0, w, rows, k, x, block_rows=0)
    y512 = run_rows(dev, q.Q4_0, w, rows, k, x, block_rows=512)
    assert bits_equal(y0, y512)
    ref, a = oracle.gemv_rows(q.Q4_0, w, rows, k, x)
    check(y0, ref, a, what="cfg2")


# --- bit identity across block sizes, windows, grids, repeats ------------------------

@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("k", [1024, 2880, 11008])
def test_block_rows_and_windows_bit_identical(dev, fmt, k):
    rows = 700
    w = synth.blocks(fmt, rows, k, seed=3000 + k)
    x = synth.x_vec(k, seed=3100 + k)
    full = run_rows(dev, fmt, w, rows, k, x)
    for b in [1, 7, 100, 128, 512, 2048]:
        assert bits_equal(run_rows(dev, fmt, w, rows, k, x, block_rows=b), full), f"block_rows {b}"
    for r0, r1, b in [(0, 1, 0), (1, 2, 0), (5, 333, 7), (333, 700, 128), (699, 700, 3), (64, 129, 64)]:
        y = run_rows(dev, fmt, w, rows, k, x, r0, r1, block_rows=b, pad=5)
        assert bits_equal(y, full[r0:r1]), f"window {r0}:{r1} B={b}"
    for _ in range(3):
        assert bits_equal(run_rows(dev, fmt, w, rows, k, x), full)


def test_empty_windows_are_noops(dev):
    import torch
    rows, k = 16, 64
    w = dput(synth.blocks(q.Q8_0, rows, k, 5), dev)
    x = dput(synth.x_vec(k, 6), dev)
    y = nan_f32(4, dev)
    q.qgemv_rows(q.Matrix(w, q.Q8_0, rows, k), 7, 7, x, y)
    q.qgemv_windows([], fmt=q.Q8_0, k=k)
    empty = torch.empty(0, dtype=torch.uint8, device=dev)
    q.qgemv_rows(q.Matrix(empty, q.Q8_0, 0, k), 0, 0, x, y)
    torch.cuda.synchronize()
    assert np.isnan(y.cpu().numpy()).all()


@pytest.mark.parametrize("fmt", FMTS)
def test_windows_grid_equals_single_rows(dev, fmt):
    """One qgemv_windows grid over windows of different matrices, inputs and
    outputs gives the same bits as one qgemv_rows call per window."""
    import torch
    k = 2880
    mats = []
    for i, rows in enumerate([500, 37, 1200]):
        w = synth.blocks(fmt, rows, k, seed=4000 + i)
        mats.append((w, rows, q.Matrix(dput(w, dev), fmt, rows, k)))
    xs = [dput(synth.x_vec(k, 4100 + i), dev) for i in range(3)]
    spec = [(0, 10, 490, 0), (1, 0, 37, 1), (2, 100, 1199, 2), (0, 0, 500, 2), (2, 1199, 1200, 0)]
    wins, outs = [], []
    for mi, r0, r1, xi in spec:
        y = nan_f32(r1 - r0, dev)
        outs.append(y)
        wins.append(q.Window(mats[mi][2], r0, r1, xs[xi], y))
    q.qgemv_windows(wins, block_rows=64)
    torch.cuda.synchronize()
    for (mi, r0, r1, xi), y in zip(spec, outs):
        single = nan_f32(r1 - r0, dev)
        q.qgemv_rows(mats[mi][2], r0, r1, xs[xi], single)
        torch.cuda.synchronize()
        assert bits_equal(y.cpu().numpy(), single.cpu().numpy())
        w, rows, _ = mats[mi]
        ref, a = oracle.gemv_rows(fmt, w, rows, k, xs[xi].cpu().numpy(), r0, r1)
        check(y.cpu().numpy(), ref, a, what=f"window {mi}:{r0}:{r1}")


# --- elementwise steps ------------------------------------------------------------------

def test_silu_mul(dev):
    import torch
    n = 11008 + 13
    g = np.random.default_rng(1).standard_normal(n).astype(np.float32) * 4
    g[:8] = [-100.0, -89.0, -50.0, -0.0, 0.0, 30.0, 89.0, 100.0]  # exp2 overflow / underflow ends
    u = np.random.default_rng(2).standard_normal(n).astype(np.float32)
    h = torch.empty(n, dtype=torch.float32, device=dev)
    q.qgemv_silu_mul(dput(g, dev), dput(u, dev), h)
    torch.cuda.synchronize()
    ref = oracle.silu_mul(g, u)
    # hardware exp2 and reciprocal: about (|g| + 4) 2^-24 relative
    tol = (np.abs(g.astype(np.float64)) + 8) * 2.0 ** -24 * np.abs(ref) + 1e-30
    assert np.all(np.abs(h.cpu().numpy() - ref) <= tol)


@pytest.mark.parametrize("gelu", [False, True])
@pytest.mark.parametrize("n", [1, 6144, 24576, 18432 // 3 + 5])
def test_rms_carry(dev, gelu, n):
    import torch
    v = np.random.default_rng(n).standard_normal(n).astype(np.float32) * 3
    out = torch.empty(n, dtype=torch.float32, device=dev)
    q.qgemv_rms_carry(dput(v, dev), out, 1e-6, gelu)
    torch.cuda.synchronize()
    ref = oracle.rms_carry(v, 1e-6, gelu)
    assert np.max(np.abs(out.cpu().numpy() - ref)) <= 1e-5 * max(1.0, np.abs(ref).max())
