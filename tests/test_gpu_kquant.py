"""GPU parity for the K-quant formats (Q4_K, Q6_K: 256-weight super-blocks)
through the C ABI against the CPU oracle.

Bars as for the 32-weight formats: dequantized weights bit-exact (every byte
pattern, NaN/inf/subnormal scales included); y within the gates of
tests/gates.py; outputs bit-identical across block sizes, windows, grids,
repeats, expert windows and streamed or host-mapped weights.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import quantized_gemv_gguf_amd as q
import synth
from gates import bits_equal, check

pytestmark = pytest.mark.gpu

KFMTS = [q.Q4_K, q.Q6_K]


def dput(a, dev):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def nan_f32(n, dev):
    import torch
    return torch.full((n,), float("nan"), dtype=torch.float32, device=dev)


def sync():
    import torch
    torch.cuda.synchronize()


def pinned(a):
    import torch
    t = torch.empty(a.shape, dtype=torch.uint8, pin_memory=True)
    t.numpy()[...] = a
    return t


def run_rows(dev, fmt, w, rows, k, x, r0=0, r1=None, block_rows=0, pad=0):
    r1 = rows if r1 is None else r1
    buf = nan_f32(r1 - r0 + 2 * pad, dev)
    y = buf[pad:pad + (r1 - r0)]
    q.qgemv_rows(q.Matrix(dput(w, dev), fmt, rows, k), r0, r1, dput(x, dev), y, block_rows)
    sync()
    out = buf.cpu().numpy()
    if pad:
        assert np.isnan(out[:pad]).all() and np.isnan(out[-pad:]).all(), "write outside the window"
    return out[pad:pad + (r1 - r0)]


@pytest.mark.parametrize("fmt", KFMTS)
@pytest.mark.parametrize("kind", ["config", "all_bytes"])
def test_kquant_dequant_bit_exact(dev, fmt, kind):
    import torch
    rows, k = 96, 2048
    w = synth.blocks(fmt, rows, k, seed=11 + fmt) if kind == "config" else synth.random_bytes(fmt, rows, k, 21 + fmt)
    out = torch.empty(rows * k, dtype=torch.float32, device=dev)
    q.qgemv_dequant_rows(q.Matrix(dput(w, dev), fmt, rows, k), 0, rows, out)
    sync()
    assert bits_equal(out.cpu().numpy().reshape(rows, k), oracle.dequant_rows(fmt, w, rows, k))


@pytest.mark.parametrize("fmt", KFMTS)
def test_kquant_dequant_window_offsets(dev, fmt):
    import torch
    rows, k = 40, 512
    w = synth.random_bytes(fmt, rows, k, seed=31)
    wd = dput(w, dev)
    for r0, r1 in [(0, 1), (3, 17), (39, 40), (5, 5)]:
        out = torch.full(((r1 - r0) * k + 8,), float("nan"), dtype=torch.float32, device=dev)
        q.qgemv_dequant_rows(q.Matrix(wd, fmt, rows, k), r0, r1, out)
        sync()
        o = out.cpu().numpy()
        assert bits_equal(o[:(r1 - r0) * k].reshape(r1 - r0, k), oracle.dequant_rows(fmt, w, rows, k, r0, r1))
        assert np.isnan(o[(r1 - r0) * k:]).all()


@pytest.mark.parametrize("fmt", KFMTS)
@pytest.mark.parametrize("k", [256, 512, 2816, 4096, 6144, 11008, 24576, 32768, 49152])
def test_kquant_gemv_shapes(dev, fmt, k):
    """One column per lane up to k = 24576 (12 waves), two above."""
    rows = 301 if k <= 6144 else 83
    w = synth.blocks(fmt, rows, k, seed=1000 + k + fmt)
    x = synth.x_vec(k, seed=2000 + k)
    y = run_rows(dev, fmt, w, rows, k, x, pad=3)
    ref, a = oracle.gemv_rows(fmt, w, rows, k, x)
    check(y, ref, a, what=f"fmt{fmt} k{k}")


@pytest.mark.parametrize("fmt", KFMTS)
def test_kquant_unit_vectors_give_columns(dev, fmt):
    """x = e_i gives column i of dec(W) bit for bit; x = 0 gives zeros."""
    rows, k = 64, 1024
    w = synth.blocks(fmt, rows, k, seed=77)
    dec = oracle.dequant_rows(fmt, w, rows, k)
    for i in [0, 15, 16, 31, 32, 255, 256, 700, 1023]:
        x = np.zeros(k, np.float32)
        x[i] = 1.0
        y = run_rows(dev, fmt, w, rows, k, x)
        assert np.array_equal(y, dec[:, i]), f"column {i}"
    assert np.all(run_rows(dev, fmt, w, rows, k, np.zeros(k, np.float32)) == 0)


@pytest.mark.parametrize("fmt", KFMTS)
@pytest.mark.parametrize("k", [2816, 11008])
def test_kquant_block_rows_and_windows_bit_identical(dev, fmt, k):
    rows = 700
    w = synth.blocks(fmt, rows, k, seed=3000 + k)
    x = synth.x_vec(k, seed=3100 + k)
    full = run_rows(dev, fmt, w, rows, k, x)
    for b in [1, 7, 128, 512]:
        assert bits_equal(run_rows(dev, fmt, w, rows, k, x, block_rows=b), full), f"block_rows {b}"
    for r0, r1, b in [(0, 1, 0), (5, 333, 7), (333, 700, 128), (699, 700, 3)]:
        y = run_rows(dev, fmt, w, rows, k, x, r0, r1, block_rows=b, pad=5)
        assert bits_equal(y, full[r0:r1]), f"window {r0}:{r1} B={b}"
    assert bits_equal(run_rows(dev, fmt, w, rows, k, x), full)


@pytest.mark.parametrize("fmt", KFMTS)
def test_kquant_expert_windows(dev, fmt):
    """Expert windows of a stacked (8, 256, 1024) tensor: one grid over the
    selected experts' rows equals one qgemv_rows call per expert."""
    import torch
    E, out, k, sel = 8, 256, 1024, [1, 4, 7]
    w = synth.blocks(fmt, E * out, k, seed=5000 + fmt)
    m = q.Matrix(dput(w, dev), fmt, E * out, k)
    xs = np.stack([synth.x_vec(k, 5100 + s) for s in range(len(sel))])
    xd = dput(xs.reshape(-1), dev)
    y = nan_f32(len(sel) * out, dev)
    q.qgemv_expert_windows([m], E, sel, xd, k, y, block_rows=100)
    sync()
    got = y.cpu().numpy().reshape(len(sel), out)
    for s, e in enumerate(sel):
        single = nan_f32(out, dev)
        q.qgemv_rows(m, e * out, (e + 1) * out, dput(xs[s], dev), single)
        sync()
        assert bits_equal(got[s], single.cpu().numpy())
        ref, a = oracle.gemv_rows(fmt, w, E * out, k, xs[s], e * out, (e + 1) * out)
        check(got[s], ref, a, what=f"expert {e}")


@pytest.mark.parametrize("fmt", KFMTS)
def test_kquant_streamed_and_mapped_equal_resident(dev, fmt):
    import torch
    rows, k = 3000, 4096
    w = synth.blocks(fmt, rows, k, seed=6000 + fmt)
    x = dput(synth.x_vec(k, 6100), dev)
    ref = nan_f32(rows, dev)
    q.qgemv_rows(q.Matrix(dput(w, dev), fmt, rows, k), 0, rows, x, ref)
    pin = q.Matrix(pinned(w), fmt, rows, k)
    rb = q.qgemv_weight_bytes(fmt, 1, k)
    for B in (128, 512):
        with q.Streamer(B * rb, 2) as st:
            y = nan_f32(rows, dev)
            st.rows(pin, 0, rows, x, y, B)
            sync()
            assert bits_equal(y.cpu().numpy(), ref.cpu().numpy()), f"streamed B={B}"
        y = nan_f32(rows, dev)
        q.qgemv_mapped_rows(pin, 0, rows, x, y, B)
        sync()
        assert bits_equal(y.cpu().numpy(), ref.cpu().numpy()), f"mapped B={B}"
