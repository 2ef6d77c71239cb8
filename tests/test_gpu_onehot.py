"""GPU: the GEMV kernels' own decoders, position by position.

With x a unit vector e_i, row r's product is its weight w[r, i] times 1 plus
exact zeros, so y[r] must equal the oracle's dequantized weight exactly.  That
pins every GEMV decoder (the one-token kernel, the several-token kernel and the
matrix-core kernel, each with its own code formation) at every position of a
block -- all 32 of a block in the first and second column of a lane, all 256 of
a K-quant super-block -- and at scales of every kind: positive and negative,
fp16 subnormal and largest, E8M0 from 2^-127 (subnormal weights) to 2^125.
Scale fields are finite, so no other weight turns the zeros into NaN.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import quantized_gemv_gguf_amd as q
import synth

pytestmark = pytest.mark.gpu

ROWS = 24
K = 4096
HALVES = [0x3C00, 0xBC00, 0x0001, 0x03FF, 0x83FF, 0x7BFF, 0x1A3F, 0x9A3F, 0x2E66, 0xC500]
E8M0 = [0, 1, 50, 100, 127, 140, 200, 252]


def dput(a, dev):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def matrix(fmt, seed):
    """Uniform random payload bytes with finite scale fields of every kind
    (row r takes the r-th kinds, cycling)."""
    rng = np.random.default_rng(seed)
    w = synth.random_bytes(fmt, ROWS, K, seed)
    bb = synth.BLOCK_BYTES[fmt]
    v = w.reshape(ROWS, -1, bb)
    for r in range(ROWS):
        if fmt in (q.Q8_0, q.Q4_0):
            h = HALVES[r % len(HALVES)]
            v[r, :, 0], v[r, :, 1] = h & 0xFF, h >> 8
        elif fmt == q.MXFP4:
            v[r, :, 0] = E8M0[r % len(E8M0)]
        elif fmt == q.Q4_K:
            d, dm = HALVES[r % len(HALVES)], HALVES[(r + 3) % len(HALVES)]
            v[r, :, 0], v[r, :, 1] = d & 0xFF, d >> 8
            v[r, :, 2], v[r, :, 3] = dm & 0xFF, dm >> 8
        else:  # Q6_K: d last; int8 scales of any value
            d = HALVES[r % len(HALVES)]
            v[r, :, 208], v[r, :, 209] = d & 0xFF, d >> 8
    assert np.all(np.isfinite(oracle.dequant_rows(fmt, w, ROWS, K)))
    return w


def positions(fmt):
    if synth.BLOCK_WEIGHTS[fmt] == 256:  # every position of super-blocks 0 and 15
        return [p for b in (0, 15) for p in range(256 * b, 256 * b + 256)]
    # every position of blocks 0, 1, 63 (a lane's first column) and 64, 127
    # (the second column of the two-column formats)
    return [p for b in (0, 1, 63, 64, 127) for p in range(32 * b, 32 * b + 32)]


def unit_vectors(pos):
    xs = np.zeros((len(pos), K), np.float32)
    xs[np.arange(len(pos)), pos] = 1.0
    return xs


@pytest.mark.parametrize("fmt", [q.Q8_0, q.Q4_0, q.MXFP4, q.Q4_K, q.Q6_K])
def test_one_hot_single_and_batch(dev, fmt):
    import torch
    w = matrix(fmt, synth.seed_of(50, fmt))
    dec = oracle.dequant_rows(fmt, w, ROWS, K)
    M = q.Matrix(dput(w, dev), fmt, ROWS, K)
    pos = positions(fmt)
    xs = unit_vectors(pos)
    xd = dput(xs, dev)
    want = dec[:, pos].T  # (n_pos, ROWS)
    y1 = torch.full((len(pos), ROWS), float("nan"), dtype=torch.float32, device=dev)
    for t in range(len(pos)):
        q.qgemv_rows(M, 0, ROWS, xd[t], y1[t])
    yb = torch.full((len(pos), ROWS), float("nan"), dtype=torch.float32, device=dev)
    q.qgemv_rows_batch(M, 0, ROWS, xd, yb)
    torch.cuda.synchronize()
    for name, y in (("qgemv_rows", y1), ("qgemv_rows_batch", yb)):
        got = y.cpu().numpy()
        bad = np.argwhere(got != want)
        assert bad.size == 0, (f"{name}: {len(bad)} mismatches, first at position {pos[bad[0][0]]} row "
                               f"{bad[0][1]}: {got[tuple(bad[0])]!r} vs {want[tuple(bad[0])]!r}")


@pytest.mark.parametrize("fmt", [q.Q8_0, q.Q4_0, q.MXFP4, q.Q4_K, q.Q6_K])
def test_one_hot_mfma(dev, fmt):
    import torch
    w = matrix(fmt, synth.seed_of(51, fmt))
    dec = oracle.dequant_rows(fmt, w, ROWS, K)
    M = q.Matrix(dput(w, dev), fmt, ROWS, K)
    pos = positions(fmt)
    xs = unit_vectors(pos)
    y = torch.full((len(pos), ROWS), float("nan"), dtype=torch.float32, device=dev)
    q.qgemv_rows_mfma(M, 0, ROWS, dput(xs, dev), y)
    torch.cuda.synchronize()
    got = y.cpu().numpy()
    want = dec[:, pos].T
    bad = np.argwhere(got != want)
    assert bad.size == 0, (f"{len(bad)} mismatches, first at position {pos[bad[0][0]]} row {bad[0][1]}: "
                           f"{got[tuple(bad[0])]!r} vs {want[tuple(bad[0])]!r}")
