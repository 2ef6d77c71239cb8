"""GPU parity for qgemv_rows_batch: several tokens per pass over the weights.

Each token's y must have the bits of a one-token qgemv_rows call on its own x
(the per-row order does not depend on the batch), and pass the oracle's gates.
"""
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


# (format, rows, k): one column per lane at 3, 8 and 12 waves, two columns,
# and the single-token fallback above k = 32768
SHAPES = [(q.Q8_0, 300, 6144), (q.Q8_0, 97, 16384), (q.Q8_0, 65, 24576), (q.Q4_0, 257, 4096),
          (q.MXFP4, 200, 2880), (q.Q4_K, 130, 6144), (q.Q6_K, 71, 24576), (q.Q8_0, 40, 32768),
          (q.Q4_0, 33, 49152), (q.Q8_0, 9, 96)]


def singles(dev, M, rows, xs, r0, r1):
    import torch
    out = []
    for x in xs:
        y = torch.full((r1 - r0,), float("nan"), dtype=torch.float32, device=dev)
        q.qgemv_rows(M, r0, r1, dput(x, dev), y)
        out.append(y)
    sync()
    return np.stack([y.cpu().numpy() for y in out]) if out else np.empty((0, r1 - r0), np.float32)


@pytest.mark.parametrize("fmt,rows,k", SHAPES)
def test_batch_equals_single_tokens(dev, fmt, rows, k):
    import torch
    w = synth.blocks(fmt, rows, k, synth.seed_of(9, fmt))
    M = q.Matrix(dput(w, dev), fmt, rows, k)
    xs = np.stack([synth.x_vec(k, synth.seed_of(9, 100 + t)) for t in range(16)])
    ref = singles(dev, M, rows, xs, 0, rows)
    for n_tok in (1, 2, 3, 4, 5, 7, 8, 16):
        y = torch.full((n_tok, rows), float("nan"), dtype=torch.float32, device=dev)
        q.qgemv_rows_batch(M, 0, rows, dput(xs[:n_tok], dev), y)
        sync()
        assert bits_equal(y.cpu().numpy(), ref[:n_tok]), f"n_tok {n_tok}"
    for t in (0, 5, 15):
        r, a = oracle.gemv_rows(fmt, w, rows, k, xs[t])
        check(ref[t], r, a, what=f"token {t}")


@pytest.mark.parametrize("fmt,rows,k", [(q.Q8_0, 700, 4096), (q.Q4_K, 333, 2816), (q.MXFP4, 401, 2880)])
def test_batch_windows_strides_and_block_rows(dev, fmt, rows, k):
    """Padded strides, a window, row blocks: the same bits as single calls,
    and nothing written between the outputs."""
    import torch
    w = synth.blocks(fmt, rows, k, synth.seed_of(9, 20 + fmt))
    M = q.Matrix(dput(w, dev), fmt, rows, k)
    n_tok, r0, r1 = 6, 17, rows - 5
    xs = np.stack([synth.x_vec(k, synth.seed_of(9, 200 + t)) for t in range(n_tok)])
    ref = singles(dev, M, rows, xs, r0, r1)
    xpad = np.zeros((n_tok, k + 40), np.float32)
    xpad[:, :k] = xs
    for B in (0, 1, 7, 128):
        ybuf = torch.full((n_tok, (r1 - r0) + 9), float("nan"), dtype=torch.float32, device=dev)
        q.qgemv_rows_batch(M, r0, r1, dput(xpad, dev), ybuf, block_rows=B)
        sync()
        got = ybuf.cpu().numpy()
        assert bits_equal(got[:, :r1 - r0], ref), f"block_rows {B}"
        assert np.isnan(got[:, r1 - r0:]).all(), "wrote between outputs"


def test_batch_degenerate(dev):
    import torch
    fmt, rows, k = q.Q8_0, 64, 1024
    w = synth.blocks(fmt, rows, k, 3)
    M = q.Matrix(dput(w, dev), fmt, rows, k)
    y = torch.full((0, rows), float("nan"), dtype=torch.float32, device=dev)
    q.qgemv_rows_batch(M, 0, rows, torch.zeros((0, k), dtype=torch.float32, device=dev), y)
    y = torch.full((3, 5), float("nan"), dtype=torch.float32, device=dev)
    q.qgemv_rows_batch(M, 10, 10, torch.zeros((3, k), dtype=torch.float32, device=dev), y)
    sync()
    assert np.isnan(y.cpu().numpy()).all()
    # identical tokens give identical rows; a zero token gives zeros
    x = synth.x_vec(k, 4)
    xs = np.stack([x, x, np.zeros(k, np.float32), x])
    y = torch.empty((4, rows), dtype=torch.float32, device=dev)
    q.qgemv_rows_batch(M, 0, rows, dput(xs, dev), y)
    sync()
    yh = y.cpu().numpy()
    assert bits_equal(yh[0], yh[1]) and bits_equal(yh[0], yh[3]) and np.all(yh[2] == 0)
