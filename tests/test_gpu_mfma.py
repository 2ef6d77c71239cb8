"""GPU parity for qgemv_rows_mfma: up to 16 tokens per pass on the fp32 matrix
cores.

The matrix cores add in their own order, so the results are checked against
the oracle's gates (normwise and componentwise, 1e-4) for every token, not for
bit identity with the one-token kernels; windows, strides, row and k tails,
token counts that are not a multiple of 16, and the no-op and error cases as
for qgemv_rows_batch.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import quantized_gemv_gguf_amd as q
import synth
from gates import check

pytestmark = pytest.mark.gpu


def dput(a, dev):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def sync():
    import torch
    torch.cuda.synchronize()


# (format, rows, k): whole and ragged 32-row workgroup tiles; the LDS-staged
# kernel with one chunk (Q8_0 k = 256), whole chunks, and a last chunk moved
# back over its predecessor (Q8_0 and Q4_0 k = 2080, MXFP4 k = 2880); the
# register kernel below one chunk (Q8_0 k = 96, Q4_0 k = 480, MXFP4 k = 32);
# Q4_K with one, 24 and 11 super-blocks per row; Q6_K (register kernel) with
# 96, one and 11
SHAPES = [(q.Q8_0, 300, 6144), (q.Q8_0, 17, 24576), (q.Q8_0, 64, 256), (q.Q8_0, 50, 2080), (q.Q8_0, 5, 96),
          (q.Q4_0, 257, 4096), (q.Q4_0, 33, 2080), (q.Q4_0, 20, 480), (q.MXFP4, 200, 2880), (q.MXFP4, 16, 32),
          (q.Q4_K, 130, 6144), (q.Q4_K, 33, 256), (q.Q4_K, 70, 2816),
          (q.Q6_K, 71, 24576), (q.Q6_K, 40, 256), (q.Q6_K, 33, 2816)]


def oracle_tokens(fmt, w, rows, k, xs):
    refs, abss = [], []
    for x in xs:
        r, a = oracle.gemv_rows(fmt, w, rows, k, x)
        refs.append(r)
        abss.append(a)
    return np.stack(refs), np.stack(abss)


@pytest.mark.parametrize("fmt,rows,k", SHAPES)
def test_mfma_against_oracle(dev, fmt, rows, k):
    import torch
    w = synth.blocks(fmt, rows, k, synth.seed_of(31, fmt))
    M = q.Matrix(dput(w, dev), fmt, rows, k)
    xs = np.stack([synth.x_vec(k, synth.seed_of(31, 100 + t)) for t in range(33)])
    ref, a = oracle_tokens(fmt, w, rows, k, xs)
    for n_tok in (1, 3, 16, 17, 33):
        y = torch.full((n_tok, rows), float("nan"), dtype=torch.float32, device=dev)
        q.qgemv_rows_mfma(M, 0, rows, dput(xs[:n_tok], dev), y)
        sync()
        got = y.cpu().numpy()
        for t in range(n_tok):
            check(got[t], ref[t], a[t], what=f"n_tok {n_tok} token {t}")


@pytest.mark.parametrize("fmt,rows,k", [(q.Q8_0, 700, 4096), (q.MXFP4, 401, 2880)])
def test_mfma_windows_and_strides(dev, fmt, rows, k):
    """A row window with padded x and y strides: every token within the gates,
    nothing written past a token's outputs."""
    import torch
    w = synth.blocks(fmt, rows, k, synth.seed_of(31, 20 + fmt))
    M = q.Matrix(dput(w, dev), fmt, rows, k)
    n_tok, r0, r1 = 6, 17, rows - 5
    xs = np.stack([synth.x_vec(k, synth.seed_of(31, 200 + t)) for t in range(n_tok)])
    ref, a = oracle_tokens(fmt, w, rows, k, xs)
    xpad = np.zeros((n_tok, k + 40), np.float32)
    xpad[:, :k] = xs
    ybuf = torch.full((n_tok, (r1 - r0) + 9), float("nan"), dtype=torch.float32, device=dev)
    q.qgemv_rows_mfma(M, r0, r1, dput(xpad, dev), ybuf)
    sync()
    got = ybuf.cpu().numpy()
    assert np.all(np.isnan(got[:, r1 - r0:])), "wrote past a token's outputs"
    for t in range(n_tok):
        check(got[t, :r1 - r0], ref[t, r0:r1], a[t, r0:r1], what=f"token {t}")


def test_mfma_matches_batch_within_gates(dev):
    """The matrix-core and the bit-exact several-token paths agree to the
    oracle's tolerance on the same inputs."""
    import torch
    fmt, rows, k = q.Q8_0, 160, 6144
    w = synth.blocks(fmt, rows, k, synth.seed_of(31, 40))
    M = q.Matrix(dput(w, dev), fmt, rows, k)
    xs = np.stack([synth.x_vec(k, synth.seed_of(31, 300 + t)) for t in range(16)])
    _, a = oracle_tokens(fmt, w, rows, k, xs)
    y1 = torch.empty((16, rows), dtype=torch.float32, device=dev)
    y2 = torch.empty((16, rows), dtype=torch.float32, device=dev)
    X = dput(xs, dev)
    q.qgemv_rows_mfma(M, 0, rows, X, y1)
    q.qgemv_rows_batch(M, 0, rows, X, y2)
    sync()
    for t in range(16):
        check(y1[t].cpu().numpy(), y2[t].cpu().numpy(), a[t], what=f"token {t}")


def test_mfma_special_values(dev):
    """NaN scales (MXFP4 e = 255) make exactly their rows NaN; rows of
    fp32-subnormal weights (e = 0) pass the gates like any other; Q8_0
    zero-scale rows give exact zeros; the largest fp16 scale stays finite and
    within the gates."""
    import torch
    k = 512
    w = synth.blocks(q.MXFP4, 48, k, synth.seed_of(31, 50)).reshape(48, -1)
    w[5, 17 * 3] = 255  # the scale byte of row 5's block 3
    w[20, ::17] = 0     # row 20: every block at e = 0 (2^-127, subnormal weights)
    M = q.Matrix(dput(w.reshape(-1), dev), q.MXFP4, 48, k)
    xs = np.stack([synth.x_vec(k, synth.seed_of(31, 400 + t)) for t in range(4)])
    y = torch.empty((4, 48), dtype=torch.float32, device=dev)
    q.qgemv_rows_mfma(M, 0, 48, dput(xs, dev), y)
    sync()
    got = y.cpu().numpy()
    assert np.all(np.isnan(got[:, 5]))
    assert np.all(np.isfinite(np.delete(got, 5, axis=1)))
    ref, a = oracle_tokens(q.MXFP4, w.reshape(-1), 48, k, xs)
    keep = [r for r in range(48) if r != 5]
    for t in range(4):
        check(got[t, keep], ref[t, keep], a[t, keep], what=f"token {t}")
        # row 20: fp32-subnormal weights, which the matrix cores must not flush
        check(got[t, 20:21], ref[t, 20:21], a[t, 20:21], what=f"subnormal row, token {t}")

    w8 = synth.blocks(q.Q8_0, 32, k, synth.seed_of(31, 51)).reshape(32, -1)
    w8[3, 0::34] = 0; w8[3, 1::34] = 0          # row 3: d = 0
    w8[9, 0::34] = 0xff; w8[9, 1::34] = 0x7b    # row 9: d = 65504, the largest fp16
    M8 = q.Matrix(dput(w8.reshape(-1), dev), q.Q8_0, 32, k)
    y8 = torch.empty((4, 32), dtype=torch.float32, device=dev)
    q.qgemv_rows_mfma(M8, 0, 32, dput(xs, dev), y8)
    sync()
    got8 = y8.cpu().numpy()
    assert np.all(got8[:, 3] == 0.0)
    ref8, a8 = oracle_tokens(q.Q8_0, w8.reshape(-1), 32, k, xs)
    for t in range(4):
        check(got8[t], ref8[t], a8[t], what=f"Q8_0 token {t}")


def test_mfma_noops_and_errors(dev):
    import torch
    fmt, rows, k = q.Q8_0, 40, 256
    w = synth.blocks(fmt, rows, k, synth.seed_of(31, 60))
    M = q.Matrix(dput(w, dev), fmt, rows, k)
    y = torch.full((2, rows), 7.0, dtype=torch.float32, device=dev)
    x = dput(np.ones((2, k), np.float32), dev)
    q.qgemv_rows_mfma(M, 10, 10, x, y)               # empty window
    q.qgemv_rows_mfma(M, 0, rows, x[:0], y[:0])      # no tokens
    sync()
    assert np.all(y.cpu().numpy() == 7.0)
    y2 = torch.empty((2, rows + 1), dtype=torch.float32, device=dev)
    with pytest.raises(q.QgemvError):
        q.qgemv_rows_mfma(M, 0, rows + 1, x, y2)


@pytest.mark.parametrize("fmt", [q.Q8_0, q.Q4_0, q.MXFP4])
def test_mfma_largest_k_single_row_and_shared_x(dev, fmt):
    """k = QG_MAX_K (49152; 1536 blocks, the last Q4_0/MXFP4 chunk whole,
    Q8_0's 192 chunks over 8 waves), a one-row window (31 clamped rows in its
    tile), and x_stride = 0: every token reads the same x, so the 16 results
    of a row are the same sums and must agree to the gates with the oracle."""
    import torch
    k, rows = 49152, 40
    w = synth.blocks(fmt, rows, k, synth.seed_of(31, 70 + fmt))
    M = q.Matrix(dput(w, dev), fmt, rows, k)
    xs = np.stack([synth.x_vec(k, synth.seed_of(31, 500 + t)) for t in range(16)])
    ref, a = oracle_tokens(fmt, w, rows, k, xs)
    y = torch.full((16, rows), float("nan"), dtype=torch.float32, device=dev)
    q.qgemv_rows_mfma(M, 0, rows, dput(xs, dev), y)
    y1 = torch.full((16, 1), float("nan"), dtype=torch.float32, device=dev)
    q.qgemv_rows_mfma(M, 23, 24, dput(xs, dev), y1)
    X0 = dput(xs[:1], dev)
    ys = torch.full((16, rows), float("nan"), dtype=torch.float32, device=dev)
    import ctypes
    m = M.c()
    rc = q.lib().qgemv_rows_mfma(ctypes.byref(m), 0, rows, X0.data_ptr(), 0, 16, ys.data_ptr(), rows, None)
    assert rc == 0
    sync()
    got, got1, gots = y.cpu().numpy(), y1.cpu().numpy(), ys.cpu().numpy()
    for t in range(16):
        check(got[t], ref[t], a[t], what=f"token {t}")
        check(got1[t], ref[t, 23:24], a[t, 23:24], what=f"one row, token {t}")
        check(gots[t], ref[0], a[0], what=f"shared x, token {t}")
    # the same x and the same launch give the same sums for every token
    assert np.array_equal(gots, np.broadcast_to(gots[0], gots.shape))
