"""GPU parity on rows whose weights are all zero, or all zero but a few.

A weight of zero must add exactly zero to its row's sum, so a row of zero
weights returns exactly 0 and a sparse row returns the sum of its few nonzero
products within fp32 rounding of those alone.  The oracle's componentwise gate
(tests/gates.py: |y - r| <= 1e-4 sum |w x|) demands exactly that: for a zero
row its bound is 0.  The zero weights are written in each format's own zero
code: Q4_0 code 8 (w = d (q - 8)), Q6_K code 32 (w = d scale (q - 32)), Q8_0
code 0, MXFP4 codes 0 and 8 (+0 and -0), and Q4_K sub-blocks with sc = m = 0
(the encoding of a constant zero sub-block) -- with finite, nonzero scales, so
only the codes make the weights zero.

Every entry point that runs the fused row dot is covered: qgemv_rows at several
block_rows, qgemv_windows, qgemv_rows_batch, qgemv_rows_op, qgemv_rows_swiglu,
qgemv_expert_windows, qgemv_rows_mfma, the streamer, host-mapped weights and
(for the 32-weight formats) a chain.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import quantized_gemv_gguf_amd as q
import synth
from gates import bits_equal, check

pytestmark = pytest.mark.gpu

FMTS = [q.Q8_0, q.Q4_0, q.MXFP4, q.Q4_K, q.Q6_K]
K_OF = {q.Q8_0: 4096, q.Q4_0: 4096, q.MXFP4: 2880, q.Q4_K: 4096, q.Q6_K: 4096}


def dput(a, dev):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def sync():
    import torch
    torch.cuda.synchronize()


def zero_codes(fmt, blk):
    """Write the format's zero code into every weight of the block array
    blk (n, block bytes), keeping its scale fields."""
    if fmt == q.Q8_0:
        blk[:, 2:] = 0
    elif fmt == q.Q4_0:
        blk[:, 2:] = 0x88
    elif fmt == q.MXFP4:
        blk[:, 1:] = 0x00
    elif fmt == q.Q4_K:
        blk[:, 4:16] = 0  # every sub-block's sc and m
    else:  # Q6_K: low nibbles 0, high bit pairs 2 -> q = 32
        blk[:, 0:128] = 0
        blk[:, 128:192] = 0xAA


def sparse_codes(fmt, blk, rng):
    """A few random payload bytes of each block made nonzero again (each
    changes one or two weights)."""
    n, bb = blk.shape
    lo = {q.Q8_0: 2, q.Q4_0: 2, q.MXFP4: 1, q.Q4_K: 16, q.Q6_K: 0}[fmt]
    hi = {q.Q8_0: 34, q.Q4_0: 18, q.MXFP4: 17, q.Q4_K: 144, q.Q6_K: 128}[fmt]
    for i in range(n):
        for j in rng.choice(np.arange(lo, hi), size=2, replace=False):
            blk[i, j] = rng.integers(0, 256)
    if fmt == q.Q4_K:
        # sub-blocks keep m = 0 (no offset), with nonzero scales sc for s < 4
        blk[:, 4:8] = rng.integers(1, 64, size=(n, 4))


def mixed_matrix(fmt, rows, k, seed):
    """Rows cycle through: zero, sparse, dense (the config generator's)."""
    rng = np.random.default_rng(seed)
    w = synth.blocks(fmt, rows, k, seed)
    bb = synth.BLOCK_BYTES[fmt]
    nb = k // synth.BLOCK_WEIGHTS[fmt]
    v = w.reshape(rows, nb, bb)
    for r in range(rows):
        if r % 3 == 2:
            continue
        blk = v[r].copy()
        zero_codes(fmt, blk)
        if r % 3 == 1:
            sparse_codes(fmt, blk, rng)
        v[r] = blk
    return w


def expect(fmt, w, rows, k, x, r0=0, r1=None):
    r1 = rows if r1 is None else r1
    ref, a = oracle.gemv_rows(fmt, w, rows, k, x, r0, r1)
    zero = np.array([(r % 3 == 0) for r in range(r0, r1)])
    assert np.all(ref[zero] == 0) and np.all(a[zero] == 0), "the oracle's zero rows"
    return ref, a


@pytest.mark.parametrize("fmt", FMTS)
def test_rows_windows(dev, fmt):
    import torch
    rows, k = 96, K_OF[fmt]
    w = mixed_matrix(fmt, rows, k, synth.seed_of(40, fmt))
    x = synth.x_vec(k, synth.seed_of(40, 9))
    ref, a = expect(fmt, w, rows, k, x)
    M = q.Matrix(dput(w, dev), fmt, rows, k)
    xd = dput(x, dev)
    outs = []
    for B in (0, 1, 7, 64):
        y = torch.full((rows,), float("nan"), dtype=torch.float32, device=dev)
        q.qgemv_rows(M, 0, rows, xd, y, B)
        sync()
        outs.append(y.cpu().numpy())
        check(outs[-1], ref, a, what=f"rows B={B}")
        assert np.all(outs[-1][0::3] == 0), "zero rows"
    for o in outs[1:]:
        assert bits_equal(o, outs[0])
    # one grid over windows of the same matrix
    ys = [torch.full((32,), float("nan"), dtype=torch.float32, device=dev) for _ in range(3)]
    q.qgemv_windows([q.Window(M, 32 * i, 32 * i + 32, xd, ys[i]) for i in range(3)])
    sync()
    assert bits_equal(np.concatenate([y.cpu().numpy() for y in ys]), outs[0])


@pytest.mark.parametrize("fmt", FMTS)
def test_batch_and_op(dev, fmt):
    import torch
    rows, k = 60, K_OF[fmt]
    w = mixed_matrix(fmt, rows, k, synth.seed_of(41, fmt))
    xs = np.stack([synth.x_vec(k, synth.seed_of(41, 100 + t)) for t in range(5)])
    M = q.Matrix(dput(w, dev), fmt, rows, k)
    y = torch.full((5, rows), float("nan"), dtype=torch.float32, device=dev)
    q.qgemv_rows_batch(M, 0, rows, dput(xs, dev), y)
    sync()
    yb = y.cpu().numpy()
    for t in range(5):
        ref, a = expect(fmt, w, rows, k, xs[t])
        check(yb[t], ref, a, what=f"batch token {t}")
    # fused RMS at the x-load: the oracle normalises x in fp64
    yo = torch.full((rows,), float("nan"), dtype=torch.float32, device=dev)
    q.qgemv_rows_op(M, 0, rows, dput(xs[0], dev), yo, q.IN_RMS, 1e-6)
    sync()
    xn = oracle.rms_carry(xs[0].astype(np.float64), 1e-6).astype(np.float32)
    ref, a = expect(fmt, w, rows, k, xn)
    got = yo.cpu().numpy()
    assert np.all(got[0::3] == 0)
    # the fp32 normalised x differs from the fp64 one by rounding: 1e-4 covers it
    check(got, ref, a, what="rows_op RMS")


@pytest.mark.parametrize("fmt", FMTS)
def test_swiglu_and_experts(dev, fmt):
    import torch
    E, out, k = 4, 48, K_OF[fmt]
    wg = mixed_matrix(fmt, E * out, k, synth.seed_of(42, fmt))
    wu = mixed_matrix(fmt, E * out, k, synth.seed_of(42, 10 + fmt))
    G, U = q.Matrix(dput(wg, dev), fmt, E * out, k), q.Matrix(dput(wu, dev), fmt, E * out, k)
    x = synth.x_vec(k, synth.seed_of(42, 9))
    xd = dput(x, dev)
    f32 = dict(dtype=torch.float32, device=dev)
    ids = [3, 0, 2]
    gu = torch.full((2 * len(ids) * out,), float("nan"), **f32)
    q.qgemv_expert_windows([G, U], E, ids, xd, 0, gu)
    h = torch.full((E * out,), float("nan"), **f32)
    q.qgemv_rows_swiglu(G, U, 0, E * out, xd, h)
    sync()
    g = gu.cpu().numpy()
    for m, wm in enumerate((wg, wu)):
        for s, e in enumerate(ids):
            ref, a = expect(fmt, wm, E * out, k, x, e * out, (e + 1) * out)
            check(g[(m * len(ids) + s) * out:(m * len(ids) + s + 1) * out], ref, a, what=f"expert {e} mat {m}")
    # silu(gate) * up is exactly 0 wherever gate's or up's row is zero
    hh = h.cpu().numpy()
    assert np.all(hh[0::3] == 0), "SwiGLU of zero rows"


@pytest.mark.parametrize("fmt", FMTS)
def test_mfma(dev, fmt):
    import torch
    rows, k = 96, K_OF[fmt]
    w = mixed_matrix(fmt, rows, k, synth.seed_of(43, fmt))
    xs = np.stack([synth.x_vec(k, synth.seed_of(43, 100 + t)) for t in range(16)])
    M = q.Matrix(dput(w, dev), fmt, rows, k)
    y = torch.full((16, rows), float("nan"), dtype=torch.float32, device=dev)
    q.qgemv_rows_mfma(M, 0, rows, dput(xs, dev), y)
    sync()
    ym = y.cpu().numpy()
    for t in (0, 7, 15):
        ref, a = expect(fmt, w, rows, k, xs[t])
        check(ym[t], ref, a, what=f"mfma token {t}")


@pytest.mark.parametrize("fmt", FMTS)
def test_streamed_and_mapped(dev, fmt):
    import torch
    rows, k = 200, K_OF[fmt]
    w = mixed_matrix(fmt, rows, k, synth.seed_of(44, fmt))
    x = synth.x_vec(k, synth.seed_of(44, 9))
    ref, a = expect(fmt, w, rows, k, x)
    xd = dput(x, dev)
    pin = torch.empty(w.shape, dtype=torch.uint8, pin_memory=True)
    pin.numpy()[...] = w
    P = q.Matrix(pin, fmt, rows, k)
    res = torch.empty(rows, dtype=torch.float32, device=dev)
    q.qgemv_rows(q.Matrix(dput(w, dev), fmt, rows, k), 0, rows, xd, res)
    rb = synth.row_bytes(fmt, k)
    with q.Streamer(32 * rb, 1) as st:
        ys = torch.full((rows,), float("nan"), dtype=torch.float32, device=dev)
        st.rows(P, 0, rows, xd, ys, 32)
        ym = torch.full((rows,), float("nan"), dtype=torch.float32, device=dev)
        q.qgemv_mapped_rows(P, 0, rows, xd, ym, 0)
        sync()
    r = res.cpu().numpy()
    check(r, ref, a, what="resident")
    assert bits_equal(ys.cpu().numpy(), r), "streamed vs resident"
    assert bits_equal(ym.cpu().numpy(), r), "mapped vs resident"


@pytest.mark.parametrize("fmt", [q.Q8_0, q.Q4_0, q.MXFP4])
def test_chain(dev, fmt):
    """Two dependent steps in one chain launch: y1 = W1 x, y2 = W2 rms(y1)."""
    import torch
    k = 2048
    w1 = mixed_matrix(fmt, k, k, synth.seed_of(45, fmt))
    w2 = mixed_matrix(fmt, 300, k, synth.seed_of(45, 10 + fmt))
    M1, M2 = q.Matrix(dput(w1, dev), fmt, k, k), q.Matrix(dput(w2, dev), fmt, 300, k)
    x = synth.x_vec(k, synth.seed_of(45, 9))
    xd = dput(x, dev)
    f32 = dict(dtype=torch.float32, device=dev)
    y1, y2 = torch.full((k,), float("nan"), **f32), torch.full((300,), float("nan"), **f32)
    steps = [q.ChainStep([q.ChainWindow(M1, 0, k, xd, y1)], q.IN_X),
             q.ChainStep([q.ChainWindow(M2, 0, 300, y1, y2)], q.IN_RMS, 1e-6)]
    with q.Chain(fmt, steps) as c:
        c.run()
        c.check()
        sync()
        g1, g2 = y1.cpu().numpy(), y2.cpu().numpy()
    ref, a = expect(fmt, w1, k, k, x)
    check(g1, ref, a, what="chain step 0")
    xn = oracle.rms_carry(g1.astype(np.float64), 1e-6).astype(np.float32)
    ref, a = expect(fmt, w2, 300, k, xn)
    check(g2, ref, a, what="chain step 1 (teacher-forced)")
