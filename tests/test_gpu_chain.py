"""GPU: chains (qgemv_chain_*) -- dependent GEMVs in one persistent launch.

Bars:
  * every step's y is bit-identical to the same step run as separate calls
    (qgemv_rms_carry / qgemv_silu_mul, then qgemv_rows / qgemv_expert_windows):
    the chain changes when rows are computed, never how;
  * every step's y passes the oracle gates of tests/gates.py, teacher-forced:
    the oracle applies the step's transform in fp64 to the GPU's own input
    vector and multiplies in fp64;
  * repeated runs give identical bits and the barrier reports no time-out.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import quantized_gemv_gguf_amd as q
import synth
from gates import bits_equal, check

pytestmark = pytest.mark.gpu

EPS = 1e-6


def dput(a, dev):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def host(t):
    return t.cpu().numpy()


class Dense:
    """L layers of {QKV 3H x H, out H x H, up F x H, down H x F}; step inputs as
    in the synthetic decode pass: rms(x0), rms(V third of qkv), rms(out),
    rms(gelu(up)), then rms(down) into the next layer."""

    def __init__(self, dev, fmt, H, F, L, seed):
        import torch
        self.fmt, self.H, self.F, self.L = fmt, H, F, L
        shapes = [(3 * H, H), (H, H), (F, H), (H, F)]
        self.w, self.wd, self.y = [], [], []
        for l in range(L):
            for m, (rows, k) in enumerate(shapes):
                w = synth.blocks(fmt, rows, k, seed=seed + 4 * l + m)
                self.w.append((w, rows, k))
                self.wd.append(q.Matrix(dput(w, dev), fmt, rows, k))
                self.y.append(torch.full((rows,), float("nan"), dtype=torch.float32, device=dev))
        self.x0 = dput(synth.x_vec(H, seed + 999), dev)

    def source(self, s):
        """(input vector, transform) of step s."""
        H, m = self.H, s % 4
        if s == 0:
            return self.x0, q.IN_RMS
        if m == 1:
            return self.y[s - 1][2 * H:3 * H], q.IN_RMS
        return self.y[s - 1], (q.IN_GELU_RMS if m == 3 else q.IN_RMS)

    def steps(self, ys=None):
        ys = self.y if ys is None else ys
        out = []
        for s, W in enumerate(self.wd):
            x, op = self.source(s)
            out.append(q.ChainStep([q.ChainWindow(W, 0, W.n_rows, x, ys[s])], op, EPS))
        return out


def separate(dense, dev):
    """The same pass as separate calls: carry kernel, then qgemv_rows."""
    import torch
    ys = [torch.full_like(y, float("nan")) for y in dense.y]
    for s, W in enumerate(dense.wd):
        x, op = dense.source(s)
        if s > 0:  # read the separate run's own previous outputs
            if s % 4 == 1:
                x = ys[s - 1][2 * dense.H:3 * dense.H]
            else:
                x = ys[s - 1]
        c = torch.empty(W.k, dtype=torch.float32, device=dev)
        q.qgemv_rms_carry(x, c, EPS, gelu=(op == q.IN_GELU_RMS))
        q.qgemv_rows(W, 0, W.n_rows, c, ys[s])
    torch.cuda.synchronize()
    return ys


def teacher_forced(dense, s, y):
    x, op = dense.source(s)
    c = oracle.rms_carry(host(x).astype(np.float64), EPS, gelu=(op == q.IN_GELU_RMS))
    w, rows, k = dense.w[s]
    ref, a = oracle.gemv_rows(dense.fmt, w, rows, k, c)
    check(host(y), ref, a, what=f"step {s}")


@pytest.mark.parametrize("fmt", [q.Q8_0, q.Q4_0, q.MXFP4])
@pytest.mark.parametrize("H,F,L", [(3072, 8192, 2), (1024, 24576, 1), (3072, 14336, 2)])
def test_dense_chain_matches_separate_calls_and_oracle(dev, fmt, H, F, L):
    """Team shapes covered: k = 1024 (1 wave, 12 teams per workgroup), 3072
    (2 waves), 8192 (4 waves), 24576 (12 waves, the whole workgroup), and for
    Q8_0 k = 14336 (one team of 7 waves, 5 idle: the step after it reads its
    output with every wave busy)."""
    import torch
    d = Dense(dev, fmt, H, F, L, seed=7000 + 10 * fmt)
    with q.Chain(fmt, d.steps()) as ch:
        assert ch.grid >= 1
        ch.run()
        ch.check()
        ys = separate(d, dev)
        for s in range(4 * L):
            assert bits_equal(host(d.y[s]), host(ys[s])), f"step {s} differs from the separate calls"
            teacher_forced(d, s, d.y[s])
        # a second and third run reproduce the first bit for bit
        first = [host(y) for y in d.y]
        for _ in range(2):
            for y in d.y:
                y.fill_(float("nan"))
            ch.run()
            ch.check()
            for s in range(4 * L):
                assert bits_equal(host(d.y[s]), first[s])
    torch.cuda.synchronize()


def test_dense_chain_full_size_layer(dev):
    """One layer of the 20B-class Q8_0 pass at its real shape (H 6144, F 24576),
    the configuration the benchmark runs, checked on sampled rows."""
    d = Dense(dev, q.Q8_0, 6144, 24576, 1, seed=9100)
    with q.Chain(q.Q8_0, d.steps()) as ch:
        ch.run()
        ch.check()
    ys = separate(d, dev)
    rng = np.random.default_rng(5)
    for s in range(4):
        assert bits_equal(host(d.y[s]), host(ys[s]))
        x, op = d.source(s)
        c = oracle.rms_carry(host(x).astype(np.float64), EPS, gelu=(op == q.IN_GELU_RMS))
        w, rows, k = d.w[s]
        sel = np.sort(rng.choice(rows, 64, replace=False))
        ref, a = np.empty(len(sel)), np.empty(len(sel))
        for j, r in enumerate(sel):
            rr, aa = oracle.gemv_rows(q.Q8_0, w, rows, k, c, int(r), int(r) + 1)
            ref[j], a[j] = rr[0], aa[0]
        check(host(d.y[s])[sel], ref, a, what=f"step {s}, 64 sampled rows")


def test_moe_chain_matches_expert_windows(dev):
    """Two tokens of a routed MXFP4 expert FFN as one chain: gate/up windows of
    the selected experts (shared x), then down windows with SiLU(gate) * up
    applied per expert as x is loaded; against qgemv_expert_windows +
    qgemv_silu_mul + qgemv_expert_windows, and the oracle."""
    import torch
    E, out, k, n_sel = 16, 2880, 2880, 4
    fmt = q.MXFP4
    ws = [synth.blocks(fmt, E * out, k, seed=8200 + m) for m in range(3)]
    W = [q.Matrix(dput(w, dev), fmt, E * out, k) for w in ws]
    rng = np.random.default_rng(3)
    tokens = []
    steps = []
    for t in range(2):
        ids = sorted(rng.choice(E, n_sel, replace=False).tolist())
        x = dput(synth.x_vec(k, 8300 + t), dev)
        gu = torch.full((2 * n_sel * out,), float("nan"), dtype=torch.float32, device=dev)
        yd = torch.full((n_sel * out,), float("nan"), dtype=torch.float32, device=dev)
        wins = []
        for m in range(2):
            for s, e in enumerate(ids):
                wins.append(q.ChainWindow(W[m], e * out, (e + 1) * out, x, gu[(m * n_sel + s) * out:][:out]))
        steps.append(q.ChainStep(wins, q.IN_X))
        wins = [q.ChainWindow(W[2], e * out, (e + 1) * out, gu[s * out:][:out], yd[s * out:][:out],
                              x2=gu[(n_sel + s) * out:][:out]) for s, e in enumerate(ids)]
        steps.append(q.ChainStep(wins, q.IN_SILU_MUL))
        tokens.append((ids, x, gu, yd))
    with q.Chain(fmt, steps) as ch:
        ch.run()
        ch.check()
    for ids, x, gu, yd in tokens:
        gu2 = torch.full_like(gu, float("nan"))
        yd2 = torch.full_like(yd, float("nan"))
        h = torch.empty(n_sel * out, dtype=torch.float32, device=dev)
        q.qgemv_expert_windows(W[:2], E, ids, x, 0, gu2)
        q.qgemv_silu_mul(gu2[:n_sel * out], gu2[n_sel * out:], h)
        q.qgemv_expert_windows(W[2:], E, ids, h, out, yd2)
        torch.cuda.synchronize()
        assert bits_equal(host(gu), host(gu2))
        assert bits_equal(host(yd), host(yd2))
        xh, g = host(x).astype(np.float64), host(gu).astype(np.float64)
        for s, e in enumerate(ids):
            for m in range(2):
                ref, a = oracle.gemv_rows(fmt, ws[m], E * out, k, xh, e * out, (e + 1) * out)
                check(g[(m * n_sel + s) * out:][:out], ref, a, what=f"gate/up {m} expert {e}")
            hh = oracle.silu_mul(g[s * out:][:out], g[(n_sel + s) * out:][:out])
            ref, a = oracle.gemv_rows(fmt, ws[2], E * out, k, hh, e * out, (e + 1) * out)
            check(host(yd)[s * out:][:out], ref, a, what=f"down expert {e}")


@pytest.mark.parametrize("fmt", [q.Q8_0, q.Q4_0, q.MXFP4])
def test_chain_edges(dev, fmt):
    """Ragged and degenerate steps: k = 32 (one block per row), k = 2080 (65
    blocks: a second wave with one block), single-row and empty windows, a step
    with fewer tiles than the grid has teams, windows sharing one matrix, and
    many short steps; against separate calls and the oracle."""
    import torch
    rng = np.random.default_rng(fmt)
    plan = [  # (k, [(rows, r0, r1), ...], op)
        (32, [(40, 0, 40)], q.IN_X),
        (2080, [(7, 0, 7), (7, 3, 3), (300, 299, 300)], q.IN_X),
        (4096, [(1, 0, 1)], q.IN_X),
        (2080, [(513, 0, 513), (513, 100, 101)], q.IN_X),
        (24576, [(37, 5, 36)], q.IN_X),
        (32, [(3, 0, 3)], q.IN_X),
    ] * 3
    steps, expect = [], []
    for i, (k, wins, op) in enumerate(plan):
        x = dput(synth.x_vec(k, 600 + i), dev)
        cw, ex = [], []
        for j, (rows, r0, r1) in enumerate(wins):
            w = synth.blocks(fmt, rows, k, seed=int(rng.integers(1 << 30)))
            W = q.Matrix(dput(w, dev), fmt, rows, k)
            y = torch.full((max(r1 - r0, 0) + 2,), float("nan"), dtype=torch.float32, device=dev)
            cw.append(q.ChainWindow(W, r0, r1, x, y[1:1 + r1 - r0]))
            ex.append((w, W, rows, k, r0, r1, x, y))
        steps.append(q.ChainStep(cw, op))
        expect.append(ex)
    with q.Chain(fmt, steps) as ch:
        for rep in range(2):
            ch.run()
            ch.check()
            for ex in expect:
                for w, W, rows, k, r0, r1, x, y in ex:
                    yh = host(y)
                    assert np.isnan(yh[0]) and np.isnan(yh[-1]), "write outside the window"
                    y2 = torch.full((max(r1 - r0, 1),), float("nan"), dtype=torch.float32, device=dev)
                    q.qgemv_rows(W, r0, r1, x, y2[:r1 - r0])
                    torch.cuda.synchronize()
                    assert bits_equal(yh[1:1 + r1 - r0], host(y2)[:r1 - r0])
                    if rep == 0 and r1 > r0:
                        ref, a = oracle.gemv_rows(fmt, w, rows, k, host(x).astype(np.float64), r0, r1)
                        check(yh[1:1 + r1 - r0], ref, a, what=f"k {k} rows {r0}:{r1}")


def test_chain_many_steps_and_silu(dev):
    """120 dependent steps alternating the four transforms on small vectors:
    the barrier runs 119 times per launch and carries its state between runs."""
    import torch
    fmt, n = q.Q8_0, 256
    w = synth.blocks(fmt, 2 * n, n, seed=77)
    W = q.Matrix(dput(w, dev), fmt, 2 * n, n)
    ys = [torch.full((2 * n,), float("nan"), dtype=torch.float32, device=dev) for _ in range(120)]
    x0 = dput(synth.x_vec(2 * n, 78), dev)
    ops = [q.IN_RMS, q.IN_GELU_RMS, q.IN_SILU_MUL, q.IN_X]
    steps = []
    for s in range(120):
        src = x0 if s == 0 else ys[s - 1]
        op = ops[s % 4]
        x, x2 = src[:n], (src[n:] if op == q.IN_SILU_MUL else None)
        steps.append(q.ChainStep([q.ChainWindow(W, 0, 2 * n, x, ys[s], x2=x2)], op, EPS))
    with q.Chain(fmt, steps) as ch:
        for _ in range(3):
            ch.run()
        ch.check()
    ref = [torch.full_like(y, float("nan")) for y in ys]
    c = torch.empty(n, dtype=torch.float32, device=dev)
    for s in range(120):
        src = x0 if s == 0 else ref[s - 1]
        op = ops[s % 4]
        if op == q.IN_X:
            c.copy_(src[:n])
        elif op == q.IN_SILU_MUL:
            q.qgemv_silu_mul(src[:n], src[n:], c)
        else:
            q.qgemv_rms_carry(src[:n], c, EPS, gelu=(op == q.IN_GELU_RMS))
        q.qgemv_rows(W, 0, 2 * n, c, ref[s])
    torch.cuda.synchronize()
    for s in range(120):
        assert bits_equal(host(ys[s]), host(ref[s])), f"step {s}"


def test_chain_barrier_failure_is_reported_and_reset(dev):
    """A barrier that gives up (forced from the host: a spin limit of one poll,
    far below the time a device-wide barrier takes) lets the run finish with
    undefined outputs; once the host can see the failure, run enqueues nothing
    and reports QG_E_BARRIER until check resets the state; after that, runs
    are correct again."""
    import torch
    dense = Dense(dev, q.Q8_0, 1024, 2048, 2, seed=8100)
    with q.Chain(q.Q8_0, dense.steps()) as c:
        c.run()
        c.check()
        torch.cuda.synchronize()
        good = [y.cpu().numpy().copy() for y in dense.y]
        c.set_spin_limit(1)
        c.run()
        torch.cuda.synchronize()
        with pytest.raises(q.QgemvError) as e:
            c.run()
        assert e.value.status == -9
        with pytest.raises(q.QgemvError) as e:
            c.check()
        assert e.value.status == -9
        c.set_spin_limit(1 << 22)
        for y in dense.y:
            y.fill_(float("nan"))
        c.run()
        c.check()
        torch.cuda.synchronize()
        for s, y in enumerate(dense.y):
            assert bits_equal(y.cpu().numpy(), good[s]), f"step {s}"
