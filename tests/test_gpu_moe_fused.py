"""GPU parity for the fused MoE token: the down grid taking silu(gate) * up as
it loads it (qgemv_expert_windows_op), the RMS-normalised input fused into the
gate/up grid, and the router-weighted combine (qgemv_combine), at the MXFP4
128 x 2880 x 2880 top-4 workload's full size and on the K-quants."""
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


@pytest.fixture(scope="module")
def moe(dev):
    c = synth.CONFIGS[4]
    E, out, k = c["n_expert"], c["out"], c["k"]
    host = [synth.blocks(q.MXFP4, E * out, k, synth.seed_of(4, t)) for t in range(3)]
    mats = [q.Matrix(dput(h, dev), q.MXFP4, E * out, k) for h in host]
    ids = synth.expert_ids(E, c["n_sel"], c["tokens"], synth.seed_of(4, 8))
    w = synth.router_weights(c["tokens"], c["n_sel"], synth.seed_of(4, 9))
    return dict(fmt=q.MXFP4, E=E, out=out, k=k, host=host, mats=mats, ids=ids, w=w)


def separate(dev, m, x, ids, in_rms=False):
    """The unfused token: (rms), gate/up grid, silu_mul, down grid."""
    import torch
    n_sel, out, k = len(ids), m["out"], m["k"]
    f32 = dict(dtype=torch.float32, device=dev)
    xd = dput(x, dev)
    if in_rms:
        t = torch.empty(k, **f32)
        q.qgemv_rms_carry(xd, t, 1e-6, False)
        xd = t
    gu = torch.empty(2 * n_sel * out, **f32)
    h = torch.empty(n_sel * out, **f32)
    y = torch.empty(n_sel * out, **f32)
    q.qgemv_expert_windows(m["mats"][:2], m["E"], ids, xd, 0, gu)
    q.qgemv_silu_mul(gu[:n_sel * out], gu[n_sel * out:], h)
    q.qgemv_expert_windows(m["mats"][2:], m["E"], ids, h, out, y)
    sync()
    return gu.cpu().numpy(), y.cpu().numpy()


def fused(dev, m, x, ids, in_rms=False, block_rows=0):
    """gate/up grid (RMS at load if asked), down grid with SiLU*up at load."""
    import torch
    n_sel, out = len(ids), m["out"]
    f32 = dict(dtype=torch.float32, device=dev)
    gu = torch.empty(2 * n_sel * out, **f32)
    y = torch.full((n_sel * out,), float("nan"), **f32)
    q.qgemv_expert_windows_op(m["mats"][:2], m["E"], ids, dput(x, dev), 0, gu, q.IN_RMS if in_rms else q.IN_X,
                              1e-6, q.OUT_Y, block_rows=block_rows)
    q.qgemv_expert_windows_op(m["mats"][2:], m["E"], ids, gu[:n_sel * out], out, y, q.IN_SILU_MUL, 0.0, q.OUT_Y,
                              x2=gu[n_sel * out:], block_rows=block_rows)
    sync()
    return gu.cpu().numpy(), y.cpu().numpy()


@pytest.mark.parametrize("token", [0, 17, 63])
def test_fused_token_equals_separate(dev, moe, token):
    ids = [int(v) for v in moe["ids"][token]]
    x = synth.x_vec(moe["k"], synth.seed_of(4, 100 + token))
    for in_rms in (False, True):
        gu_s, y_s = separate(dev, moe, x, ids, in_rms)
        for B in (0, 128):
            gu_f, y_f = fused(dev, moe, x, ids, in_rms, B)
            assert bits_equal(gu_f, gu_s) and bits_equal(y_f, y_s), f"rms {in_rms} block_rows {B}"


def test_combine_against_oracle(dev, moe):
    import torch
    token = 5
    ids = [int(v) for v in moe["ids"][token]]
    n_sel, out = len(ids), moe["out"]
    x = synth.x_vec(moe["k"], synth.seed_of(4, 100 + token))
    _, y = fused(dev, moe, x, ids)
    w = moe["w"][token]
    o = torch.full((out + 3,), float("nan"), dtype=torch.float32, device=dev)
    q.qgemv_combine(dput(y, dev), out, n_sel, dput(w, dev), out, o[:out])
    sync()
    got = o.cpu().numpy()
    assert np.isnan(got[out:]).all()
    ye = y.reshape(n_sel, out).astype(np.float64)
    ref = oracle.combine(ye, w)
    a = np.abs(w.astype(np.float64)[:, None] * ye).sum(axis=0)
    # n_sel fp32 fmas: at most n_sel roundings of at most 2^-24 of the running sum
    assert np.all(np.abs(got[:out] - ref) <= n_sel * 2.0 ** -24 * a + 1e-30)
    # the down projection of each expert against the oracle (teacher-forced input)
    gu, _ = separate(dev, moe, x, ids)
    h = oracle.silu_mul(gu[:n_sel * out], gu[n_sel * out:]).astype(np.float32)
    for s, e in enumerate(ids):
        r, a2 = oracle.gemv_rows(moe["fmt"], moe["host"][2], moe["E"] * out, moe["k"], h[s * out:(s + 1) * out],
                                 e * out, (e + 1) * out)
        check(y[s * out:(s + 1) * out], r, a2, what=f"down expert {e}")


def test_combine_degenerate(dev):
    import torch
    n = 100
    y = dput(np.arange(3 * n, dtype=np.float32), dev)
    o = torch.full((n,), float("nan"), dtype=torch.float32, device=dev)
    q.qgemv_combine(y, n, 0, dput(np.zeros(1, np.float32), dev), n, o)
    sync()
    assert np.all(o.cpu().numpy() == 0)
    q.qgemv_combine(y, n, 3, dput(np.array([0, 1, 0], np.float32), dev), n, o)
    sync()
    assert np.array_equal(o.cpu().numpy(), np.arange(n, 2 * n, dtype=np.float32))


@pytest.mark.parametrize("fmt", [q.Q8_0, q.Q4_K, q.Q6_K])
def test_fused_experts_other_formats(dev, fmt):
    """(16 experts, 512, 1024) stacks of other formats: fused down grid equals
    the separate calls."""
    E, out, k = 16, 512, 1024
    host = [synth.blocks(fmt, E * out, k, synth.seed_of(11, 10 * fmt + t)) for t in range(2)]
    down = synth.blocks(fmt, E * out, out, synth.seed_of(11, 10 * fmt + 2))
    mats = [q.Matrix(dput(h, dev), fmt, E * out, k) for h in host] + [q.Matrix(dput(down, dev), fmt, E * out, out)]
    m = dict(fmt=fmt, E=E, out=out, k=k, mats=mats)
    ids = [2, 7, 11, 15]
    x = synth.x_vec(k, 5)
    gu_s, y_s = separate(dev, m, x, ids)
    gu_f, y_f = fused(dev, m, x, ids)
    assert bits_equal(gu_f, gu_s) and bits_equal(y_f, y_s)
