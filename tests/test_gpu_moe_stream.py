"""GPU parity for the expert-window dispatcher (MXFP4 MoE, 128 x 2880 x 2880,
top-4) and the pinned-host block streamer (Q8_0 FFN trio 11008/4096), at the
workloads' full sizes, through the C ABI."""
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


def pinned(a):
    import torch
    t = torch.empty(a.shape, dtype=torch.uint8, pin_memory=True)
    t.numpy()[...] = a
    return t


def sync():
    import torch
    torch.cuda.synchronize()


# --- MoE expert windows -----------------------------------------------------------------

@pytest.fixture(scope="module")
def moe(dev):
    c = synth.CONFIGS[4]
    E, out, k = c["n_expert"], c["out"], c["k"]
    host = [synth.blocks(q.MXFP4, E * out, k, synth.seed_of(4, t)) for t in range(3)]
    mats = [q.Matrix(dput(h, dev), q.MXFP4, E * out, k) for h in host]
    ids = synth.expert_ids(E, c["n_sel"], c["tokens"], synth.seed_of(4, 8))
    return dict(E=E, out=out, k=k, host=host, mats=mats, ids=ids)


def moe_token(dev, m, x, ids, block_rows):
    """gate/up windows of the selected experts in one grid, SiLU*up, down
    windows in one grid; returns (g, u, h, y) as host arrays."""
    import torch
    n_sel, out = len(ids), m["out"]
    gu = torch.empty(2 * n_sel * out, dtype=torch.float32, device=dev)
    h = torch.empty(n_sel * out, dtype=torch.float32, device=dev)
    y = torch.empty(n_sel * out, dtype=torch.float32, device=dev)
    xd = dput(x, dev)
    q.qgemv_expert_windows(m["mats"][:2], m["E"], ids, xd, 0, gu, block_rows)
    q.qgemv_silu_mul(gu[:n_sel * out], gu[n_sel * out:], h)
    q.qgemv_expert_windows(m["mats"][2:], m["E"], ids, h, out, y, block_rows)
    sync()
    gu = gu.cpu().numpy()
    return gu[:n_sel * out], gu[n_sel * out:], h.cpu().numpy(), y.cpu().numpy()


@pytest.mark.parametrize("token", [0, 1, 63])
def test_moe_token_against_oracle(dev, moe, token):
    m = moe
    E, out, k = m["E"], m["out"], m["k"]
    ids = m["ids"][token]
    x = synth.x_vec(k, synth.seed_of(4, 100 + token))
    g, u, h, y = moe_token(dev, m, x, ids, 0)
    for s, e in enumerate(ids):
        r0, r1 = int(e) * out, (int(e) + 1) * out
        rg, ag = oracle.gemv_rows(q.MXFP4, m["host"][0], E * out, k, x, r0, r1)
        ru, au = oracle.gemv_rows(q.MXFP4, m["host"][1], E * out, k, x, r0, r1)
        check(g[s * out:(s + 1) * out], rg, ag, what=f"gate e{e}")
        check(u[s * out:(s + 1) * out], ru, au, what=f"up e{e}")
        # teacher-forced down: the oracle takes the GPU's fp32 h
        he = h[s * out:(s + 1) * out]
        rd, ad = oracle.gemv_rows(q.MXFP4, m["host"][2], E * out, k, he, r0, r1)
        check(y[s * out:(s + 1) * out], rd, ad, what=f"down e{e}")
        # the SiLU*up step itself against the fp64 oracle on the GPU's g, u
        ref_h = oracle.silu_mul(g[s * out:(s + 1) * out], u[s * out:(s + 1) * out])
        assert np.all(np.abs(he - ref_h) <= 1e-6 * (np.abs(g[s * out:(s + 1) * out] * u[s * out:(s + 1) * out]) + 1e-30))


def test_moe_block_rows_and_single_windows_bit_identical(dev, moe):
    import torch
    m = moe
    out, k = m["out"], m["k"]
    ids = m["ids"][5]
    x = synth.x_vec(k, synth.seed_of(4, 105))
    ref = moe_token(dev, m, x, ids, 0)
    for b in (128, 512):
        got = moe_token(dev, m, x, ids, b)
        for a, r in zip(got, ref):
            assert bits_equal(a, r), f"block_rows {b}"
    # one window per call equals the one-grid dispatch
    xd = dput(x, dev)
    for s, e in enumerate(ids):
        yd = torch.empty(out, dtype=torch.float32, device=dev)
        q.qgemv_rows(m["mats"][0], int(e) * out, (int(e) + 1) * out, xd, yd)
        sync()
        assert bits_equal(yd.cpu().numpy(), ref[0][s * out:(s + 1) * out])


def test_moe_routing_is_four_distinct_of_128(moe):
    ids = moe["ids"]
    assert ids.shape == (64, 4)
    assert all(len(set(r)) == 4 for r in ids) and ids.min() >= 0 and ids.max() < 128


# --- streamer -------------------------------------------------------------------------------

def test_ring_is_lookahead_plus_one_slots(dev):
    """The page's 0.39 MB arena peak: 128-row MXFP4 blocks of a 2880-wide
    expert, lookahead 1 -> two slots."""
    rb = q.qgemv_weight_bytes(q.MXFP4, 1, 2880)
    with q.Streamer(128 * rb, 1) as st:
        assert st.ring_bytes == 391_680
        assert q.qgemv_weight_bytes(q.MXFP4, 2880, 2880) / st.ring_bytes == pytest.approx(11.25)


@pytest.fixture(scope="module")
def ffn(dev):
    c = synth.CONFIGS[3]
    H, F = c["hidden"], c["ffn"]
    gate = synth.blocks(q.Q8_0, F, H, synth.seed_of(3, 0))
    up = synth.blocks(q.Q8_0, F, H, synth.seed_of(3, 1))
    down = synth.blocks(q.Q8_0, H, F, synth.seed_of(3, 2))
    x = synth.x_vec(H, synth.seed_of(3, 9))
    host = dict(gate=gate, up=up, down=down)
    pin = {n: pinned(a) for n, a in host.items()}
    res = {n: dput(a, dev) for n, a in host.items()}
    return dict(H=H, F=F, host=host, pin=pin, res=res, x=x)


def ffn_resident(dev, f):
    import torch
    H, F = f["H"], f["F"]
    xd = dput(f["x"], dev)
    g = torch.empty(F, dtype=torch.float32, device=dev)
    u = torch.empty(F, dtype=torch.float32, device=dev)
    h = torch.empty(F, dtype=torch.float32, device=dev)
    y = torch.empty(H, dtype=torch.float32, device=dev)
    q.qgemv_windows([q.Window(q.Matrix(f["res"]["gate"], q.Q8_0, F, H), 0, F, xd, g),
                     q.Window(q.Matrix(f["res"]["up"], q.Q8_0, F, H), 0, F, xd, u)])
    q.qgemv_silu_mul(g, u, h)
    q.qgemv_rows(q.Matrix(f["res"]["down"], q.Q8_0, H, F), 0, H, h, y)
    sync()
    return [t.cpu().numpy() for t in (g, u, h, y)]


def ffn_streamed(dev, f, st, block_rows):
    import torch
    H, F = f["H"], f["F"]
    xd = dput(f["x"], dev)
    g = torch.full((F,), float("nan"), dtype=torch.float32, device=dev)
    u = torch.full((F,), float("nan"), dtype=torch.float32, device=dev)
    h = torch.empty(F, dtype=torch.float32, device=dev)
    y = torch.full((H,), float("nan"), dtype=torch.float32, device=dev)
    st.windows([q.Window(q.Matrix(f["pin"]["gate"], q.Q8_0, F, H), 0, F, xd, g),
                q.Window(q.Matrix(f["pin"]["up"], q.Q8_0, F, H), 0, F, xd, u)], block_rows)
    q.qgemv_silu_mul(g, u, h)
    st.rows(q.Matrix(f["pin"]["down"], q.Q8_0, H, F), 0, H, h, y, block_rows)
    sync()
    return [t.cpu().numpy() for t in (g, u, h, y)]


def test_ffn_resident_against_oracle(dev, ffn):
    f = ffn
    H, F = f["H"], f["F"]
    g, u, h, y = ffn_resident(dev, f)
    rg, ag = oracle.gemv_rows(q.Q8_0, f["host"]["gate"], F, H, f["x"])
    ru, au = oracle.gemv_rows(q.Q8_0, f["host"]["up"], F, H, f["x"])
    check(g, rg, ag, what="gate")
    check(u, ru, au, what="up")
    rd, ad = oracle.gemv_rows(q.Q8_0, f["host"]["down"], H, F, h)  # teacher-forced
    check(y, rd, ad, what="down")


@pytest.mark.parametrize("block_rows", [128, 512, 2048])
def test_ffn_streamed_equals_resident(dev, ffn, block_rows):
    f = ffn
    ref = ffn_resident(dev, f)
    rb_down = q.qgemv_weight_bytes(q.Q8_0, 1, f["F"])
    with q.Streamer(block_rows * rb_down, 2) as st:
        got = ffn_streamed(dev, f, st, block_rows)
        for a, r, n in zip(got, ref, "guhy"):
            assert bits_equal(a, r), f"{n} differs at block_rows {block_rows}"
        # the same streamer again (slot reuse across calls)
        got = ffn_streamed(dev, f, st, block_rows)
        assert bits_equal(got[3], ref[3])


def test_minimal_ring_many_blocks(dev, ffn):
    """lookahead 1 (two slots, each exactly one block): every slot is reused
    many times; the result still equals the resident one."""
    f = ffn
    ref = ffn_resident(dev, f)
    rb_down = q.qgemv_weight_bytes(q.Q8_0, 1, f["F"])
    with q.Streamer(7 * rb_down, 1) as st:
        got = ffn_streamed(dev, f, st, 7)
        assert bits_equal(got[3], ref[3])


def test_streamer_rejects_pageable_and_device_memory(dev, ffn):
    import torch
    f = ffn
    H, F = f["H"], f["F"]
    y = torch.empty(F, dtype=torch.float32, device=dev)
    xd = dput(f["x"], dev)
    pageable = torch.from_numpy(f["host"]["gate"])
    with q.Streamer(1 << 20, 1) as st:
        for data in (pageable, f["res"]["gate"]):
            with pytest.raises(q.QgemvError) as e:
                st.rows(q.Matrix(data, q.Q8_0, F, H), 0, 64, xd, y, 16)
            assert e.value.name == "QG_E_NOT_PINNED"
        with pytest.raises(q.QgemvError) as e:  # a 512-row block does not fit 1 MiB
            st.rows(q.Matrix(f["pin"]["gate"], q.Q8_0, F, H), 0, 1024, xd, y, 512)
        assert e.value.name == "QG_E_CAPACITY"
