"""GPU: streamed plans (qgemv_stream_plan_*) and the streamer at the pages'
MoE block size.

A plan walks a layer's streamed GEMV steps and the elementwise steps between
them as one replayed graph; each y must have the bits of the resident
computation.  Covered: the Q8_0 FFN trio (gate and up, SiLU * up, down) at
block_rows 128/512/2048 with lookahead 2; MXFP4 MoE tokens (the selected
experts' gate/up windows, SiLU * up, down windows, router-weighted combine)
at block_rows 128 with lookahead 1 -- a ring of 2 x 128 rows x 1,530 bytes =
391,680 bytes, neurostream README, "The idea" ("0.39 MB") -- re-pointed at
each token's experts, with a run enqueued before the re-pointing keeping its
own experts; and the per-call streamer (qgemv_stream_windows) at the same
128-row, lookahead-1 setting.
"""
from __future__ import annotations

import numpy as np
import pytest

import quantized_gemv_gguf_amd as q
import synth
from gates import bits_equal

pytestmark = pytest.mark.gpu


def dput(a, dev):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def pinned(a):
    import torch
    t = torch.empty(a.shape, dtype=torch.uint8, pin_memory=True)
    t.numpy()[...] = a
    return t


@pytest.mark.parametrize("B", [128, 512, 2048])
def test_ffn_trio_plan_equals_resident(dev, B):
    import torch
    H, F = 4096, 11008
    f32 = dict(dtype=torch.float32, device=dev)
    host = [synth.blocks(q.Q8_0, F, H, synth.seed_of(3, 0)), synth.blocks(q.Q8_0, F, H, synth.seed_of(3, 1)),
            synth.blocks(q.Q8_0, H, F, synth.seed_of(3, 2))]
    R = [q.Matrix(dput(host[0], dev), q.Q8_0, F, H), q.Matrix(dput(host[1], dev), q.Q8_0, F, H),
         q.Matrix(dput(host[2], dev), q.Q8_0, H, F)]
    P = [q.Matrix(pinned(host[0]), q.Q8_0, F, H), q.Matrix(pinned(host[1]), q.Q8_0, F, H),
         q.Matrix(pinned(host[2]), q.Q8_0, H, F)]
    x = dput(synth.x_vec(H, synth.seed_of(3, 9)), dev)
    g, u, h, y = (torch.empty(n, **f32) for n in (F, F, F, H))
    q.qgemv_windows([q.Window(R[0], 0, F, x, g), q.Window(R[1], 0, F, x, u)])
    q.qgemv_silu_mul(g, u, h)
    q.qgemv_rows(R[2], 0, H, h, y)
    torch.cuda.synchronize()
    ref = [t.cpu().numpy().copy() for t in (g, u, y)]
    g2, u2, h2, y2 = (torch.full((n,), float("nan"), **f32) for n in (F, F, F, H))
    steps = [q.PlanGemv([q.Window(P[0], 0, F, x, g2), q.Window(P[1], 0, F, x, u2)], B),
             q.PlanSiluMul(g2, u2, h2), q.PlanGemv([q.Window(P[2], 0, H, h2, y2)], B)]
    with q.StreamPlan(B * synth.row_bytes(q.Q8_0, F), 2, steps) as plan:
        for run in range(3):
            y2.fill_(float("nan"))
            plan.run()
            torch.cuda.synchronize()
            for got, want in zip((g2, u2, y2), ref):
                assert bits_equal(got.cpu().numpy(), want), f"run {run}"


def moe_setup(dev):
    import torch
    c = synth.CONFIGS[4]
    E, out, k, ns = c["n_expert"], c["out"], c["k"], c["n_sel"]
    host = [synth.blocks(q.MXFP4, E * out, k, synth.seed_of(4, t)) for t in range(3)]
    R = [q.Matrix(dput(h, dev), q.MXFP4, E * out, k) for h in host]
    P = [q.Matrix(pinned(h), q.MXFP4, E * out, k) for h in host]
    ids = synth.expert_ids(E, ns, c["tokens"], synth.seed_of(4, 8))
    xs = [dput(synth.x_vec(k, synth.seed_of(4, 100 + t)), dev) for t in range(4)]
    wts = dput(synth.router_weights(c["tokens"], ns, synth.seed_of(4, 9)), dev)
    return E, out, k, ns, R, P, ids, xs, wts


def moe_resident(dev, E, out, k, ns, R, ids_t, x, w):
    import torch
    f32 = dict(dtype=torch.float32, device=dev)
    gu, h, ye, y = torch.empty(2 * ns * out, **f32), torch.empty(ns * out, **f32), torch.empty(ns * out, **f32), \
        torch.empty(out, **f32)
    q.qgemv_expert_windows(R[:2], E, ids_t, x, 0, gu)
    q.qgemv_silu_mul(gu[:ns * out], gu[ns * out:], h)
    q.qgemv_expert_windows(R[2:], E, ids_t, h, out, ye)
    q.qgemv_combine(ye, out, ns, w, out, y)
    torch.cuda.synchronize()
    return ye.cpu().numpy(), y.cpu().numpy()


def test_moe_plan_128_rows_lookahead_1(dev):
    import torch
    E, out, k, ns, R, P, ids, xs, wts = moe_setup(dev)
    f32 = dict(dtype=torch.float32, device=dev)
    x = torch.empty(k, **f32)
    w = torch.empty(ns, **f32)
    gu, h, ye, y = torch.empty(2 * ns * out, **f32), torch.empty(ns * out, **f32), torch.empty(ns * out, **f32), \
        torch.empty(out, **f32)
    sel0 = [int(e) for e in ids[0]]
    gw = [q.Window(P[m], e * out, (e + 1) * out, x, gu[(m * ns + s) * out:(m * ns + s + 1) * out])
          for m in range(2) for s, e in enumerate(sel0)]
    dw = [q.Window(P[2], e * out, (e + 1) * out, h[s * out:(s + 1) * out], ye[s * out:(s + 1) * out])
          for s, e in enumerate(sel0)]
    steps = [q.PlanGemv(gw, 128), q.PlanSiluMul(gu[:ns * out], gu[ns * out:], h), q.PlanGemv(dw, 128),
             q.PlanCombine(ye, out, ns, w, out, y)]
    rb = synth.row_bytes(q.MXFP4, k)
    with q.StreamPlan(128 * rb, 1, steps) as plan:
        assert plan.ring_bytes == 391680  # 2 slots x 128 rows x 1,530 bytes: the page's 0.39 MB
        saved = []
        for t in range(4):
            sel = [int(e) for e in ids[t]]
            for s, e in enumerate(sel):
                plan.set_rows(s, e * out)           # gate window of slot s
                plan.set_rows(ns + s, e * out)      # up
                plan.set_rows(2 * ns + s, e * out)  # down
            x.copy_(xs[t])
            w.copy_(wts[t])
            plan.run()
            # (the next token re-points the plan while this run may still be in
            # flight; the copies below are ordered after it on the stream)
            saved.append((ye.clone(), y.clone()))
        torch.cuda.synchronize()
        for t in range(4):
            want_ye, want_y = moe_resident(dev, E, out, k, ns, R, ids[t], xs[t], wts[t])
            assert bits_equal(saved[t][0].cpu().numpy(), want_ye), f"token {t}: expert outputs"
            assert bits_equal(saved[t][1].cpu().numpy(), want_y), f"token {t}: combined output"


def test_streamer_moe_windows_128_rows_lookahead_1(dev):
    import torch
    E, out, k, ns, R, P, ids, xs, wts = moe_setup(dev)
    f32 = dict(dtype=torch.float32, device=dev)
    rb = synth.row_bytes(q.MXFP4, k)
    with q.Streamer(128 * rb, 1) as st:
        assert st.ring_bytes == 391680
        for t in range(2):
            sel = [int(e) for e in ids[t]]
            gu, h, ye = torch.empty(2 * ns * out, **f32), torch.empty(ns * out, **f32), torch.empty(ns * out, **f32)
            gw = [q.Window(P[m], e * out, (e + 1) * out, xs[t], gu[(m * ns + s) * out:(m * ns + s + 1) * out])
                  for m in range(2) for s, e in enumerate(sel)]
            dw = [q.Window(P[2], e * out, (e + 1) * out, h[s * out:(s + 1) * out], ye[s * out:(s + 1) * out])
                  for s, e in enumerate(sel)]
            st.windows(gw, 128)
            q.qgemv_silu_mul(gu[:ns * out], gu[ns * out:], h)
            st.windows(dw, 128)
            torch.cuda.synchronize()
            want_ye, _ = moe_resident(dev, E, out, k, ns, R, ids[t], xs[t], wts[t])
            assert bits_equal(ye.cpu().numpy(), want_ye), f"token {t}"


def test_plan_errors(dev):
    import torch
    fmt, rows, k = q.Q8_0, 256, 1024
    w = synth.blocks(fmt, rows, k, 5)
    x = dput(synth.x_vec(k, 6), dev)
    y = torch.empty(rows, dtype=torch.float32, device=dev)
    P = q.Matrix(pinned(w), fmt, rows, k)
    D = q.Matrix(dput(w, dev), fmt, rows, k)
    rb = synth.row_bytes(fmt, k)
    with pytest.raises(q.QgemvError) as e:   # a block larger than a slot
        q.StreamPlan(64 * rb, 1, [q.PlanGemv([q.Window(P, 0, rows, x, y)], 65)])
    assert e.value.status == -8
    with pytest.raises(q.QgemvError) as e:   # device memory is not pinned host memory
        q.StreamPlan(64 * rb, 1, [q.PlanGemv([q.Window(D, 0, rows, x, y)], 64)])
    assert e.value.status == -7
    with q.StreamPlan(64 * rb, 1, [q.PlanGemv([q.Window(P, 0, 100, x, y[:100])], 64)]) as plan:
        with pytest.raises(q.QgemvError) as e:
            plan.set_rows(0, 200)            # 200 + 100 rows > 256
        assert e.value.status == -4
        plan.set_rows(0, 156)
        plan.run()
        ref = torch.empty(100, dtype=torch.float32, device=dev)
        q.qgemv_rows(D, 156, 256, x, ref)
        torch.cuda.synchronize()
        assert bits_equal(y[:100].cpu().numpy(), ref.cpu().numpy())
