"""GPU: the dense pass's fused launches captured into one HIP graph and
replayed.  Each replay must give exactly the bits of the same token run
eagerly from the same carry, on every replay, with unrelated eager work and
synchronisations between the replays (a captured launch keeps its kernel
arguments, so the graph reads and writes the buffers it was captured on)."""
from __future__ import annotations

import numpy as np
import pytest

import quantized_gemv_gguf_amd as q
import synth
from gates import bits_equal

pytestmark = pytest.mark.gpu

H, F = 2048, 5632


def _layers(dev, fmts, n_layers):
    import torch
    shapes = synth.dense_layer_shapes(H, F)
    out = []
    for l in range(n_layers):
        ms = []
        for m, (_, r, k) in enumerate(shapes):
            fmt = fmts[m]
            w = torch.from_numpy(synth.blocks(fmt, r, k, synth.seed_of(11, 4 * l + m))).to(dev)
            ms.append(q.Matrix(w, fmt, r, k))
        out.append(ms)
    return out


def _token(layers, d, qkv, ov, a, stream=None):
    for M in layers:
        q.qgemv_rows_op(M[0], 0, 3 * H, d, qkv, q.IN_RMS, 1e-6, stream=stream)
        q.qgemv_rows_op(M[1], 0, H, qkv[2 * H:], ov, q.IN_RMS, 1e-6, stream=stream)
        q.qgemv_rows_op(M[2], 0, F, ov, a, q.IN_RMS, 1e-6, q.OUT_GELU, stream=stream)
        q.qgemv_rows_op(M[3], 0, H, a, d, q.IN_RMS, 1e-6, stream=stream)


@pytest.mark.parametrize("fmts", [(q.Q8_0,) * 4, (q.Q4_K, q.Q4_K, q.Q4_K, q.Q6_K)],
                         ids=["q8_0", "k_mix"])
def test_graph_replays_equal_eager(dev, fmts):
    import torch
    f32 = dict(dtype=torch.float32, device=dev)
    layers = _layers(dev, fmts, 2)
    d0 = torch.from_numpy(synth.x_vec(H, synth.seed_of(11, 999))).to(dev)
    d, qkv, ov, a = d0.clone(), torch.empty(3 * H, **f32), torch.empty(H, **f32), torch.empty(F, **f32)

    # eager: three tokens from d0, the carry after each kept
    eager = []
    for _ in range(3):
        _token(layers, d, qkv, ov, a)
        eager.append(d.clone())
    torch.cuda.synchronize()

    # capture one token on a side stream (one eager run there first)
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        _token(layers, d, qkv, ov, a, stream=cap)
    torch.cuda.current_stream().wait_stream(cap)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=cap):
        _token(layers, d, qkv, ov, a, stream=cap)
    torch.cuda.synchronize()

    # unrelated eager work between replays: a GEMV into buffers of its own
    side_w = torch.from_numpy(synth.blocks(q.Q8_0, 300, 4096, synth.seed_of(11, 500))).to(dev)
    side_x = torch.from_numpy(synth.x_vec(4096, synth.seed_of(11, 501))).to(dev)
    side_y = torch.empty(300, **f32)
    side_m = q.Matrix(side_w, q.Q8_0, 300, 4096)
    q.qgemv_rows(side_m, 0, 300, side_x, side_y)
    side_ref = side_y.clone()

    d.copy_(d0)
    torch.cuda.synchronize()
    for t in range(3):
        graph.replay()
        torch.cuda.synchronize()
        got = d.clone()
        assert bits_equal(got.cpu().numpy(), eager[t].cpu().numpy()), f"replay {t} differs from eager"
        side_y.fill_(np.nan)
        q.qgemv_rows(side_m, 0, 300, side_x, side_y)
        torch.cuda.synchronize()
        assert bits_equal(side_y.cpu().numpy(), side_ref.cpu().numpy())
    # a replay from a carry written in between by the host path
    d.copy_(eager[0])
    graph.replay()
    torch.cuda.synchronize()
    assert bits_equal(d.cpu().numpy(), eager[1].cpu().numpy())
