"""GPU: qgemv_stream_rows_noalloc, the streamed GEMV for callers that cannot
allocate.  Its ring is the library's own device array; its output must have
the bits of qgemv_stream_rows (a streamer's ring) on the same input, on two
calls in a row, the second on a smaller window and matrix, in a fresh process
as well as after the other tests."""
from __future__ import annotations

import numpy as np
import pytest

import quantized_gemv_gguf_amd as q
import synth
from gates import bits_equal

pytestmark = pytest.mark.gpu


def pinned(a):
    import torch
    t = torch.empty(a.shape, dtype=torch.uint8, pin_memory=True)
    t.numpy()[...] = a
    return t


def test_noalloc_equals_streamer_twice(dev):
    import torch
    f32 = dict(dtype=torch.float32, device=dev)
    cases = [(q.Q8_0, 11008, 4096, 512, 0, 11008), (q.Q4_0, 1000, 2048, 96, 17, 803)]
    for fmt, rows, k, B, r0, r1 in cases:
        print(f"noalloc: fmt {fmt} rows {rows} k {k} block_rows {B} window {r0}:{r1}", flush=True)
        w = synth.blocks(fmt, rows, k, synth.seed_of(60, fmt))
        x = torch.from_numpy(synth.x_vec(k, synth.seed_of(60, 9))).to(dev)
        P = q.Matrix(pinned(w), fmt, rows, k)
        n = r1 - r0
        ref = torch.full((n,), float("nan"), **f32)
        with q.Streamer(B * synth.row_bytes(fmt, k), 2) as st:
            st.rows(P, r0, r1, x, ref, B)
            torch.cuda.synchronize()
        got = torch.full((n + 2,), float("nan"), **f32)
        q.qgemv_stream_rows_noalloc(P, r0, r1, x, got[1:n + 1], B)
        torch.cuda.synchronize()
        g = got.cpu().numpy()
        assert np.isnan(g[0]) and np.isnan(g[-1]), "wrote outside its rows"
        assert bits_equal(g[1:n + 1], ref.cpu().numpy())


def test_noalloc_capacity_and_pinning(dev):
    import torch
    fmt, rows, k = q.Q8_0, 1024, 24576
    w = synth.blocks(fmt, rows, k, synth.seed_of(61, 0))
    x = torch.from_numpy(synth.x_vec(k, synth.seed_of(61, 9))).to(dev)
    y = torch.empty(rows, dtype=torch.float32, device=dev)
    P = q.Matrix(pinned(w), fmt, rows, k)
    slot_rows = (q.NOALLOC_RING_BYTES // 2) // synth.row_bytes(fmt, k)
    with pytest.raises(q.QgemvError) as e:
        q.qgemv_stream_rows_noalloc(P, 0, rows, x, y, slot_rows + 1)
    assert e.value.status == -8
    q.qgemv_stream_rows_noalloc(P, 0, rows, x, y, slot_rows)  # the largest block that fits
    D = q.Matrix(torch.from_numpy(w).to(dev), fmt, rows, k)
    with pytest.raises(q.QgemvError) as e:
        q.qgemv_stream_rows_noalloc(D, 0, rows, x, y, 64)
    assert e.value.status == -7
    ref = torch.empty(rows, dtype=torch.float32, device=dev)
    q.qgemv_rows(D, 0, rows, x, ref)
    torch.cuda.synchronize()
    assert bits_equal(y.cpu().numpy(), ref.cpu().numpy())
