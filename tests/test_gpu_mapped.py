"""GPU parity for host-mapped weights (zero copy): the GEMV kernels read
page-locked host memory in place over the host link (hipfire PR, "Design
notes": hipHostMalloc-mapped host memory, unchanged kernels dereferencing the
host-mapped alias).  A row's result must be the same bits as the resident run,
for every format, block size and window layout."""
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


@pytest.mark.parametrize("fmt,rows,k", [(q.Q8_0, 11008, 4096), (q.Q4_0, 4096, 4096), (q.MXFP4, 2880, 2880),
                                        (q.Q8_0, 77, 24576), (q.Q4_0, 33, 96), (q.Q4_K, 1000, 4096),
                                        (q.Q6_K, 300, 11008)])
def test_mapped_rows_equal_resident(dev, fmt, rows, k):
    import torch
    w = synth.blocks(fmt, rows, k, synth.seed_of(7, fmt))
    x = synth.x_vec(k, synth.seed_of(7, 9))
    xd = dput(x, dev)
    res = q.Matrix(dput(w, dev), fmt, rows, k)
    pin = q.Matrix(pinned(w), fmt, rows, k)
    ref = torch.empty(rows, dtype=torch.float32, device=dev)
    q.qgemv_rows(res, 0, rows, xd, ref)
    for B in (0, 1, 7, 512):
        y = torch.full((rows + 2,), float("nan"), dtype=torch.float32, device=dev)
        q.qgemv_mapped_rows(pin, 0, rows, xd, y[1:rows + 1], B)
        sync()
        got = y.cpu().numpy()
        assert bits_equal(got[1:rows + 1], ref.cpu().numpy()), f"block_rows {B}"
        assert np.isnan(got[0]) and np.isnan(got[rows + 1]), "wrote outside its rows"
    r, a = oracle.gemv_rows(fmt, w, rows, k, x)
    check(ref.cpu().numpy(), r, a, what="resident vs oracle")


def test_mapped_windows_equal_resident(dev):
    import torch
    fmt, rows, k = q.Q8_0, 1000, 4096
    w = synth.blocks(fmt, rows, k, synth.seed_of(7, 20))
    x = synth.x_vec(k, synth.seed_of(7, 21))
    xd = dput(x, dev)
    res = q.Matrix(dput(w, dev), fmt, rows, k)
    pin = q.Matrix(pinned(w), fmt, rows, k)
    spans = [(0, 300), (300, 301), (512, 1000), (5, 5), (900, 1000)]
    ys_r = [torch.empty(max(b - a, 1), dtype=torch.float32, device=dev) for a, b in spans]
    ys_m = [torch.empty(max(b - a, 1), dtype=torch.float32, device=dev) for a, b in spans]
    q.qgemv_windows([q.Window(res, a, b, xd, y) for (a, b), y in zip(spans, ys_r)])
    q.qgemv_mapped_windows([q.Window(pin, a, b, xd, y) for (a, b), y in zip(spans, ys_m)], 128)
    sync()
    for (a, b), yr, ym in zip(spans, ys_r, ys_m):
        n = b - a
        assert bits_equal(ym.cpu().numpy()[:n], yr.cpu().numpy()[:n]), f"window {a}:{b}"


def test_mapped_rejects_pageable_and_device_memory(dev):
    import torch
    fmt, rows, k = q.Q8_0, 64, 256
    w = synth.blocks(fmt, rows, k, synth.seed_of(7, 30))
    xd = torch.zeros(k, dtype=torch.float32, device=dev)
    y = torch.empty(rows, dtype=torch.float32, device=dev)
    for data in (torch.from_numpy(w), dput(w, dev)):
        with pytest.raises(q.QgemvError) as e:
            q.qgemv_mapped_rows(q.Matrix(data, fmt, rows, k), 0, rows, xd, y)
        assert e.value.name == "QG_E_NOT_PINNED"
        with pytest.raises(q.QgemvError) as e:
            q.qgemv_mapped_windows([q.Window(q.Matrix(data, fmt, rows, k), 0, rows, xd, y)])
        assert e.value.name == "QG_E_NOT_PINNED"
