"""The C ABI on the host (no GPU): the library loads, exports every entry point
include/qgemv.h declares, and rejects bad arguments with the documented status
before any HIP call."""
from __future__ import annotations

import ctypes
import os
import re
import subprocess

import pytest

import quantized_gemv_gguf_amd as q
from quantized_gemv_gguf_amd import qg_matrix, qg_window

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qgemv.h")

E_NULL, E_FMT, E_SHAPE, E_RANGE, E_SIZE, E_ARG, E_NOT_PINNED, E_CAPACITY, E_HIP = -1, -2, -3, -4, -5, -6, -7, -8, -100


def declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(qgemv_\w+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    names = declared()
    assert len(names) == 16, names
    out = subprocess.run(["nm", "-D", "--defined-only", q.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\sT\s(\w+)$", out, flags=re.M))
    missing = [n for n in names if n not in exported]
    assert not missing, missing
    L = q.lib()
    for n in names:
        assert hasattr(L, n)


def test_header_constants_match_binding():
    text = open(HEADER).read()
    assert re.search(r"QG_Q8_0 = 1, QG_Q4_0 = 2, QG_MXFP4 = 3", text)
    assert f"#define QG_MAX_WINDOWS {q.MAX_WINDOWS}" in text
    assert f"#define QG_MAX_K {q.MAX_K}" in text
    for code, name in q.STATUS.items():
        assert re.search(rf"{name} = {code}\b", text), name


def test_header_compiles_as_c():
    src = '#include "qgemv.h"\nint main(void){qg_matrix m; qg_window w; (void)m; (void)w; return 0;}\n'
    r = subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-fsyntax-only", f"-I{os.path.dirname(HEADER)}",
                        "-x", "c", "-"], input=src, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


def test_sizes():
    L = q.lib()
    assert [L.qgemv_block_bytes(f) for f in (1, 2, 3)] == [34, 18, 17]
    assert L.qgemv_block_bytes(0) == E_FMT and L.qgemv_block_bytes(4) == E_FMT
    assert L.qgemv_weight_bytes(3, 2880, 2880) == 4_406_400
    assert L.qgemv_weight_bytes(2, 4096, 4096) == 9_437_184
    assert L.qgemv_weight_bytes(1, 11008, 4096) == 47_906_816
    assert L.qgemv_weight_bytes(1, 0, 64) == 0
    assert L.qgemv_weight_bytes(1, 4, 48) == E_SHAPE
    assert L.qgemv_weight_bytes(1, 4, 0) == E_SHAPE
    assert L.qgemv_weight_bytes(1, -1, 64) == E_SHAPE
    assert L.qgemv_weight_bytes(9, 4, 64) == E_FMT


FAKE = 0x1000  # a non-NULL address; never dereferenced by a call that fails validation


def mat(fmt=1, rows=8, k=64, nbytes=None, data=FAKE, reserved=0):
    n = rows * (k // 32) * {1: 34, 2: 18, 3: 17}.get(fmt, 34) if nbytes is None else nbytes
    return qg_matrix(data, fmt, reserved, rows, k, n)


def rows_call(m, r0=0, r1=8, x=FAKE, y=FAKE, B=0):
    return q.lib().qgemv_rows(ctypes.byref(m) if m is not None else None, r0, r1, x, y, B, None)


def test_qgemv_rows_validation():
    assert rows_call(None) == E_NULL
    assert rows_call(mat(fmt=5)) == E_FMT
    assert rows_call(mat(k=48, nbytes=0)) == E_SHAPE
    assert rows_call(mat(k=49152 + 32)) == E_SHAPE
    assert rows_call(mat(data=FAKE + 8)) == E_ARG  # not 16-byte aligned
    assert rows_call(mat(nbytes=8 * 2 * 34 - 1)) == E_SIZE
    assert rows_call(mat(nbytes=8 * 2 * 34 + 1)) == E_SIZE
    assert rows_call(mat(), r0=-1) == E_RANGE
    assert rows_call(mat(), r0=5, r1=4) == E_RANGE
    assert rows_call(mat(), r1=9) == E_RANGE
    assert rows_call(mat(), B=-1) == E_ARG
    assert rows_call(mat(), x=0) == E_NULL
    assert rows_call(mat(), y=0) == E_NULL
    assert rows_call(mat(data=0)) == E_NULL
    assert rows_call(mat(reserved=1)) == E_ARG
    # empty window: nothing to do, no HIP call, no pointer needed
    assert rows_call(mat(), r0=3, r1=3, x=0, y=0) == 0
    assert rows_call(mat(rows=0, data=0), r0=0, r1=0) == 0


def test_dequant_validation():
    L = q.lib()
    assert L.qgemv_dequant_rows(None, 0, 1, FAKE, None) == E_NULL
    assert L.qgemv_dequant_rows(ctypes.byref(mat()), 0, 9, FAKE, None) == E_RANGE
    assert L.qgemv_dequant_rows(ctypes.byref(mat()), 0, 1, 0, None) == E_NULL
    assert L.qgemv_dequant_rows(ctypes.byref(mat(fmt=0)), 0, 1, FAKE, None) == E_FMT


def win(r0=0, r1=8, rows=8, data=FAKE, x=FAKE, y=FAKE):
    return qg_window(data, rows, r0, r1, x, y)


def test_qgemv_windows_validation():
    L = q.lib()
    arr = (qg_window * 2)(win(), win(2, 5))
    assert L.qgemv_windows(7, 64, arr, 2, 0, None) == E_FMT
    assert L.qgemv_windows(1, 40, arr, 2, 0, None) == E_SHAPE
    assert L.qgemv_windows(1, 64, arr, -1, 0, None) == E_ARG
    assert L.qgemv_windows(1, 64, arr, 65, 0, None) == E_ARG
    assert L.qgemv_windows(1, 64, None, 2, 0, None) == E_NULL
    assert L.qgemv_windows(1, 64, arr, 2, -3, None) == E_ARG
    assert L.qgemv_windows(1, 64, (qg_window * 1)(win(4, 9)), 1, 0, None) == E_RANGE
    assert L.qgemv_windows(1, 64, (qg_window * 1)(win(x=0)), 1, 0, None) == E_NULL
    assert L.qgemv_windows(1, 64, (qg_window * 1)(win(data=0)), 1, 0, None) == E_NULL
    assert L.qgemv_windows(1, 64, None, 0, 0, None) == 0
    assert L.qgemv_windows(1, 64, (qg_window * 1)(win(3, 3, x=0, y=0, data=0)), 1, 0, None) == 0


def test_expert_windows_validation():
    L = q.lib()
    mats = (qg_matrix * 2)(mat(rows=128 * 4), mat(rows=128 * 4))
    ids = (ctypes.c_int32 * 4)(0, 5, 127, 3)

    def call(m=mats, nm=2, ne=128, i=ids, ns=4, x=FAKE, xs=0, y=FAKE, B=0):
        return L.qgemv_expert_windows(m, nm, ne, i, ns, x, xs, y, B, None)

    assert call(m=None) == E_NULL
    assert call(i=None) == E_NULL
    assert call(nm=0) == E_ARG
    assert call(ns=-1) == E_ARG
    assert call(xs=-1) == E_ARG
    assert call(B=-1) == E_ARG
    assert call(ne=0) == E_SHAPE
    assert call(ne=3) == E_SHAPE  # 512 rows is not a multiple of 3 experts
    assert call(i=(ctypes.c_int32 * 4)(0, 5, 128, 3)) == E_RANGE
    assert call(i=(ctypes.c_int32 * 4)(0, -1, 1, 3)) == E_RANGE
    assert call(m=(qg_matrix * 2)(mat(rows=512), mat(rows=256))) == E_SHAPE
    assert call(m=(qg_matrix * 2)(mat(rows=512), mat(rows=512, fmt=2))) == E_SHAPE
    big = (ctypes.c_int32 * 33)(*range(33))
    assert call(i=big, ns=33) == E_ARG  # 2 x 33 windows > 64
    assert call(x=0) == E_NULL
    assert call(ns=0) == 0


def test_elementwise_validation():
    L = q.lib()
    assert L.qgemv_silu_mul(FAKE, FAKE, FAKE, -1, None) == E_ARG
    assert L.qgemv_silu_mul(0, FAKE, FAKE, 4, None) == E_NULL
    assert L.qgemv_silu_mul(0, 0, 0, 0, None) == 0
    assert L.qgemv_rms_carry(FAKE, FAKE, 0, 1e-6, 0, None) == E_ARG
    assert L.qgemv_rms_carry(FAKE, FAKE, 4, -1.0, 0, None) == E_ARG
    assert L.qgemv_rms_carry(FAKE, FAKE, 4, float("nan"), 0, None) == E_ARG
    assert L.qgemv_rms_carry(FAKE, FAKE, 4, 1e-6, 2, None) == E_ARG
    assert L.qgemv_rms_carry(0, FAKE, 4, 1e-6, 0, None) == E_NULL


def test_streamer_validation():
    L = q.lib()
    h = ctypes.c_void_p()
    assert L.qgemv_stream_create(1024, 1, None) == E_NULL
    assert L.qgemv_stream_create(0, 1, ctypes.byref(h)) == E_ARG
    assert L.qgemv_stream_create(1024, 0, ctypes.byref(h)) == E_ARG
    assert L.qgemv_stream_ring_bytes(None) == E_NULL
    assert L.qgemv_stream_destroy(None) == 0
    assert L.qgemv_stream_rows(None, ctypes.byref(mat()), 0, 8, 0, FAKE, FAKE, None) == E_NULL
    assert L.qgemv_stream_windows(None, 1, 64, None, 0, 0, None) == E_NULL


def test_strerror_and_version():
    L = q.lib()
    for code in [0, *q.STATUS]:
        assert L.qgemv_strerror(code)
    assert L.qgemv_strerror(-12345) == b"unknown status"
    assert re.match(rb"\d+\.\d+\.\d+", L.qgemv_version())
    assert L.qgemv_last_hip_error() == b""


def test_binding_raises_named_errors():
    with pytest.raises(q.QgemvError) as e:
        q._check(-4, "x")
    assert e.value.name == "QG_E_RANGE"
