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
E_BARRIER = -9


def declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(qgemv_\w+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    names = declared()
    assert len(names) == 39, names
    out = subprocess.run(["nm", "-D", "--defined-only", q.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\sT\s(\w+)$", out, flags=re.M))
    missing = [n for n in names if n not in exported]
    assert not missing, missing
    L = q.lib()
    for n in names:
        assert hasattr(L, n)


def test_header_constants_match_binding():
    text = open(HEADER).read()
    assert re.search(rf"QG_Q8_0 = {q.Q8_0}, QG_Q4_0 = {q.Q4_0}, QG_MXFP4 = {q.MXFP4}, QG_Q4_K = {q.Q4_K}, "
                     rf"QG_Q6_K = {q.Q6_K}", text)
    assert f"#define QG_MAX_WINDOWS {q.MAX_WINDOWS}" in text
    assert f"#define QG_MAX_K {q.MAX_K}" in text
    assert f"#define QG_CHAIN_MAX_K {q.CHAIN_MAX_K}" in text
    assert re.search(rf"QG_IN_X = {q.IN_X}, QG_IN_RMS = {q.IN_RMS}, QG_IN_GELU_RMS = {q.IN_GELU_RMS}, "
                     rf"QG_IN_SILU_MUL = {q.IN_SILU_MUL}", text)
    assert re.search(rf"QG_OUT_Y = {q.OUT_Y}, QG_OUT_GELU = {q.OUT_GELU}", text)
    for code, name in q.STATUS.items():
        assert re.search(rf"{name} = {code}\b", text), name


def test_header_compiles_as_c():
    src = ('#include "qgemv.h"\nint main(void){qg_matrix m; qg_window w; qg_chain_window cw; qg_chain_step cs;'
           ' (void)m; (void)w; (void)cw; (void)cs; return sizeof(qg_chain_step) == 24 ? 0 : 1;}\n')
    r = subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-fsyntax-only", f"-I{os.path.dirname(HEADER)}",
                        "-x", "c", "-"], input=src, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


def test_sizes():
    L = q.lib()
    assert [L.qgemv_block_bytes(f) for f in (1, 2, 3, 4, 5)] == [34, 18, 17, 144, 210]
    assert [L.qgemv_block_weights(f) for f in (1, 2, 3, 4, 5)] == [32, 32, 32, 256, 256]
    assert L.qgemv_block_bytes(0) == E_FMT and L.qgemv_block_bytes(6) == E_FMT
    assert L.qgemv_block_weights(0) == E_FMT and L.qgemv_block_weights(6) == E_FMT
    # K-quants: k a multiple of 256; 6144 x 6144 Q4_K is 4.5 bits per weight
    assert L.qgemv_weight_bytes(4, 6144, 6144) == 6144 * 6144 * 9 // 16
    assert L.qgemv_weight_bytes(5, 2, 512) == 2 * 2 * 210
    assert L.qgemv_weight_bytes(4, 4, 288) == E_SHAPE
    assert L.qgemv_weight_bytes(5, 4, 32) == E_SHAPE
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
    n = rows * (k // 32) * {1: 34, 2: 18, 3: 17, 4: 18, 5: 26.25}.get(fmt, 34) if nbytes is None else nbytes
    n = int(n)
    return qg_matrix(data, fmt, reserved, rows, k, n)


def rows_call(m, r0=0, r1=8, x=FAKE, y=FAKE, B=0):
    return q.lib().qgemv_rows(ctypes.byref(m) if m is not None else None, r0, r1, x, y, B, None)


def test_qgemv_rows_validation():
    assert rows_call(None) == E_NULL
    assert rows_call(mat(fmt=6)) == E_FMT
    assert rows_call(mat(fmt=0)) == E_FMT
    assert rows_call(mat(k=48, nbytes=0)) == E_SHAPE
    # K-quants: k a multiple of 256, n_bytes whole super-blocks
    assert rows_call(mat(fmt=4, k=288, nbytes=0)) == E_SHAPE
    assert rows_call(mat(fmt=5, k=32, nbytes=0)) == E_SHAPE
    assert rows_call(mat(fmt=4, k=512, nbytes=8 * 2 * 144 - 1)) == E_SIZE
    assert rows_call(mat(fmt=5, k=512, nbytes=8 * 2 * 210 + 16)) == E_SIZE
    assert rows_call(mat(fmt=5, k=512, nbytes=8 * 2 * 210), r1=9) == E_RANGE
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


def test_read_ceiling_validation():
    L = q.lib()
    sink = ctypes.c_void_p(0x1000)
    assert L.qgemv_read_ceiling(None, 16, sink, None) == E_NULL
    assert L.qgemv_read_ceiling(FAKE, 16, None, None) == E_NULL
    assert L.qgemv_read_ceiling(FAKE, 0, sink, None) == E_ARG
    assert L.qgemv_read_ceiling(FAKE, 24, sink, None) == E_ARG       # not a multiple of 16
    assert L.qgemv_read_ceiling(FAKE + 8, 32, sink, None) == E_ARG   # not 16-byte aligned


def test_stream_rows_noalloc_validation():
    L = q.lib()
    assert L.qgemv_stream_rows_noalloc(None, 0, 1, 0, FAKE, FAKE, None) == E_NULL
    assert L.qgemv_stream_rows_noalloc(ctypes.byref(mat()), 0, 9, 0, FAKE, FAKE, None) == E_RANGE
    assert L.qgemv_stream_rows_noalloc(ctypes.byref(mat()), 0, 1, -1, FAKE, FAKE, None) == E_ARG
    assert L.qgemv_stream_rows_noalloc(ctypes.byref(mat()), 0, 1, 0, 0, FAKE, None) == E_NULL
    assert L.qgemv_stream_rows_noalloc(ctypes.byref(mat(fmt=0)), 0, 1, 0, FAKE, FAKE, None) == E_FMT
    assert L.qgemv_stream_rows_noalloc(ctypes.byref(mat()), 1, 1, 0, 0, 0, None) == 0  # empty window
    text = open(HEADER).read()
    assert f"#define QG_NOALLOC_RING_BYTES ({q.NOALLOC_RING_BYTES >> 20}ll << 20)" in text


def test_stream_plan_validation():
    L = q.lib()
    h = ctypes.c_void_p()
    step = q.qg_plan_step(q.PLAN_GEMV, 1, 64, 0, 1, 0, None, None, None, 0, 0, 0, 0)
    win = qg_window(FAKE, 8, 0, 8, FAKE, FAKE)
    S1 = (q.qg_plan_step * 1)(step)
    W1 = (qg_window * 1)(win)
    assert L.qgemv_stream_plan_create(1024, 1, S1, 1, W1, 1, None) == E_NULL
    assert L.qgemv_stream_plan_create(1024, 1, None, 1, W1, 1, ctypes.byref(h)) == E_NULL
    assert L.qgemv_stream_plan_create(0, 1, S1, 1, W1, 1, ctypes.byref(h)) == E_ARG
    assert L.qgemv_stream_plan_create(1024, 0, S1, 1, W1, 1, ctypes.byref(h)) == E_ARG
    assert L.qgemv_stream_plan_create(1024, 1, S1, 0, W1, 1, ctypes.byref(h)) == E_ARG
    bad = (q.qg_plan_step * 1)(q.qg_plan_step(9, 1, 64, 0, 1, 0, None, None, None, 0, 0, 0, 0))
    assert L.qgemv_stream_plan_create(1024, 1, bad, 1, W1, 1, ctypes.byref(h)) == E_ARG
    two = (q.qg_plan_step * 1)(q.qg_plan_step(q.PLAN_GEMV, 1, 64, 0, 2, 0, None, None, None, 0, 0, 0, 0))
    assert L.qgemv_stream_plan_create(1024, 1, two, 1, W1, 1, ctypes.byref(h)) == E_ARG  # windows past the table
    nofmt = (q.qg_plan_step * 1)(q.qg_plan_step(q.PLAN_GEMV, 0, 64, 0, 1, 0, None, None, None, 0, 0, 0, 0))
    assert L.qgemv_stream_plan_create(1024, 1, nofmt, 1, W1, 1, ctypes.byref(h)) == E_FMT
    silu = (q.qg_plan_step * 1)(q.qg_plan_step(q.PLAN_SILU_MUL, 0, 0, 0, 0, 0, None, FAKE, FAKE, 4, 0, 0, 0))
    assert L.qgemv_stream_plan_create(1024, 1, silu, 1, W1, 1, ctypes.byref(h)) == E_NULL
    assert L.qgemv_stream_plan_set_rows(None, 0, 0) == E_NULL
    assert L.qgemv_stream_plan_run(None, None) == E_NULL
    assert L.qgemv_stream_plan_ring_bytes(None) == E_NULL
    assert L.qgemv_stream_plan_destroy(None) == 0
    assert ctypes.sizeof(q.qg_plan_step) == 80


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


def test_rows_batch_validation():
    L = q.lib()

    def call(m=None, r0=0, r1=8, x=FAKE, xs=64, nt=2, y=FAKE, ys=8, B=0):
        m = mat() if m is None else m
        return L.qgemv_rows_batch(ctypes.byref(m), r0, r1, x, xs, nt, y, ys, B, None)

    assert L.qgemv_rows_batch(None, 0, 8, FAKE, 64, 2, FAKE, 8, 0, None) == E_NULL
    assert call(m=mat(fmt=6)) == E_FMT
    assert call(m=mat(k=48, nbytes=0)) == E_SHAPE
    assert call(r1=9) == E_RANGE
    assert call(nt=-1) == E_ARG
    assert call(xs=-1) == E_ARG
    assert call(ys=7) == E_ARG  # outputs of two tokens would overlap
    assert call(B=-1) == E_ARG
    assert call(x=0) == E_NULL and call(y=0) == E_NULL
    # nothing to do: no pointer needed, no HIP call
    assert call(nt=0, x=0, y=0) == 0
    assert call(r0=3, r1=3, x=0, y=0) == 0
    # one token needs no y stride
    assert call(nt=1, ys=0, x=0) == E_NULL


def test_rows_mfma_validation():
    L = q.lib()

    def call(m=None, r0=0, r1=8, x=FAKE, xs=64, nt=2, y=FAKE, ys=8):
        m = mat() if m is None else m
        return L.qgemv_rows_mfma(ctypes.byref(m), r0, r1, x, xs, nt, y, ys, None)

    assert L.qgemv_rows_mfma(None, 0, 8, FAKE, 64, 2, FAKE, 8, None) == E_NULL
    assert call(m=mat(fmt=6)) == E_FMT
    # every format passes the format check
    assert call(m=mat(fmt=q.Q6_K, k=256, nbytes=8 * 210), x=0) == E_NULL
    assert call(m=mat(fmt=q.Q4_K, k=256, nbytes=8 * 144), x=0) == E_NULL
    assert call(m=mat(k=48, nbytes=0)) == E_SHAPE
    assert call(r1=9) == E_RANGE
    assert call(nt=-1) == E_ARG
    assert call(xs=-1) == E_ARG
    assert call(ys=7) == E_ARG
    assert call(x=0) == E_NULL and call(y=0) == E_NULL
    assert call(nt=0, x=0, y=0) == 0
    assert call(r0=3, r1=3, x=0, y=0) == 0
    assert call(nt=1, ys=0, x=0) == E_NULL


def test_expert_windows_op_and_combine_validation():
    L = q.lib()
    ids = (ctypes.c_int32 * 2)(1, 3)
    mats = (q.qg_matrix * 1)(mat(rows=8 * 4, k=64))

    def call(in_op=0, eps=0.0, out_op=0, x=FAKE, x2=FAKE, n_sel=2, m=mats):
        return L.qgemv_expert_windows_op(m, 1, 4, ids, n_sel, x, x2, 64, in_op, eps, out_op, FAKE, 0, None)

    assert call(in_op=2) == E_ARG and call(in_op=4) == E_ARG and call(out_op=2) == E_ARG
    assert call(in_op=3, out_op=1) == E_ARG
    assert call(in_op=1, eps=-1.0) == E_ARG
    assert call(in_op=3, x2=0) == E_NULL
    assert call(x=0) == E_NULL
    assert call(n_sel=0, x=0, x2=0) == 0
    big = (q.qg_matrix * 1)(mat(rows=4, k=32768 + 32))
    assert call(in_op=1, m=big) == E_ARG  # the fused RMS takes k <= 32768
    assert L.qgemv_combine(FAKE, 8, 2, FAKE, -1, FAKE, None) == E_ARG
    assert L.qgemv_combine(FAKE, 7, 2, FAKE, 8, FAKE, None) == E_ARG  # expert outputs would overlap
    assert L.qgemv_combine(FAKE, 8, -1, FAKE, 8, FAKE, None) == E_ARG
    assert L.qgemv_combine(0, 8, 2, FAKE, 8, FAKE, None) == E_NULL
    assert L.qgemv_combine(FAKE, 8, 2, 0, 8, FAKE, None) == E_NULL
    assert L.qgemv_combine(FAKE, 8, 2, FAKE, 8, 0, None) == E_NULL
    assert L.qgemv_combine(0, 0, 0, 0, 0, 0, None) == 0


def test_swiglu_validation():
    L = q.lib()
    g, u = mat(rows=8, k=64), mat(rows=8, k=64)

    def rows(gm=None, um=None, r0=0, r1=8, x=FAKE, op=0, eps=0.0, h=FAKE, B=0):
        gm = g if gm is None else gm
        um = u if um is None else um
        return L.qgemv_rows_swiglu(ctypes.byref(gm), ctypes.byref(um), r0, r1, x, op, eps, h, B, None)

    assert L.qgemv_rows_swiglu(None, ctypes.byref(u), 0, 8, FAKE, 0, 0.0, FAKE, 0, None) == E_NULL
    assert rows(um=mat(rows=9, k=64)) == E_SHAPE
    assert rows(um=mat(fmt=2, rows=8, k=64)) == E_SHAPE
    assert rows(um=mat(rows=8, k=96)) == E_SHAPE
    assert rows(op=3) == E_ARG and rows(op=2) == E_ARG
    assert rows(op=1, eps=-1.0) == E_ARG
    assert rows(r1=9) == E_RANGE
    assert rows(B=-1) == E_ARG
    assert rows(x=0) == E_NULL and rows(h=0) == E_NULL
    assert rows(r0=4, r1=4, x=0, h=0) == 0
    ids = (ctypes.c_int32 * 2)(0, 3)
    eg, eu = mat(rows=16, k=64), mat(rows=16, k=64)

    def exp(n_expert=4, n_sel=2, x=FAKE, xs=64, op=0, h=FAKE, idp=ids):
        return L.qgemv_expert_swiglu(ctypes.byref(eg), ctypes.byref(eu), n_expert, idp, n_sel, x, xs, op, 0.0, h, 0,
                                     None)

    assert exp(n_expert=0) == E_SHAPE and exp(n_expert=3) == E_SHAPE
    assert exp(n_expert=2) == E_RANGE  # id 3 >= 2
    assert exp(n_sel=-1) == E_ARG and exp(n_sel=65) == E_ARG and exp(xs=-1) == E_ARG
    assert exp(idp=None) == E_NULL and exp(x=0) == E_NULL and exp(h=0) == E_NULL
    assert exp(n_sel=0, x=0, h=0) == 0


def test_rows_op_validation():
    L = q.lib()

    def call(m=None, r0=0, r1=8, x=FAKE, x2=FAKE, in_op=0, eps=1e-6, out_op=0, y=FAKE, B=0, k=64):
        m = mat(k=k) if m is None else m
        return L.qgemv_rows_op(ctypes.byref(m), r0, r1, x, x2, in_op, eps, out_op, y, B, None)

    assert L.qgemv_rows_op(None, 0, 8, FAKE, FAKE, 0, 0.0, 0, FAKE, 0, None) == E_NULL
    assert call(m=mat(fmt=6)) == E_FMT
    assert call(r1=9) == E_RANGE
    assert call(B=-1) == E_ARG
    assert call(in_op=2) == E_ARG  # GELU_RMS: GELU belongs to the producer (QG_OUT_GELU)
    assert call(in_op=4) == E_ARG and call(in_op=-1) == E_ARG
    assert call(out_op=2) == E_ARG
    assert call(in_op=1, eps=-1.0) == E_ARG
    assert call(in_op=1, eps=float("nan")) == E_ARG
    assert call(in_op=1, eps=float("inf")) == E_ARG
    big = 32768 + 32
    assert call(m=mat(k=big), in_op=1, k=big) == E_ARG  # fused RMS only where it matches qgemv_rms_carry
    assert call(x=0) == E_NULL and call(y=0) == E_NULL
    assert call(in_op=3, x2=0) == E_NULL
    assert call(r0=4, r1=4, x=0, y=0) == 0


def test_mapped_validation():
    # argument checks precede the page-locked check (which needs the runtime)
    L = q.lib()

    def call(m, r0=0, r1=8, x=FAKE, y=FAKE, B=0):
        return L.qgemv_mapped_rows(ctypes.byref(m) if m is not None else None, r0, r1, x, y, B, None)

    assert call(None) == E_NULL
    assert call(mat(fmt=6)) == E_FMT
    assert call(mat(k=48, nbytes=0)) == E_SHAPE
    assert call(mat(data=FAKE + 4)) == E_ARG
    assert call(mat(nbytes=8 * 2 * 34 - 1)) == E_SIZE
    assert call(mat(), r1=9) == E_RANGE
    assert call(mat(), B=-1) == E_ARG
    assert call(mat(), x=0) == E_NULL
    assert call(mat(), r0=2, r1=2, x=0, y=0) == 0
    assert L.qgemv_mapped_windows(1, 64, None, 1, 0, None) == E_NULL
    assert L.qgemv_mapped_windows(1, 64, None, 0, 0, None) == 0
    assert L.qgemv_mapped_windows(1, 48, None, 0, 0, None) == E_SHAPE
    assert L.qgemv_mapped_windows(1, 64, None, 65, 0, None) == E_ARG


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


def test_chain_struct_layout_matches_header():
    assert ctypes.sizeof(q.qg_chain_step) == 24
    assert ctypes.sizeof(q.qg_chain_window) == 56
    assert q.qg_chain_window.y.offset == 48 and q.qg_chain_step.eps.offset == 20


def cwin(r0=0, r1=8, rows=8, data=FAKE, x=FAKE, x2=0, y=FAKE):
    return q.qg_chain_window(data, rows, r0, r1, x, x2, y)


def cstep(k=64, first=0, n=1, op=0, eps=1e-6):
    return q.qg_chain_step(k, first, n, op, eps)


def test_chain_validation():
    """Every rejection happens before any HIP call, so it runs without a GPU."""
    L = q.lib()
    h = ctypes.c_void_p()

    def create(steps, wins, fmt=1, out=True):
        sa = (q.qg_chain_step * max(len(steps), 1))(*steps)
        wa = (q.qg_chain_window * max(len(wins), 1))(*wins)
        return L.qgemv_chain_create(fmt, sa, len(steps), wa, len(wins), ctypes.byref(h) if out else None)

    ok_w = [cwin(), cwin(2, 5)]
    assert create([cstep(n=2)], ok_w, out=False) == E_NULL
    assert L.qgemv_chain_create(1, None, 1, (q.qg_chain_window * 1)(cwin()), 1, ctypes.byref(h)) == E_NULL
    for f in (0, 4, 5, 6):  # the K-quants have no chain kernel
        assert create([cstep()], ok_w, fmt=f) == E_FMT
    assert create([], ok_w) == E_ARG
    assert create([cstep()], []) == E_ARG
    assert create([cstep(k=48)], ok_w) == E_SHAPE
    assert create([cstep(k=24576 + 32)], ok_w) == E_SHAPE
    assert create([cstep(op=4)], ok_w) == E_ARG
    assert create([cstep(op=-1)], ok_w) == E_ARG
    assert create([cstep(n=3)], ok_w) == E_ARG  # windows past the array
    assert create([cstep(first=-1)], ok_w) == E_ARG
    assert create([cstep(n=0)], ok_w) == E_ARG
    assert create([cstep(op=1, eps=-1.0)], ok_w) == E_ARG
    assert create([cstep(op=2, eps=float("nan"))], ok_w) == E_ARG
    assert create([cstep()], [cwin(4, 9)]) == E_RANGE
    assert create([cstep()], [cwin(rows=-1)]) == E_SHAPE
    assert create([cstep()], [cwin(data=FAKE + 4)]) == E_ARG
    assert create([cstep()], [cwin(x=0)]) == E_NULL
    assert create([cstep()], [cwin(y=0)]) == E_NULL
    assert create([cstep()], [cwin(data=0)]) == E_NULL
    assert create([cstep(op=3)], [cwin()]) == E_NULL  # SiLU * up needs x2
    # the RMS transforms normalise one vector: every non-empty window shares x
    assert create([cstep(op=1, n=2)], [cwin(), cwin(x=FAKE + 256)]) == E_ARG
    assert L.qgemv_chain_run(None, None) == E_NULL
    assert L.qgemv_chain_check(None) == E_NULL
    assert L.qgemv_chain_set_spin_limit(None, 1 << 20) == E_NULL
    assert L.qgemv_chain_grid(None) == E_NULL
    assert L.qgemv_chain_destroy(None) == 0


def test_chain_binding_checks_shapes():
    import torch
    w = q.Matrix(torch.zeros(8 * 2 * 34, dtype=torch.uint8), q.Q8_0, 8, 64)
    w2 = q.Matrix(torch.zeros(8 * 4 * 34, dtype=torch.uint8), q.Q8_0, 8, 128)
    x, y = torch.zeros(64), torch.zeros(8)
    with pytest.raises(ValueError):
        q._chain_tables([q.ChainStep([])])
    with pytest.raises(ValueError):
        q._chain_tables([q.ChainStep([q.ChainWindow(w, 0, 8, x, y), q.ChainWindow(w2, 0, 8, torch.zeros(128), y)])])
    with pytest.raises(ValueError):
        q._chain_tables([q.ChainStep([q.ChainWindow(w, 0, 8, torch.zeros(32), y)])])
    sa, ns, wa, nw = q._chain_tables([q.ChainStep([q.ChainWindow(w, 0, 8, x, y)], q.IN_RMS, 1e-5),
                                      q.ChainStep([q.ChainWindow(w, 2, 6, x, y, x2=x)], q.IN_SILU_MUL)])
    assert (ns, nw) == (2, 2)
    assert (sa[1].first_win, sa[1].n_win, sa[1].in_op, sa[0].k) == (1, 1, 3, 64)
    assert wa[1].x2 == x.data_ptr() and wa[0].x2 is None
