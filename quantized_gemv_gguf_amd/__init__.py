"""Python binding of libqgemv.so (include/qgemv.h): batch-1 dequant-GEMV over
GGUF block-quantized weights (Q8_0, Q4_0, MXFP4, Q4_K, Q6_K) on MI355X.

The functions carry the C names and do argument marshalling only: torch
tensors are turned into raw pointers and sizes, the caller's torch stream into
a ``hipStream_t``, and a negative status into :class:`QgemvError`.  Every step
of the computation runs in the library's HIP kernels; there is no other path.
If ``libqgemv.so`` is missing, importing works but every call raises.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Sequence

Q8_0, Q4_0, MXFP4, Q4_K, Q6_K = 1, 2, 3, 4, 5
FORMATS = {"q8_0": Q8_0, "q4_0": Q4_0, "mxfp4": MXFP4, "q4_k": Q4_K, "q6_k": Q6_K}
MAX_WINDOWS = 64
MAX_K = 49152
CHAIN_MAX_K = 24576
IN_X, IN_RMS, IN_GELU_RMS, IN_SILU_MUL = 0, 1, 2, 3
OUT_Y, OUT_GELU = 0, 1

QG_OK = 0
STATUS = {
    -1: "QG_E_NULL", -2: "QG_E_FMT", -3: "QG_E_SHAPE", -4: "QG_E_RANGE", -5: "QG_E_SIZE",
    -6: "QG_E_ARG", -7: "QG_E_NOT_PINNED", -8: "QG_E_CAPACITY", -9: "QG_E_BARRIER", -100: "QG_E_HIP",
}

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqgemv.so")

_i32, _i64, _vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p


class QgemvError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str = ""):
        self.status = status
        self.name = STATUS.get(status, str(status))
        msg = f"{where}: {self.name} ({status})"
        if detail:
            msg += f": {detail}"
        super().__init__(msg)


class qg_matrix(ctypes.Structure):
    _fields_ = [("data", _vp), ("fmt", _i32), ("reserved", _i32), ("n_rows", _i64), ("k", _i64),
                ("n_bytes", _i64)]


class qg_window(ctypes.Structure):
    _fields_ = [("data", _vp), ("n_rows", _i64), ("row_start", _i64), ("row_end", _i64),
                ("x", _vp), ("y", _vp)]


class qg_plan_step(ctypes.Structure):
    _fields_ = [("op", _i32), ("fmt", _i32), ("k", _i64), ("first_win", _i32), ("n_win", _i32),
                ("block_rows", _i64), ("a", _vp), ("b", _vp), ("out", _vp), ("n", _i64), ("stride", _i64),
                ("n_sel", _i32), ("reserved", _i32)]


class qg_chain_window(ctypes.Structure):
    _fields_ = [("data", _vp), ("n_rows", _i64), ("row_start", _i64), ("row_end", _i64),
                ("x", _vp), ("x2", _vp), ("y", _vp)]


class qg_chain_step(ctypes.Structure):
    _fields_ = [("k", _i64), ("first_win", _i32), ("n_win", _i32), ("in_op", _i32), ("eps", ctypes.c_float)]


_lib = None


def lib():
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built (run __graft_entry__.build() or "
                           "python quantized_gemv_gguf_amd/build.py); there is no fallback path")
    L = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER
    sigs = {
        "qgemv_block_bytes": ([_i32], _i64),
        "qgemv_block_weights": ([_i32], _i64),
        "qgemv_weight_bytes": ([_i32, _i64, _i64], _i64),
        "qgemv_rows": ([P(qg_matrix), _i64, _i64, _vp, _vp, _i64, _vp], ctypes.c_int),
        "qgemv_windows": ([_i32, _i64, P(qg_window), _i32, _i64, _vp], ctypes.c_int),
        "qgemv_rows_batch": ([P(qg_matrix), _i64, _i64, _vp, _i64, _i32, _vp, _i64, _i64, _vp], ctypes.c_int),
        "qgemv_rows_mfma": ([P(qg_matrix), _i64, _i64, _vp, _i64, _i32, _vp, _i64, _vp], ctypes.c_int),
        "qgemv_expert_windows_op": ([P(qg_matrix), _i32, _i64, P(_i32), _i32, _vp, _vp, _i64, _i32, ctypes.c_float,
                                     _i32, _vp, _i64, _vp], ctypes.c_int),
        "qgemv_combine": ([_vp, _i64, _i32, _vp, _i64, _vp, _vp], ctypes.c_int),
        "qgemv_rows_swiglu": ([P(qg_matrix), P(qg_matrix), _i64, _i64, _vp, _i32, ctypes.c_float, _vp, _i64, _vp],
                              ctypes.c_int),
        "qgemv_expert_swiglu": ([P(qg_matrix), P(qg_matrix), _i64, P(_i32), _i32, _vp, _i64, _i32, ctypes.c_float,
                                 _vp, _i64, _vp], ctypes.c_int),
        "qgemv_rows_op": ([P(qg_matrix), _i64, _i64, _vp, _vp, _i32, ctypes.c_float, _i32, _vp, _i64, _vp],
                          ctypes.c_int),
        "qgemv_expert_windows": ([P(qg_matrix), _i32, _i64, P(_i32), _i32, _vp, _i64, _vp, _i64, _vp],
                                 ctypes.c_int),
        "qgemv_silu_mul": ([_vp, _vp, _vp, _i64, _vp], ctypes.c_int),
        "qgemv_rms_carry": ([_vp, _vp, _i64, ctypes.c_float, _i32, _vp], ctypes.c_int),
        "qgemv_dequant_rows": ([P(qg_matrix), _i64, _i64, _vp, _vp], ctypes.c_int),
        "qgemv_read_ceiling": ([_vp, _i64, _vp, _vp], ctypes.c_int),
        "qgemv_stream_create": ([_i64, _i32, P(_vp)], ctypes.c_int),
        "qgemv_stream_ring_bytes": ([_vp], _i64),
        "qgemv_stream_rows": ([_vp, P(qg_matrix), _i64, _i64, _i64, _vp, _vp, _vp], ctypes.c_int),
        "qgemv_stream_windows": ([_vp, _i32, _i64, P(qg_window), _i32, _i64, _vp], ctypes.c_int),
        "qgemv_stream_destroy": ([_vp], ctypes.c_int),
        "qgemv_stream_plan_create": ([_i64, _i32, P(qg_plan_step), _i32, P(qg_window), _i32, P(_vp)],
                                     ctypes.c_int),
        "qgemv_stream_plan_set_rows": ([_vp, _i32, _i64], ctypes.c_int),
        "qgemv_stream_plan_ring_bytes": ([_vp], _i64),
        "qgemv_stream_plan_run": ([_vp, _vp], ctypes.c_int),
        "qgemv_stream_plan_destroy": ([_vp], ctypes.c_int),
        "qgemv_stream_rows_noalloc": ([P(qg_matrix), _i64, _i64, _i64, _vp, _vp, _vp], ctypes.c_int),
        "qgemv_mapped_rows": ([P(qg_matrix), _i64, _i64, _vp, _vp, _i64, _vp], ctypes.c_int),
        "qgemv_mapped_windows": ([_i32, _i64, P(qg_window), _i32, _i64, _vp], ctypes.c_int),
        "qgemv_chain_create": ([_i32, P(qg_chain_step), _i32, P(qg_chain_window), _i32, P(_vp)], ctypes.c_int),
        "qgemv_chain_run": ([_vp, _vp], ctypes.c_int),
        "qgemv_chain_check": ([_vp], ctypes.c_int),
        "qgemv_chain_set_spin_limit": ([_vp, ctypes.c_uint32], ctypes.c_int),
        "qgemv_chain_grid": ([_vp], _i64),
        "qgemv_chain_destroy": ([_vp], ctypes.c_int),
        "qgemv_strerror": ([ctypes.c_int], ctypes.c_char_p),
        "qgemv_last_hip_error": ([], ctypes.c_char_p),
        "qgemv_version": ([], ctypes.c_char_p),
    }
    for name, (args, res) in sigs.items():
        f = getattr(L, name)
        f.argtypes = args
        f.restype = res
    _lib = L
    return L


def _check(rc: int, where: str) -> None:
    if rc != QG_OK:
        detail = lib().qgemv_strerror(rc).decode()
        if rc == -100:
            detail += ": " + lib().qgemv_last_hip_error().decode()
        raise QgemvError(rc, where, detail)


# --- marshalling helpers ------------------------------------------------------

def _ptr(t) -> int:
    """Raw address of a tensor (contiguity required), or 0 for None."""
    if t is None:
        return 0
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _f32(t, n: int, name: str):
    import torch
    if t.dtype != torch.float32:
        raise TypeError(f"{name} must be float32")
    if t.numel() < n:
        raise ValueError(f"{name} holds {t.numel()} values, needs {n}")
    return _ptr(t)


@dataclass
class Matrix:
    """A quantized matrix: ``data`` is a uint8 tensor of the raw blocks (device
    memory for the resident calls, pinned host memory for the streamed ones)."""
    data: object
    fmt: int
    n_rows: int
    k: int

    def c(self) -> qg_matrix:
        return qg_matrix(_ptr(self.data), int(self.fmt), 0, int(self.n_rows), int(self.k),
                         int(self.data.numel() * self.data.element_size()))


@dataclass
class Window:
    """Rows [row_start, row_end) of ``mat`` with input ``x`` (k floats) and
    output ``y`` (row_end - row_start floats)."""
    mat: Matrix
    row_start: int
    row_end: int
    x: object
    y: object

    def c(self) -> qg_window:
        n = self.row_end - self.row_start
        return qg_window(_ptr(self.mat.data), int(self.mat.n_rows), int(self.row_start), int(self.row_end),
                         _f32(self.x, self.mat.k, "x"), _f32(self.y, max(n, 0), "y"))


def _windows(ws: Sequence[Window]):
    if len(ws) == 0:
        return None, 0, None, None
    fmt, k = ws[0].mat.fmt, ws[0].mat.k
    arr = (qg_window * len(ws))(*[w.c() for w in ws])
    return arr, len(ws), fmt, k


# --- entry points ----------------------------------------------------------------

def qgemv_block_bytes(fmt: int) -> int:
    return int(lib().qgemv_block_bytes(fmt))


def qgemv_block_weights(fmt: int) -> int:
    return int(lib().qgemv_block_weights(fmt))


def qgemv_weight_bytes(fmt: int, n_rows: int, k: int) -> int:
    return int(lib().qgemv_weight_bytes(fmt, n_rows, k))


def qgemv_rows(w: Matrix, row_start: int, row_end: int, x, y, block_rows: int = 0, stream=None) -> None:
    m = w.c()
    n = max(row_end - row_start, 0)
    _check(lib().qgemv_rows(ctypes.byref(m), row_start, row_end, _f32(x, w.k, "x"), _f32(y, n, "y"),
                            block_rows, _stream(stream)), "qgemv_rows")


def qgemv_rows_op(w: Matrix, row_start: int, row_end: int, x, y, in_op: int = 0, eps: float = 0.0,
                  out_op: int = 0, x2=None, block_rows: int = 0, stream=None) -> None:
    """As qgemv_rows with a fused input transform (IN_X, IN_RMS, IN_SILU_MUL with ``x2``)
    and output transform (OUT_Y, OUT_GELU)."""
    m = w.c()
    n = max(row_end - row_start, 0)
    x2p = _f32(x2, w.k, "x2") if x2 is not None else None
    _check(lib().qgemv_rows_op(ctypes.byref(m), row_start, row_end, _f32(x, w.k, "x"), x2p, int(in_op),
                               float(eps), int(out_op), _f32(y, n, "y"), block_rows, _stream(stream)),
           "qgemv_rows_op")


def qgemv_rows_batch(w: Matrix, row_start: int, row_end: int, x, y, block_rows: int = 0, stream=None) -> None:
    """y[t] = W[row_start:row_end] . x[t] for every token t: ``x`` is (n_tok, >= k)
    and ``y`` (n_tok, >= row_end - row_start), float32 with unit column stride."""
    m = w.c()
    n = max(row_end - row_start, 0)
    if x.dim() != 2 or y.dim() != 2 or x.shape[0] != y.shape[0]:
        raise ValueError("x and y must be (n_tok, ...) with the same n_tok")
    if x.stride(1) != 1 or y.stride(1) != 1 or x.shape[1] < w.k or y.shape[1] < n:
        raise ValueError("rows of x (k floats) and y (one per output row) must be contiguous")
    nt = x.shape[0]
    _f32(x, 0, "x")
    _f32(y, 0, "y")
    _check(lib().qgemv_rows_batch(ctypes.byref(m), row_start, row_end, _ptr(x), x.stride(0), nt, _ptr(y),
                                  y.stride(0), block_rows, _stream(stream)), "qgemv_rows_batch")


def qgemv_rows_mfma(w: Matrix, row_start: int, row_end: int, x, y, stream=None) -> None:
    """As qgemv_rows_batch on the fp32 matrix cores (every format): y[t]
    within fp32 rounding of W[row_start:row_end] . x[t], not bit-identical to
    the one-token calls."""
    m = w.c()
    n = max(row_end - row_start, 0)
    if x.dim() != 2 or y.dim() != 2 or x.shape[0] != y.shape[0]:
        raise ValueError("x and y must be (n_tok, ...) with the same n_tok")
    if x.stride(1) != 1 or y.stride(1) != 1 or x.shape[1] < w.k or y.shape[1] < n:
        raise ValueError("rows of x (k floats) and y (one per output row) must be contiguous")
    nt = x.shape[0]
    _f32(x, 0, "x")
    _f32(y, 0, "y")
    _check(lib().qgemv_rows_mfma(ctypes.byref(m), row_start, row_end, _ptr(x), x.stride(0), nt, _ptr(y),
                                 y.stride(0), _stream(stream)), "qgemv_rows_mfma")


def qgemv_windows(windows: Sequence[Window], block_rows: int = 0, stream=None, fmt=None, k=None) -> None:
    arr, n, f, kk = _windows(windows)
    f = fmt if f is None else f
    kk = k if kk is None else kk
    _check(lib().qgemv_windows(int(f or Q8_0), int(kk or 32), arr, n, block_rows, _stream(stream)),
           "qgemv_windows")


def qgemv_expert_windows(mats: Sequence[Matrix], n_expert: int, ids, x, x_stride: int, y,
                         block_rows: int = 0, stream=None) -> None:
    ids = [int(i) for i in ids]
    marr = (qg_matrix * len(mats))(*[m.c() for m in mats])
    iarr = (_i32 * max(len(ids), 1))(*ids)
    k = mats[0].k if mats else 32
    out = (mats[0].n_rows // n_expert) if (mats and n_expert > 0) else 0
    xp = _f32(x, k + (len(ids) - 1) * x_stride if ids else 0, "x")
    yp = _f32(y, len(mats) * len(ids) * out, "y")
    _check(lib().qgemv_expert_windows(marr, len(mats), n_expert, iarr, len(ids), xp, x_stride, yp,
                                      block_rows, _stream(stream)), "qgemv_expert_windows")


def qgemv_expert_windows_op(mats: Sequence[Matrix], n_expert: int, ids, x, x_stride: int, y, in_op: int = 0,
                            eps: float = 0.0, out_op: int = 0, x2=None, block_rows: int = 0,
                            stream=None) -> None:
    """As qgemv_expert_windows with qgemv_rows_op's transforms per window (x2
    strided like x, for IN_SILU_MUL)."""
    ids = [int(i) for i in ids]
    marr = (qg_matrix * len(mats))(*[m.c() for m in mats])
    iarr = (_i32 * max(len(ids), 1))(*ids)
    k = mats[0].k if mats else 32
    out = (mats[0].n_rows // n_expert) if (mats and n_expert > 0) else 0
    need = k + (len(ids) - 1) * x_stride if ids else 0
    xp = _f32(x, need, "x")
    x2p = _f32(x2, need, "x2") if x2 is not None else None
    yp = _f32(y, len(mats) * len(ids) * out, "y")
    _check(lib().qgemv_expert_windows_op(marr, len(mats), n_expert, iarr, len(ids), xp, x2p, x_stride, int(in_op),
                                         float(eps), int(out_op), yp, block_rows, _stream(stream)),
           "qgemv_expert_windows_op")


def qgemv_rows_swiglu(gate: Matrix, up: Matrix, row_start: int, row_end: int, x, h, in_op: int = 0,
                      eps: float = 0.0, block_rows: int = 0, stream=None) -> None:
    """h = silu(gate[rows] . x') * (up[rows] . x'), x' = x (IN_X) or rms(x) (IN_RMS)."""
    g, u = gate.c(), up.c()
    n = max(row_end - row_start, 0)
    _check(lib().qgemv_rows_swiglu(ctypes.byref(g), ctypes.byref(u), row_start, row_end, _f32(x, gate.k, "x"),
                                   int(in_op), float(eps), _f32(h, n, "h"), block_rows, _stream(stream)),
           "qgemv_rows_swiglu")


def qgemv_expert_swiglu(gate: Matrix, up: Matrix, n_expert: int, ids, x, x_stride: int, h, in_op: int = 0,
                        eps: float = 0.0, block_rows: int = 0, stream=None) -> None:
    ids = [int(i) for i in ids]
    g, u = gate.c(), up.c()
    iarr = (_i32 * max(len(ids), 1))(*ids)
    out = gate.n_rows // n_expert if n_expert > 0 else 0
    xp = _f32(x, gate.k + (len(ids) - 1) * x_stride if ids else 0, "x")
    _check(lib().qgemv_expert_swiglu(ctypes.byref(g), ctypes.byref(u), n_expert, iarr, len(ids), xp, x_stride,
                                     int(in_op), float(eps), _f32(h, len(ids) * out, "h"), block_rows,
                                     _stream(stream)), "qgemv_expert_swiglu")


def qgemv_combine(y, y_stride: int, n_sel: int, w, n: int, out, stream=None) -> None:
    """out[i] = sum_s w[s] * y[s * y_stride + i] (device tensors)."""
    yp = _f32(y, (n_sel - 1) * y_stride + n if n_sel > 0 else 0, "y")
    wp = _f32(w, n_sel, "w")
    _check(lib().qgemv_combine(yp, y_stride, n_sel, wp, n, _f32(out, n, "out"), _stream(stream)), "qgemv_combine")


def qgemv_mapped_rows(w: Matrix, row_start: int, row_end: int, x, y, block_rows: int = 0,
                      stream=None) -> None:
    """As qgemv_rows, with ``w.data`` a pinned host tensor read in place over the host link."""
    m = w.c()
    n = max(row_end - row_start, 0)
    _check(lib().qgemv_mapped_rows(ctypes.byref(m), row_start, row_end, _f32(x, w.k, "x"), _f32(y, n, "y"),
                                   block_rows, _stream(stream)), "qgemv_mapped_rows")


def qgemv_mapped_windows(windows: Sequence[Window], block_rows: int = 0, stream=None, fmt=None, k=None) -> None:
    """As qgemv_windows, with every window's matrix in pinned host memory."""
    arr, n, f, kk = _windows(windows)
    f = fmt if f is None else f
    kk = k if kk is None else kk
    _check(lib().qgemv_mapped_windows(int(f or Q8_0), int(kk or 32), arr, n, block_rows, _stream(stream)),
           "qgemv_mapped_windows")


def qgemv_silu_mul(g, u, h, stream=None) -> None:
    n = h.numel()
    _check(lib().qgemv_silu_mul(_f32(g, n, "g"), _f32(u, n, "u"), _f32(h, n, "h"), n, _stream(stream)),
           "qgemv_silu_mul")


def qgemv_rms_carry(v, out, eps: float = 1e-6, gelu: bool = False, stream=None) -> None:
    n = v.numel()
    _check(lib().qgemv_rms_carry(_f32(v, n, "v"), _f32(out, n, "out"), n, float(eps), int(bool(gelu)),
                                 _stream(stream)), "qgemv_rms_carry")


def qgemv_read_ceiling(data, sink, stream=None) -> None:
    """One plain streaming read of the device tensor ``data`` (its whole
    storage; a multiple of 16 bytes); the xor of what was read is xor-ed into
    the uint32/int32 device tensor ``sink``."""
    n = data.numel() * data.element_size()
    if not data.is_cuda or not sink.is_cuda or sink.element_size() != 4:
        raise ValueError("data and sink must be device tensors, sink 32-bit")
    _check(lib().qgemv_read_ceiling(_ptr(data), n, _ptr(sink), _stream(stream)), "qgemv_read_ceiling")


def qgemv_dequant_rows(w: Matrix, row_start: int, row_end: int, out, stream=None) -> None:
    m = w.c()
    n = max(row_end - row_start, 0) * w.k
    _check(lib().qgemv_dequant_rows(ctypes.byref(m), row_start, row_end, _f32(out, n, "out"),
                                    _stream(stream)), "qgemv_dequant_rows")


class Streamer:
    """Owner of a qg_streamer: lookahead + 1 device slots of slot_bytes each."""

    def __init__(self, slot_bytes: int, lookahead: int):
        h = _vp()
        _check(lib().qgemv_stream_create(int(slot_bytes), int(lookahead), ctypes.byref(h)),
               "qgemv_stream_create")
        self._h = h
        self.slot_bytes = int(slot_bytes)
        self.lookahead = int(lookahead)

    @property
    def ring_bytes(self) -> int:
        return int(lib().qgemv_stream_ring_bytes(self._h))

    def rows(self, w: Matrix, row_start: int, row_end: int, x, y, block_rows: int = 0, stream=None) -> None:
        m = w.c()
        n = max(row_end - row_start, 0)
        _check(lib().qgemv_stream_rows(self._h, ctypes.byref(m), row_start, row_end, block_rows,
                                       _f32(x, w.k, "x"), _f32(y, n, "y"), _stream(stream)),
               "qgemv_stream_rows")

    def windows(self, windows: Sequence[Window], block_rows: int = 0, stream=None) -> None:
        arr, n, f, k = _windows(windows)
        _check(lib().qgemv_stream_windows(self._h, int(f or Q8_0), int(k or 32), arr, n, block_rows,
                                          _stream(stream)), "qgemv_stream_windows")

    def close(self) -> None:
        if getattr(self, "_h", None) is not None and self._h.value:
            h, self._h = self._h, None
            _check(lib().qgemv_stream_destroy(h), "qgemv_stream_destroy")

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


PLAN_GEMV, PLAN_SILU_MUL, PLAN_COMBINE = 1, 2, 3


@dataclass
class PlanGemv:
    """A streamed GEMV step of a plan: its windows (same fmt and k; data in
    pinned host memory) walked in blocks of block_rows."""
    windows: Sequence[Window]
    block_rows: int = 0


@dataclass
class PlanSiluMul:
    """h = silu(g) * u between the steps of a plan."""
    g: object
    u: object
    h: object


@dataclass
class PlanCombine:
    """out = sum_s w[s] y[s] (as qgemv_combine) between the steps of a plan."""
    y: object
    y_stride: int
    n_sel: int
    w: object
    n: int
    out: object


class StreamPlan:
    """Owner of a qg_stream_plan: a fixed walk of streamed GEMV steps and
    elementwise steps, replayed by run()."""

    def __init__(self, slot_bytes: int, lookahead: int, steps):
        wins, cs = [], []
        for st in steps:
            if isinstance(st, PlanGemv):
                first = len(wins)
                fmt, k = st.windows[0].mat.fmt, st.windows[0].mat.k
                wins.extend(st.windows)
                cs.append(qg_plan_step(PLAN_GEMV, int(fmt), int(k), first, len(st.windows), int(st.block_rows),
                                       None, None, None, 0, 0, 0, 0))
            elif isinstance(st, PlanSiluMul):
                n = st.h.numel()
                cs.append(qg_plan_step(PLAN_SILU_MUL, 0, 0, 0, 0, 0, _f32(st.g, n, "g"), _f32(st.u, n, "u"),
                                       _f32(st.h, n, "h"), n, 0, 0, 0))
            elif isinstance(st, PlanCombine):
                cs.append(qg_plan_step(PLAN_COMBINE, 0, 0, 0, 0, 0, _ptr(st.y), _ptr(st.w), _f32(st.out, st.n, "out"),
                                       int(st.n), int(st.y_stride), int(st.n_sel), 0))
            else:
                raise TypeError(f"not a plan step: {st!r}")
        sarr = (qg_plan_step * len(cs))(*cs)
        warr = (qg_window * max(len(wins), 1))(*[w.c() for w in wins])
        h = _vp()
        _check(lib().qgemv_stream_plan_create(int(slot_bytes), int(lookahead), sarr, len(cs), warr, len(wins),
                                              ctypes.byref(h)), "qgemv_stream_plan_create")
        self._h = h
        self._keep = list(steps)  # the tensors must outlive the plan

    @property
    def ring_bytes(self) -> int:
        return int(lib().qgemv_stream_plan_ring_bytes(self._h))

    def set_rows(self, w: int, row_start: int) -> None:
        _check(lib().qgemv_stream_plan_set_rows(self._h, int(w), int(row_start)), "qgemv_stream_plan_set_rows")

    def run(self, stream=None) -> None:
        _check(lib().qgemv_stream_plan_run(self._h, _stream(stream)), "qgemv_stream_plan_run")

    def close(self) -> None:
        if getattr(self, "_h", None) is not None and self._h.value:
            h, self._h = self._h, None
            _check(lib().qgemv_stream_plan_destroy(h), "qgemv_stream_plan_destroy")

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


NOALLOC_RING_BYTES = 32 << 20


def qgemv_stream_rows_noalloc(w: Matrix, row_start: int, row_end: int, x, y, block_rows: int = 0,
                              stream=None) -> None:
    """Streamed rows through the library's own two-slot ring (no allocation;
    blocks up to NOALLOC_RING_BYTES / 2 bytes; calls must not overlap on a GPU)."""
    m = w.c()
    n = max(row_end - row_start, 0)
    _check(lib().qgemv_stream_rows_noalloc(ctypes.byref(m), row_start, row_end, block_rows, _f32(x, w.k, "x"),
                                           _f32(y, n, "y"), _stream(stream)), "qgemv_stream_rows_noalloc")


def qgemv_stream_create(slot_bytes: int, lookahead: int) -> Streamer:
    return Streamer(slot_bytes, lookahead)


@dataclass
class ChainWindow:
    """Rows [row_start, row_end) of ``mat``: y = W[row_start:row_end] . op(x),
    op the step's input transform (``x2`` is the multiplier of IN_SILU_MUL)."""
    mat: Matrix
    row_start: int
    row_end: int
    x: object
    y: object
    x2: object = None


@dataclass
class ChainStep:
    """One step of a chain: its windows (same fmt and k) and input transform."""
    windows: Sequence[ChainWindow]
    in_op: int = IN_X
    eps: float = 1e-6


def _chain_tables(steps: Sequence[ChainStep]):
    wins, cs = [], []
    for st in steps:
        if not st.windows:
            raise ValueError("a chain step needs at least one window")
        k = st.windows[0].mat.k
        first = len(wins)
        for w in st.windows:
            if w.mat.k != k:
                raise ValueError("the windows of a chain step must share k")
            n = max(w.row_end - w.row_start, 0)
            x2 = _f32(w.x2, k, "x2") if w.x2 is not None else 0
            wins.append(qg_chain_window(_ptr(w.mat.data), int(w.mat.n_rows), int(w.row_start), int(w.row_end),
                                        _f32(w.x, k, "x"), x2, _f32(w.y, n, "y")))
        cs.append(qg_chain_step(int(k), first, len(st.windows), int(st.in_op), float(st.eps)))
    return (qg_chain_step * len(cs))(*cs), len(cs), (qg_chain_window * len(wins))(*wins), len(wins)


class Chain:
    """Owner of a qg_chain: the steps run in order by one launch per run()."""

    def __init__(self, fmt: int, steps: Sequence[ChainStep]):
        sarr, ns, warr, nw = _chain_tables(steps)
        h = _vp()
        _check(lib().qgemv_chain_create(int(fmt), sarr, ns, warr, nw, ctypes.byref(h)), "qgemv_chain_create")
        self._h = h
        self._keep = list(steps)  # the tensors must outlive the chain
        self.fmt = int(fmt)
        self.n_steps = ns

    @property
    def grid(self) -> int:
        return int(lib().qgemv_chain_grid(self._h))

    @property
    def handle(self) -> int:
        return int(self._h.value)

    def run(self, stream=None) -> None:
        _check(lib().qgemv_chain_run(self._h, _stream(stream)), "qgemv_chain_run")

    def check(self) -> None:
        _check(lib().qgemv_chain_check(self._h), "qgemv_chain_check")

    def set_spin_limit(self, polls: int) -> None:
        """Polls (>= 1) a barrier waits before it gives up (default 2^22)."""
        _check(lib().qgemv_chain_set_spin_limit(self._h, int(polls)), "qgemv_chain_set_spin_limit")

    def close(self) -> None:
        if getattr(self, "_h", None) is not None and self._h.value:
            h, self._h = self._h, None
            _check(lib().qgemv_chain_destroy(h), "qgemv_chain_destroy")

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def qgemv_chain_create(fmt: int, steps: Sequence[ChainStep]) -> Chain:
    return Chain(fmt, steps)


def qgemv_version() -> str:
    return lib().qgemv_version().decode()
