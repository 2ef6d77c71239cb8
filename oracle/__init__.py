"""CPU oracle for the batch-1 dequant-GEMV over GGUF blocks (Q8_0, Q4_0, MXFP4,
Q4_K, Q6_K).

TEST INFRASTRUCTURE ONLY.  Only the test suite, the package smoke check and the
CPU-baseline leg of the benchmark may import this module.  It shares no code
with the HIP library: the arithmetic lives in ``oracle.c`` (plain scalar C,
fp64 sums), built here with gcc and called through ctypes.

Functions (each follows the passage cited in ``oracle.c``):

* ``dequant_rows(fmt, w, n_rows, k, r0, r1)`` -> fp32 ``(r1-r0, k)``: the block
  decoders of RAMforge README "Milestone 5" (Q8_0 ``d*q``, Q4_0 ``d*(q-8)``,
  Q4_K ``d*sc*q - dmin*m`` over 256-weight super-blocks), the 17-byte MXFP4
  block implied by neurostream README "The idea", and Q6_K in GGUF's layout
  (the pages name it without printing its layout).
* ``gemv_rows(fmt, w, n_rows, k, r0, r1, x)`` -> ``(y, a)`` in fp64, with
  ``y[j] = sum_i W[r0+j, i] x[i]`` (RAMforge README "Milestone 6", matrix
  layout) and ``a[j] = sum_i |W[r0+j, i] x[i]|``.
* ``silu_mul(g, u)``, ``rms_carry(v, eps, gelu)`` and ``combine(y, w)`` (the
  router-weighted sum of expert outputs) in fp64.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

Q8_0, Q4_0, MXFP4, Q4_K, Q6_K = 1, 2, 3, 4, 5

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-pthread"]

_lib = None


def build(src: str = _SRC, out: str = _LIB) -> str:
    """Compile the oracle with gcc (no fast-math, no intrinsics)."""
    tmp = out + ".tmp"
    subprocess.run(["gcc", *CFLAGS, src, "-o", tmp, "-lm"], check=True)
    os.replace(tmp, out)
    return out


def load(path: str | None = None):
    """Load (building first if absent) and declare the C signatures."""
    global _lib
    if path is None and _lib is not None:
        return _lib
    p = path or _LIB
    if not os.path.exists(p) or (path is None and os.path.getmtime(p) < os.path.getmtime(_SRC)):
        build(out=p)
    lib = ctypes.CDLL(p)
    i32, i64, vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p
    lib.orc_block_bytes.argtypes = [i32]
    lib.orc_block_bytes.restype = i64
    lib.orc_block_weights.argtypes = [i32]
    lib.orc_block_weights.restype = i64
    lib.orc_row_bytes.argtypes = [i32, i64]
    lib.orc_row_bytes.restype = i64
    lib.orc_half_to_double.argtypes = [ctypes.c_uint16]
    lib.orc_half_to_double.restype = ctypes.c_double
    lib.orc_half_to_double_n.argtypes = [vp, vp, i64]
    lib.orc_half_to_double_n.restype = None
    lib.orc_dequant_rows.argtypes = [i32, vp, i64, i64, i64, i64, vp]
    lib.orc_dequant_rows.restype = ctypes.c_int
    lib.orc_gemv_rows.argtypes = [i32, vp, i64, i64, i64, i64, vp, vp, vp, i32]
    lib.orc_gemv_rows.restype = ctypes.c_int
    lib.orc_silu_mul.argtypes = [vp, vp, vp, i64]
    lib.orc_silu_mul.restype = None
    lib.orc_rms_carry.argtypes = [vp, vp, i64, ctypes.c_double, i32]
    lib.orc_rms_carry.restype = None
    lib.orc_combine.argtypes = [vp, i64, i32, vp, i64, vp]
    lib.orc_combine.restype = None
    if path is None:
        _lib = lib
    return lib


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def block_bytes(fmt: int, lib=None) -> int:
    return int((lib or load()).orc_block_bytes(fmt))


def block_weights(fmt: int, lib=None) -> int:
    return int((lib or load()).orc_block_weights(fmt))


def row_bytes(fmt: int, k: int, lib=None) -> int:
    return int((lib or load()).orc_row_bytes(fmt, k))


def half_to_double(bits: np.ndarray, lib=None) -> np.ndarray:
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    out = np.empty(bits.shape, dtype=np.float64)
    (lib or load()).orc_half_to_double_n(_ptr(bits), _ptr(out), bits.size)
    return out


def _as_bytes(w) -> np.ndarray:
    w = np.ascontiguousarray(w)
    if w.dtype != np.uint8:
        w = w.view(np.uint8)
    return w


def dequant_rows(fmt, w, n_rows, k, r0=0, r1=None, lib=None) -> np.ndarray:
    r1 = n_rows if r1 is None else r1
    w = _as_bytes(w)
    out = np.empty((max(r1 - r0, 0), k), dtype=np.float32)
    rc = (lib or load()).orc_dequant_rows(fmt, _ptr(w), n_rows, k, r0, r1, _ptr(out))
    if rc != 0:
        raise ValueError("oracle rejected the arguments")
    return out


def gemv_rows(fmt, w, n_rows, k, x, r0=0, r1=None, threads=None, lib=None):
    """Return (y, a) as fp64 arrays of length r1 - r0."""
    r1 = n_rows if r1 is None else r1
    w = _as_bytes(w)
    x = np.ascontiguousarray(x, dtype=np.float32)
    if x.size != k:
        raise ValueError("x must hold k values")
    n = max(r1 - r0, 0)
    y = np.empty(n, dtype=np.float64)
    a = np.empty(n, dtype=np.float64)
    t = threads if threads is not None else (os.cpu_count() or 1)
    rc = (lib or load()).orc_gemv_rows(fmt, _ptr(w), n_rows, k, r0, r1, _ptr(x), _ptr(y), _ptr(a), t)
    if rc != 0:
        raise ValueError("oracle rejected the arguments")
    return y, a


def silu_mul(g, u, lib=None) -> np.ndarray:
    g = np.ascontiguousarray(g, dtype=np.float64)
    u = np.ascontiguousarray(u, dtype=np.float64)
    h = np.empty_like(g)
    (lib or load()).orc_silu_mul(_ptr(g), _ptr(u), _ptr(h), g.size)
    return h


def rms_carry(v, eps=1e-6, gelu=False, lib=None) -> np.ndarray:
    v = np.ascontiguousarray(v, dtype=np.float64)
    out = np.empty_like(v)
    (lib or load()).orc_rms_carry(_ptr(v), _ptr(out), v.size, float(eps), int(bool(gelu)))
    return out


def combine(y, w, lib=None) -> np.ndarray:
    """out = sum_s w[s] * y[s] in fp64; y is (n_sel, n)."""
    y = np.ascontiguousarray(y, dtype=np.float64)
    w = np.ascontiguousarray(w, dtype=np.float64)
    n_sel, n = y.shape
    out = np.empty(n, dtype=np.float64)
    (lib or load()).orc_combine(_ptr(y), n, n_sel, _ptr(w), n, _ptr(out))
    return out
