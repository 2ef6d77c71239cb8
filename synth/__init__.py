"""Seeded synthetic inputs shared by the tests, the benchmark and the oracle.

This module holds generators only: it writes quant blocks directly as bytes
(scales and codes drawn from the stated distributions), fp32 activation
vectors and expert ids.  It decodes nothing, multiplies nothing and holds no
table of the formats' values, so it carries none of the GEMV's arithmetic.

Every generator is a pure function of its seed: quant blocks come from the
counter-based generator in ``synth.c`` (SplitMix64 output function, built with
gcc), activations and expert ids from numpy ``Generator(PCG64)``.  Seeds
follow ``1000 * cfg + tensor_id`` for the five workloads below.

Block layouts written here (byte order little-endian):
  Q8_0  (34 B): fp16 scale bits, then 32 int8 codes
  Q4_0  (18 B): fp16 scale bits, then 16 bytes of packed 4-bit codes
  MXFP4 (17 B): E8M0 scale byte, then 16 bytes of packed 4-bit codes
and per 256-weight super-block:
  Q4_K (144 B): fp16 d, fp16 dmin, 12 bytes of packed scales/mins, 128 bytes
                of packed 4-bit codes
  Q6_K (210 B): 128 bytes of low nibbles, 64 bytes of 2-bit high parts,
                16 int8 scales, fp16 d
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

Q8_0, Q4_0, MXFP4, Q4_K, Q6_K = 1, 2, 3, 4, 5
FMT_NAMES = {Q8_0: "q8_0", Q4_0: "q4_0", MXFP4: "mxfp4", Q4_K: "q4_k", Q6_K: "q6_k"}
BLOCK_BYTES = {Q8_0: 34, Q4_0: 18, MXFP4: 17, Q4_K: 144, Q6_K: 210}
BLOCK_WEIGHTS = {Q8_0: 32, Q4_0: 32, MXFP4: 32, Q4_K: 256, Q6_K: 256}


def rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "synth.c")
_LIB = os.path.join(_HERE, "libsynth.so")
_lib = None


def build() -> str:
    tmp = _LIB + ".tmp"
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread", _SRC, "-o", tmp, "-lm"], check=True)
    os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        L = ctypes.CDLL(_LIB)
        L.synth_fill.argtypes = [ctypes.c_int32, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                 ctypes.c_uint64, ctypes.c_double, ctypes.c_double, ctypes.c_int32, ctypes.c_int32,
                                 ctypes.c_int32, ctypes.c_int32]
        L.synth_fill.restype = ctypes.c_int
        L.synth_word.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_uint64]
        L.synth_word.restype = ctypes.c_uint64
        L.synth_half_bits.argtypes = [ctypes.c_double]
        L.synth_half_bits.restype = ctypes.c_uint16
        _lib = L
    return _lib


DEFAULTS = {
    Q8_0: dict(scale_lo=1e-3, scale_hi=1e-2, random_sign=True),
    Q4_0: dict(scale_lo=1e-3, scale_hi=1e-2, random_sign=False),
    MXFP4: dict(e_lo=118, e_hi=130),
    Q4_K: dict(scale_lo=1e-4, scale_hi=1e-3, random_sign=False),
    Q6_K: dict(scale_lo=1e-4, scale_hi=1e-3, random_sign=False),
}


def row_bytes(fmt: int, k: int) -> int:
    return (k // BLOCK_WEIGHTS[fmt]) * BLOCK_BYTES[fmt]


def blocks(fmt: int, n_rows: int, k: int, seed: int, r0: int = 0, r1: int | None = None, out=None,
           threads: int | None = None, **p) -> np.ndarray:
    """Rows [r0, r1) of the seeded (n_rows, k/32 * block_bytes) uint8 matrix.

    Every block is drawn from its own counter range (synth.c), so a row range
    can be regenerated alone and the bytes do not depend on the thread count.
      Q8_0 : d ~ fp16(U[1e-3, 1e-2)) * (+-1), q ~ U{-127..127}
      Q4_0 : d ~ fp16(U[1e-3, 1e-2)), every code byte ~ U{0..255}
      MXFP4: e ~ U{118..130}, every code byte ~ U{0..255}
      Q4_K : d ~ fp16(U[1e-4, 1e-3)), dmin = 8 d, sub-block scales sc ~ U{0..63},
             mins m = round(15 sc / 16) (centred sub-blocks), code bytes ~ U{0..255}
      Q6_K : d ~ fp16(U[1e-4, 1e-3)), code bytes ~ U{0..255}, scales ~ U{-127..127}
    ``out`` (optional) is a C-contiguous uint8 array of the result's shape.
    """
    assert k % BLOCK_WEIGHTS[fmt] == 0 and k > 0
    r1 = n_rows if r1 is None else r1
    assert 0 <= r0 <= r1 <= n_rows
    q = dict(DEFAULTS[fmt])
    q.update(p)
    rb = row_bytes(fmt, k)
    if out is None:
        out = np.empty((r1 - r0, rb), dtype=np.uint8)
    assert out.dtype == np.uint8 and out.flags.c_contiguous and out.size == (r1 - r0) * rb
    t = threads or int(os.environ.get("OMP_NUM_THREADS", 0) or (os.cpu_count() or 1))
    rc = _load().synth_fill(fmt, out.ctypes.data, k, r0, r1, seed & (2 ** 64 - 1), float(q.get("scale_lo", 1e-3)),
                            float(q.get("scale_hi", 1e-2)), int(bool(q.get("random_sign", False))),
                            int(q.get("e_lo", 118)), int(q.get("e_hi", 130)), min(t, 64))
    if rc != 0:
        raise ValueError("synth_fill rejected the arguments")
    return out.reshape(r1 - r0, rb)


def q8_0_blocks(n_rows, k, seed, **p):
    return blocks(Q8_0, n_rows, k, seed, **p)


def q4_0_blocks(n_rows, k, seed, **p):
    return blocks(Q4_0, n_rows, k, seed, **p)


def mxfp4_blocks(n_rows, k, seed, **p):
    return blocks(MXFP4, n_rows, k, seed, **p)


def random_bytes(fmt: int, n_rows: int, k: int, seed: int) -> np.ndarray:
    """Blocks with every byte uniform (scales included): exercises every scale
    pattern, NaN/inf/subnormal scales among them, for the bit-exact decode checks."""
    g = rng(seed)
    return g.integers(0, 256, size=(n_rows, row_bytes(fmt, k)), dtype=np.uint8)


def x_vec(k: int, seed: int) -> np.ndarray:
    """fp32 activations ~ N(0, 1)."""
    return rng(seed).standard_normal(k).astype(np.float32)


def expert_ids(n_expert: int, n_sel: int, n_tokens: int, seed: int) -> np.ndarray:
    """(n_tokens, n_sel) int32: per token, n_sel distinct ids drawn uniformly
    without replacement from [0, n_expert), listed in ascending order."""
    g = rng(seed)
    ids = np.stack([np.sort(g.choice(n_expert, n_sel, replace=False)) for _ in range(n_tokens)])
    return ids.astype(np.int32)


def router_weights(n_tokens: int, n_sel: int, seed: int) -> np.ndarray:
    """(n_tokens, n_sel) float32 mixing weights of the selected experts: per
    token, uniform draws in [0.05, 1) scaled to sum to 1."""
    g = rng(seed)
    u = g.uniform(0.05, 1.0, size=(n_tokens, n_sel))
    return (u / u.sum(axis=1, keepdims=True)).astype(np.float32)


# --- the workloads ----------------------------------------------------------------

def seed_of(cfg: int, tensor_id: int) -> int:
    return 1000 * cfg + tensor_id


CONFIGS = {
    1: dict(name="q8_0_256x1024", fmt=Q8_0, rows=256, k=1024),
    2: dict(name="q4_0_4096x4096", fmt=Q4_0, rows=4096, k=4096, block_rows=(0, 512)),
    3: dict(name="q8_0_ffn_11008x4096_streamed", fmt=Q8_0, hidden=4096, ffn=11008,
            block_rows=(128, 512, 2048), lookahead=2),
    4: dict(name="mxfp4_moe_128x2880x2880_top4", fmt=MXFP4, n_expert=128, out=2880, k=2880,
            n_sel=4, tokens=64, block_rows=(0, 128, 512)),
    5: dict(name="q8_0_dense20b_44L_h6144_f24576", fmt=Q8_0, layers=44, hidden=6144, ffn=24576,
            tokens=32, fmts=(Q8_0, Q8_0, Q8_0, Q8_0)),
    # the same pass in the K-quant mix of a "Q4_K_M" file: Q4_K with a Q6_K
    # down projection (12.9 GB resident)
    6: dict(name="q4_k_m_dense20b_44L_h6144_f24576", fmt=Q4_K, layers=44, hidden=6144, ffn=24576,
            tokens=32, fmts=(Q4_K, Q4_K, Q4_K, Q6_K)),
}


def dense_layer_shapes(hidden: int = 6144, ffn: int = 24576):
    """(name, rows, k) of the four weight matrices of one dense decoder layer."""
    return [("qkv", 3 * hidden, hidden), ("out", hidden, hidden), ("up", ffn, hidden), ("down", hidden, ffn)]
