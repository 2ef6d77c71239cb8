"""Seeded synthetic inputs shared by the tests, the benchmark and the oracle.

This module holds generators only: it writes quant blocks directly as bytes
(scales and codes drawn from the stated distributions), fp32 activation
vectors and expert ids.  It decodes nothing, multiplies nothing and holds no
table of the formats' values, so it carries none of the GEMV's arithmetic.

Every generator is a pure function of its seed (numpy ``Generator(PCG64)``).
Seeds follow ``1000 * cfg + tensor_id`` for the five workloads below.

Block layouts written here (byte order little-endian):
  Q8_0  (34 B): fp16 scale bits, then 32 int8 codes
  Q4_0  (18 B): fp16 scale bits, then 16 bytes of packed 4-bit codes
  MXFP4 (17 B): E8M0 scale byte, then 16 bytes of packed 4-bit codes
"""
from __future__ import annotations

import numpy as np

Q8_0, Q4_0, MXFP4 = 1, 2, 3
FMT_NAMES = {Q8_0: "q8_0", Q4_0: "q4_0", MXFP4: "mxfp4"}
BLOCK_BYTES = {Q8_0: 34, Q4_0: 18, MXFP4: 17}


def rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


CHUNK_ROWS = 256  # rows per independently seeded chunk


def _fp16_scale_bits(g: np.random.Generator, n: int, lo: float, hi: float, random_sign: bool) -> np.ndarray:
    """Scales drawn as doubles in [lo, hi), rounded once to binary16 (round to
    nearest even, numpy's cast), optionally given a uniform random sign.
    Returned as the raw 16-bit patterns."""
    u = g.random(n)
    d = (lo + (hi - lo) * u).astype(np.float16)
    if random_sign:
        neg = g.integers(0, 2, size=n).astype(bool)
        d = np.where(neg, -d, d).astype(np.float16)
    return d.view(np.uint16)


def _chunk(fmt: int, rows: int, k: int, g: np.random.Generator, p: dict) -> np.ndarray:
    """One chunk of rows: all code bytes first (drawn over the whole block so
    that the scale bytes are overwritten afterwards), then the scales."""
    bb = BLOCK_BYTES[fmt]
    nb = rows * (k // 32)
    if fmt == Q8_0:
        out = g.integers(-127, 128, size=nb * bb, dtype=np.int8).view(np.uint8).reshape(nb, bb)
        out[:, 0:2] = _fp16_scale_bits(g, nb, p.get("scale_lo", 1e-3), p.get("scale_hi", 1e-2),
                                       p.get("random_sign", True)).view(np.uint8).reshape(nb, 2)
    elif fmt == Q4_0:
        out = g.integers(0, 256, size=nb * bb, dtype=np.uint8).reshape(nb, bb)
        out[:, 0:2] = _fp16_scale_bits(g, nb, p.get("scale_lo", 1e-3), p.get("scale_hi", 1e-2),
                                       p.get("random_sign", False)).view(np.uint8).reshape(nb, 2)
    elif fmt == MXFP4:
        out = g.integers(0, 256, size=nb * bb, dtype=np.uint8).reshape(nb, bb)
        out[:, 0] = g.integers(p.get("e_lo", 118), p.get("e_hi", 130) + 1, size=nb, dtype=np.uint8)
    else:
        raise ValueError(f"unknown format {fmt}")
    return out.reshape(rows, (k // 32) * bb)


def blocks(fmt: int, n_rows: int, k: int, seed: int, r0: int = 0, r1: int | None = None, **p) -> np.ndarray:
    """Rows [r0, r1) of a seeded (n_rows, k/32 * block_bytes) uint8 matrix.

    Rows come in chunks of CHUNK_ROWS, chunk c drawn from
    PCG64(SeedSequence([seed, c])), so any row range can be regenerated
    without the rest of the matrix.  Distributions:
      Q8_0 : d ~ fp16(U[1e-3, 1e-2)) * (+-1), q ~ U{-127..127}
      Q4_0 : d ~ fp16(U[1e-3, 1e-2)), every code byte ~ U{0..255}
      MXFP4: e ~ U{118..130}, every code byte ~ U{0..255}
    """
    assert k % 32 == 0 and k > 0
    r1 = n_rows if r1 is None else r1
    assert 0 <= r0 <= r1 <= n_rows
    rb = (k // 32) * BLOCK_BYTES[fmt]
    out = np.empty((r1 - r0, rb), dtype=np.uint8)
    c0, c1 = r0 // CHUNK_ROWS, (r1 + CHUNK_ROWS - 1) // CHUNK_ROWS
    for c in range(c0, c1):
        lo, hi = c * CHUNK_ROWS, min((c + 1) * CHUNK_ROWS, n_rows)
        g = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, c])))
        ch = _chunk(fmt, hi - lo, k, g, p)
        a, b = max(lo, r0), min(hi, r1)
        out[a - r0:b - r0] = ch[a - lo:b - lo]
    return out


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
    return g.integers(0, 256, size=(n_rows, (k // 32) * BLOCK_BYTES[fmt]), dtype=np.uint8)


def x_vec(k: int, seed: int) -> np.ndarray:
    """fp32 activations ~ N(0, 1)."""
    return rng(seed).standard_normal(k).astype(np.float32)


def expert_ids(n_expert: int, n_sel: int, n_tokens: int, seed: int) -> np.ndarray:
    """(n_tokens, n_sel) int32: per token, n_sel distinct ids drawn uniformly
    without replacement from [0, n_expert), listed in ascending order."""
    g = rng(seed)
    ids = np.stack([np.sort(g.choice(n_expert, n_sel, replace=False)) for _ in range(n_tokens)])
    return ids.astype(np.int32)


# --- the five workloads --------------------------------------------------------

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
            tokens=32),
}


def dense_layer_shapes(hidden: int = 6144, ffn: int = 24576):
    """(name, rows, k) of the four weight matrices of one dense decoder layer."""
    return [("qkv", 3 * hidden, hidden), ("out", hidden, hidden), ("up", ffn, hidden), ("down", hidden, ffn)]
