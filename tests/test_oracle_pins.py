"""Pins of the CPU oracle to facts outside itself (no GPU).

Each test checks the oracle against something it does not share code with:
the page's printed sizes (tests/golden/page_sizes.txt), published value tables
(tests/golden/ocp_e2m1_e8m0.txt), independent library decoders (struct's and
numpy's binary16, torch's E8M0), exact rational arithmetic, brute force over
tiny inputs, closed forms, and the page's invariant that a block-walked or
windowed result equals the whole-matrix result bit for bit.
"""
from __future__ import annotations

import math
import os
import struct
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
Q8_0, Q4_0, MXFP4, Q4_K, Q6_K = oracle.Q8_0, oracle.Q4_0, oracle.MXFP4, oracle.Q4_K, oracle.Q6_K


def golden_sizes():
    out = {}
    for line in open(os.path.join(GOLDEN, "page_sizes.txt")):
        line = line.split("#")[0].strip()
        if line:
            k, v = [t.strip() for t in line.split("=")]
            out[k] = float(v)
    return out


def golden_ocp():
    e2m1, e8m0 = {}, {}
    for line in open(os.path.join(GOLDEN, "ocp_e2m1_e8m0.txt")):
        line = line.split("#")[0].strip()
        if not line:
            continue
        kind, code, val = line.split()
        if kind == "e2m1":
            e2m1[int(code)] = float(val)
        else:
            if val == "nan":
                e8m0[int(code)] = math.nan
            elif val.startswith("2^"):
                e8m0[int(code)] = math.ldexp(1.0, int(val[2:]))
            else:
                e8m0[int(code)] = float(val)
    return e2m1, e8m0


def f32_bits_equal(a, b):
    a = np.asarray(a, np.float32)
    b = np.asarray(b, np.float32)
    na, nb = np.isnan(a), np.isnan(b)
    return np.array_equal(na, nb) and np.array_equal(a.view(np.uint32)[~na], b.view(np.uint32)[~nb])


# --- sizes the pages print ---------------------------------------------------------------

def test_block_sizes_match_pages():
    g = golden_sizes()
    assert oracle.block_bytes(Q4_0) == g["q4_0_block_bytes"]
    assert oracle.block_bytes(Q8_0) == g["q8_0_block_bytes"]
    # MXFP4: the page gives the size of one expert matrix, not of a block.
    rows, k = int(g["mxfp4_expert_rows"]), int(g["mxfp4_expert_k"])
    expert = rows * oracle.row_bytes(MXFP4, k)
    assert round(expert / 1e6, 2) == g["mxfp4_expert_mb"]
    # two ring slots of 128 rows (lookahead 1 -> lookahead + 1 buffers)
    ring = (int(g["arena_lookahead"]) + 1) * int(g["arena_peak_block_rows"]) * oracle.row_bytes(MXFP4, k)
    assert round(ring / 1e6, 2) == g["arena_peak_mb"]
    assert int(expert / ring) == g["arena_memory_ratio"]
    # the neighbouring block sizes would break these page numbers
    for bb in (16, 18):
        assert round(rows * (k // 32) * bb / 1e6, 2) != g["mxfp4_expert_mb"]
    # Q4_K: 144 bytes per 256 weights = 4.5 bits per weight, 7.1x below F32
    assert oracle.block_bytes(Q4_K) == g["q4_k_block_bytes"]
    assert oracle.block_weights(Q4_K) == g["q4_k_block_weights"]
    assert oracle.row_bytes(Q4_K, 512) == 2 * g["q4_k_block_bytes"]
    assert 8 * oracle.block_bytes(Q4_K) / oracle.block_weights(Q4_K) == g["q4_bits_per_weight"]
    assert round(4 * oracle.block_weights(Q4_K) / oracle.block_bytes(Q4_K), 1) == g["q4_k_f32_ratio"]
    assert 2 + 2 + g["q4_k_scale_bytes"] + oracle.block_weights(Q4_K) // 2 == g["q4_k_block_bytes"]
    assert 16 * 6 == 8 * g["q4_k_scale_bytes"]  # 8 scales + 8 mins of 6 bits fill the 12 bytes
    assert oracle.block_weights(Q8_0) == g["block_weights"] == oracle.block_weights(MXFP4)


def test_row_bytes_rejects_bad_k():
    for k in (0, -32, 16, 33, 100):
        assert oracle.row_bytes(Q8_0, k) < 0
    for k in (32, 288, 100):
        assert oracle.row_bytes(Q4_K, k) < 0 and oracle.row_bytes(Q6_K, k) < 0
    assert oracle.block_bytes(7) < 0 and oracle.block_weights(7) < 0


# --- fp16 scale decode ----------------------------------------------------------------

def test_fp16_all_65536_patterns_match_struct():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = oracle.half_to_double(bits)
    for b in range(65536):
        ref = struct.unpack("<e", struct.pack("<H", b))[0]
        g = got[b]
        if math.isnan(ref):
            assert math.isnan(g), b
        else:
            assert g == ref and math.copysign(1.0, g) == math.copysign(1.0, ref), b


# --- Q8_0 -----------------------------------------------------------------------------

def _q8_blocks(d_bits: np.ndarray, q: np.ndarray) -> np.ndarray:
    """Blocks with the given scale patterns and int8 codes (rows of 32)."""
    n = d_bits.size
    b = np.empty((n, 34), np.uint8)
    b[:, 0:2] = d_bits.astype("<u2").view(np.uint8).reshape(n, 2)
    b[:, 2:] = q.astype(np.int8).view(np.uint8).reshape(n, 32)
    return b


def test_q8_0_bruteforce_every_scale_and_code():
    """Every binary16 scale pattern x every int8 code, against numpy's own
    binary16 decode and an fp64 product rounded once to fp32."""
    d = np.repeat(np.arange(65536, dtype=np.uint32).astype(np.uint16), 8)
    q = np.tile(np.arange(-128, 128, dtype=np.int16).reshape(8, 32), (65536, 1))
    blocks = _q8_blocks(d, q)
    n = blocks.shape[0]
    got = oracle.dequant_rows(Q8_0, blocks, n, 32)
    dv = d.view(np.float16).astype(np.float64)
    with np.errstate(invalid="ignore", over="ignore"):
        ref = (dv[:, None] * q.astype(np.float64)).astype(np.float32)
    assert f32_bits_equal(got, ref)


def test_q8_0_hand_built_blocks():
    q = np.arange(32) - 16
    got = oracle.dequant_rows(Q8_0, _q8_blocks(np.array([0x3C00], np.uint16), q[None]), 1, 32)
    assert np.array_equal(got[0], q.astype(np.float32))  # d = 1.0
    got = oracle.dequant_rows(Q8_0, _q8_blocks(np.array([0x0001], np.uint16), q[None]), 1, 32)
    assert np.array_equal(got[0], (q * 2.0 ** -24).astype(np.float32))  # smallest subnormal d
    got = oracle.dequant_rows(Q8_0, _q8_blocks(np.array([0xC000], np.uint16), q[None]), 1, 32)
    assert np.array_equal(got[0], (-2.0 * q).astype(np.float32))  # d = -2


# --- Q4_0 -----------------------------------------------------------------------------

def _q4_block(d_bits: int, nibbles) -> np.ndarray:
    """One Q4_0 block from 32 element codes (element j<16 -> low nibble of
    byte j, element j+16 -> high nibble)."""
    nb = np.asarray(nibbles, np.uint8)
    b = np.empty(18, np.uint8)
    b[0:2] = np.array([d_bits], "<u2").view(np.uint8)
    b[2:] = nb[:16] | (nb[16:] << 4)
    return b


def test_q4_0_hand_built_block():
    b = np.empty(18, np.uint8)
    b[0:2] = np.array([0x3C00], "<u2").view(np.uint8)  # d = 1
    j = np.arange(16)
    b[2:] = ((15 - j) << 4) | j
    got = oracle.dequant_rows(Q4_0, b, 1, 32)[0]
    assert np.array_equal(got[:16], (j - 8).astype(np.float32))
    assert np.array_equal(got[16:], (7 - j).astype(np.float32))


def test_q4_0_every_code_at_every_position():
    """Code c at position p, all other codes 8 (weight 0): locates every nibble."""
    blocks, expect = [], []
    for p in range(32):
        for c in range(16):
            codes = [8] * 32
            codes[p] = c
            blocks.append(_q4_block(0x4000, codes))  # d = 2
            e = np.zeros(32, np.float32)
            e[p] = 2.0 * (c - 8)
            expect.append(e)
    got = oracle.dequant_rows(Q4_0, np.stack(blocks), len(blocks), 32)
    assert np.array_equal(got, np.stack(expect))


def test_q4_0_every_scale_pattern():
    d = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    codes = np.arange(32) % 16
    blocks = np.stack([_q4_block(int(x), codes) for x in d])
    got = oracle.dequant_rows(Q4_0, blocks, 65536, 32)
    dv = d.view(np.float16).astype(np.float64)
    with np.errstate(invalid="ignore", over="ignore"):
        ref = (dv[:, None] * (codes - 8).astype(np.float64)).astype(np.float32)
    assert f32_bits_equal(got, ref)


# --- MXFP4 ----------------------------------------------------------------------------

def test_mxfp4_every_scale_and_code_against_published_tables():
    e2m1, _ = golden_ocp()
    import torch
    e = np.repeat(np.arange(256, dtype=np.uint8), 1)
    # per block: codes 0..15 in the low nibbles, 15..0 in the high nibbles
    j = np.arange(16, dtype=np.uint8)
    blocks = np.empty((256, 17), np.uint8)
    blocks[:, 0] = e
    blocks[:, 1:] = (j | ((15 - j) << 4))[None, :]
    got = oracle.dequant_rows(MXFP4, blocks, 256, 32)
    # independent scale decode: torch's E8M0 dtype
    scale = torch.from_numpy(e.copy()).view(torch.float8_e8m0fnu).double().numpy()
    codes = np.concatenate([j, 15 - j])
    vals = np.array([e2m1[int(c)] for c in codes])
    with np.errstate(invalid="ignore", over="ignore"):
        ref = (scale[:, None] * vals[None, :]).astype(np.float32)
    assert f32_bits_equal(got, ref)
    # e = 127: the table itself, in order then reversed; code 8 is -0
    row = got[127]
    assert np.array_equal(row[:16], np.array([e2m1[c] for c in range(16)], np.float32))
    assert math.copysign(1.0, row[8]) == -1.0 and row[8] == 0.0
    assert np.isnan(got[255]).all()
    assert got[0][1] == np.float32(2.0 ** -128)  # an fp32 subnormal, kept exactly


def test_e8m0_golden_points():
    _, e8m0 = golden_ocp()
    for code, val in e8m0.items():
        b = np.zeros((1, 17), np.uint8)
        b[0, 0] = code
        b[0, 1] = 2  # element 0 -> code 2 = 1.0
        got = oracle.dequant_rows(MXFP4, b, 1, 32)[0, 0]
        if math.isnan(val):
            assert np.isnan(got)
        else:
            assert got == np.float32(val)


# --- the dot product ---------------------------------------------------------------------

@pytest.mark.parametrize("fmt", [Q8_0, Q4_0, MXFP4])
@pytest.mark.parametrize("k", [32, 64, 96, 160])
def test_gemv_against_exact_rationals(fmt, k):
    rows = 5
    w = synth.blocks(fmt, rows, k, seed=50 + k + fmt)
    x = synth.x_vec(k, seed=60 + k)
    dec = oracle.dequant_rows(fmt, w, rows, k)  # pinned above
    y, a = oracle.gemv_rows(fmt, w, rows, k, x)
    for r in range(rows):
        exact = sum(Fraction(float(dec[r, i])) * Fraction(float(x[i])) for i in range(k))
        absum = sum(abs(Fraction(float(dec[r, i])) * Fraction(float(x[i]))) for i in range(k))
        assert abs(Fraction(y[r]) - exact) <= Fraction(k) * Fraction(2) ** -53 * absum
        assert abs(Fraction(a[r]) - absum) <= Fraction(k) * Fraction(2) ** -53 * absum


def test_layout_is_row_major_out_by_in():
    """x = e_i returns column i of the decoded matrix (y[o] = sum_i W[o,i] x[i]);
    a transposed reading fails on this non-square matrix."""
    rows, k = 3, 64
    w = synth.blocks(Q8_0, rows, k, seed=5)
    dec = oracle.dequant_rows(Q8_0, w, rows, k)
    for i in range(k):
        x = np.zeros(k, np.float32)
        x[i] = 1.0
        y, _ = oracle.gemv_rows(Q8_0, w, rows, k, x)
        assert np.array_equal(y, dec[:, i].astype(np.float64))


def test_closed_forms():
    k = 128
    x = synth.x_vec(k, 3)
    # every block d = 0.5, every q = 3: y = 1.5 * sum(x)
    b = _q8_blocks(np.full(k // 32, 0x3800, np.uint16), np.full((k // 32, 32), 3))
    y, _ = oracle.gemv_rows(Q8_0, b.reshape(1, -1), 1, k, x)
    assert y[0] == pytest.approx(1.5 * float(np.sum(x.astype(np.float64))), rel=1e-15)
    # one-hot code: q = 0 except q[7] = 1 in block 2 -> d * x[2*32+7]
    q = np.zeros((k // 32, 32))
    q[2, 7] = 1
    b = _q8_blocks(np.full(k // 32, 0x3C00, np.uint16), q)
    y, _ = oracle.gemv_rows(Q8_0, b.reshape(1, -1), 1, k, x)
    assert y[0] == float(x[71])
    # zero scale -> zero
    b = _q8_blocks(np.zeros(k // 32, np.uint16), np.full((k // 32, 32), 100))
    y, a = oracle.gemv_rows(Q8_0, b.reshape(1, -1), 1, k, x)
    assert y[0] == 0.0 and a[0] == 0.0
    # Q4_0 with every code 8 is the zero matrix
    blk = _q4_block(0x3C00, [8] * 32)
    y, _ = oracle.gemv_rows(Q4_0, np.tile(blk, k // 32).reshape(1, -1), 1, k, x)
    assert y[0] == 0.0


@pytest.mark.parametrize("fmt", [Q8_0, Q4_0, MXFP4])
def test_windows_equal_slices_of_the_whole(fmt):
    """Every window of a tiny matrix, walked whole or in row blocks of any size,
    equals the slice of the whole-matrix result bit for bit (neurostream README,
    "The idea": the same output, bit for bit)."""
    rows, k = 9, 64
    w = synth.blocks(fmt, rows, k, seed=9)
    x = synth.x_vec(k, 10)
    full, _ = oracle.gemv_rows(fmt, w, rows, k, x)
    for r0 in range(rows + 1):
        for r1 in range(r0, rows + 1):
            y, _ = oracle.gemv_rows(fmt, w, rows, k, x, r0, r1)
            assert np.array_equal(y, full[r0:r1])
            for B in (1, 2, 3, rows):
                parts = [oracle.gemv_rows(fmt, w, rows, k, x, s, min(s + B, r1))[0] for s in range(r0, r1, B)]
                got = np.concatenate(parts) if parts else np.empty(0)
                assert np.array_equal(got, full[r0:r1])


def test_thread_count_does_not_change_bits():
    rows, k = 77, 256
    w = synth.blocks(Q4_0, rows, k, seed=12)
    x = synth.x_vec(k, 13)
    ref = oracle.gemv_rows(Q4_0, w, rows, k, x, threads=1)
    for t in (2, 3, 8, 100):
        got = oracle.gemv_rows(Q4_0, w, rows, k, x, threads=t)
        assert np.array_equal(got[0], ref[0]) and np.array_equal(got[1], ref[1])


def test_argument_rejection():
    w = synth.blocks(Q8_0, 4, 64, seed=1)
    x = synth.x_vec(64, 1)
    for r0, r1 in [(-1, 2), (3, 2), (0, 5)]:
        with pytest.raises(ValueError):
            oracle.gemv_rows(Q8_0, w, 4, 64, x, r0, r1)
    with pytest.raises(ValueError):
        oracle.gemv_rows(Q8_0, w, 4, 64, x[:32])


# --- elementwise steps -----------------------------------------------------------------

def test_silu_mul_against_scipy_expit():
    from scipy.special import expit
    g = np.linspace(-30, 30, 2001)
    u = np.cos(g)
    h = oracle.silu_mul(g, u)
    assert np.allclose(h, g * expit(g) * u, rtol=1e-14, atol=1e-300)
    # silu(v) - silu(-v) = v
    assert np.allclose(oracle.silu_mul(g, np.ones_like(g)) - oracle.silu_mul(-g, np.ones_like(g)), g,
                       rtol=1e-13, atol=1e-13)
    assert oracle.silu_mul(np.zeros(1), np.ones(1))[0] == 0.0


def test_rms_carry_closed_forms():
    from scipy.stats import norm
    v = np.random.default_rng(4).standard_normal(1000) * 3
    out = oracle.rms_carry(v, eps=0.0)
    assert np.mean(out ** 2) == pytest.approx(1.0, rel=1e-12)
    assert np.allclose(out / v, out[0] / v[0])
    eps = 0.25
    out = oracle.rms_carry(v, eps=eps)
    ms = np.mean(v ** 2)
    assert np.mean(out ** 2) == pytest.approx(ms / (ms + eps), rel=1e-12)
    # exact GELU = v * Phi(v)
    g = oracle.rms_carry(v, eps=0.0, gelu=True)
    t = v * norm.cdf(v)
    assert np.allclose(g, t / np.sqrt(np.mean(t ** 2)), rtol=1e-12, atol=1e-14)
    # ... to full relative accuracy far below 0, where every GELU value is tiny
    # and the normalisation scales them back up to O(1)
    v = -np.linspace(5.0, 30.0, 51)
    g = oracle.rms_carry(v, eps=0.0, gelu=True)
    t = v * norm.cdf(v)
    assert np.allclose(g, t / np.sqrt(np.mean(t ** 2)), rtol=1e-10, atol=0)


# --- K-quants -------------------------------------------------------------------------
#
# The pages fix Q4_K's size, field order and formula (RAMforge README,
# "Milestone 5", Q4_K line) but not how the twelve scale bytes pack the eight
# 6-bit scales and mins, nor the nibble order; for Q6_K they give the name
# only.  The pins below check what the pages fix directly, check the structure
# any packing of those fields must have (every stored bit reaches exactly one
# field bit), and check the GGUF reading through encoders written here in the
# encode direction.

HALF_ONE, HALF_TWO, HALF_MINUS_ONE = 0x3C00, 0x4000, 0xBC00


def _le16(v):
    return np.array([v], "<u2").view(np.uint8)


def _q4k_pack(sc, m):
    """The 12 scale bytes holding eight 6-bit scales and mins (GGUF reading):
    fields 0..3 whole in the low six bits of bytes 0..3 (scales) and 4..7
    (mins); fields 4..7 as low nibbles in bytes 8..11 (scale low, min high)
    with their top two bits in the top bits of bytes 0..3 (scales), 4..7 (mins)."""
    sc = np.asarray(sc, np.int64)
    m = np.asarray(m, np.int64)
    out = np.zeros(12, np.int64)
    out[0:4] = (sc[0:4] & 63) | ((sc[4:8] >> 4) << 6)
    out[4:8] = (m[0:4] & 63) | ((m[4:8] >> 4) << 6)
    out[8:12] = (sc[4:8] & 15) | ((m[4:8] & 15) << 4)
    return out.astype(np.uint8)


def _q4k_block(d_bits, dmin_bits, sc, m, codes):
    """One Q4_K super-block: codes[32 s + l] is element l of sub-block s, stored
    in byte 32 (s // 2) + l of the code area, low nibble for even s."""
    c = np.asarray(codes, np.uint8).reshape(4, 2, 32)
    return np.concatenate([_le16(d_bits), _le16(dmin_bits), _q4k_pack(sc, m),
                           (c[:, 0, :] | (c[:, 1, :] << 4)).reshape(128)])


def _q6k_block(d_bits, scales, codes):
    """One Q6_K super-block from 256 six-bit codes and 16 int8 scales (GGUF
    reading): the low nibbles of the codes 128 h + 32 i + l go to low-nibble
    bytes 64 h + 32 (i % 2) + l (high half of the byte for i >= 2), their top
    bits to bit pair i of byte 32 h + l."""
    c = np.asarray(codes, np.int64).reshape(2, 4, 32)  # [h, i, l]
    ql = np.zeros((2, 2, 32), np.int64)
    qh = np.zeros((2, 32), np.int64)
    for i in range(4):
        ql[:, i % 2, :] |= (c[:, i, :] & 15) << (4 * (i // 2))
        qh |= (c[:, i, :] >> 4) << (2 * i)
    return np.concatenate([ql.reshape(128).astype(np.uint8), qh.reshape(64).astype(np.uint8),
                           np.asarray(scales, np.int8).view(np.uint8), _le16(d_bits)])


def _dq(fmt, blocks):
    b = np.ascontiguousarray(np.atleast_2d(blocks))
    return oracle.dequant_rows(fmt, b, b.shape[0], 256)


def test_q4_k_field_order_and_formula():
    """d first, dmin second, w = d sc q - dmin m: with dmin = 0 every weight
    is d times an integer in [0, 63 * 15]; with d = 0 and dmin = 1 each
    32-weight sub-block is one constant -m, m in [0, 63]; and both together
    are the difference of the two (all exact)."""
    g = np.random.default_rng(0)
    for _ in range(20):
        scales = g.integers(0, 256, 12, dtype=np.uint8)
        codes = g.integers(0, 256, 128, dtype=np.uint8)
        mk = lambda d, dm: np.concatenate([_le16(d), _le16(dm), scales, codes])  # noqa: E731
        a = _dq(Q4_K, mk(HALF_TWO, 0))[0].astype(np.float64) / 2.0
        assert np.array_equal(a, np.round(a)) and a.min() >= 0 and a.max() <= 63 * 15
        b = _dq(Q4_K, mk(0, HALF_ONE))[0].astype(np.float64)
        runs = b.reshape(8, 32)
        assert (runs == runs[:, :1]).all() and (b <= 0).all() and (b >= -63).all()
        both = _dq(Q4_K, mk(HALF_TWO, HALF_ONE))[0].astype(np.float64)
        assert np.array_equal(both, 2.0 * a + b)
        assert np.array_equal(_dq(Q4_K, mk(0, 0))[0], np.zeros(256, np.float32))


def test_q4_k_scale_field_is_a_bijection():
    """Each of the 96 bits of the scale bytes is exactly one bit of exactly one
    of the 16 six-bit fields (8 scales read with d = 1, q = 1; 8 mins read with
    d = 0, dmin = -1)."""
    seen = set()
    ones = np.full(128, 0x11, np.uint8)  # every code 1
    for t in range(96):
        f = np.zeros(12, np.uint8)
        f[t // 8] = 1 << (t % 8)
        sc = _dq(Q4_K, np.concatenate([_le16(HALF_ONE), _le16(0), f, ones]))[0].reshape(8, 32)
        mn = _dq(Q4_K, np.concatenate([_le16(0), _le16(HALF_MINUS_ONE), f, ones]))[0].reshape(8, 32)
        assert (sc == sc[:, :1]).all() and (mn == mn[:, :1]).all()
        vals = np.concatenate([sc[:, 0], mn[:, 0]])
        nz = np.flatnonzero(vals)
        assert nz.size == 1, (t, vals)
        v = int(vals[nz[0]])
        assert v > 0 and v & (v - 1) == 0 and v < 64
        seen.add((int(nz[0]), v.bit_length() - 1))
    assert len(seen) == 96


def test_q4_k_codes_are_a_bijection():
    """Each of the 1024 code bits is exactly one bit of exactly one element's
    4-bit code (d = 1, every scale 1, every min 0)."""
    sc, m = np.ones(8, int), np.zeros(8, int)
    head = np.concatenate([_le16(HALF_ONE), _le16(0), _q4k_pack(sc, m)])
    blocks = np.zeros((1024, 144), np.uint8)
    blocks[:, :16] = head
    for t in range(1024):
        blocks[t, 16 + t // 8] = 1 << (t % 8)
    w = oracle.dequant_rows(Q4_K, blocks, 1024, 256)
    seen = set()
    for t in range(1024):
        nz = np.flatnonzero(w[t])
        assert nz.size == 1
        v = int(w[t, nz[0]])
        assert v in (1, 2, 4, 8)
        seen.add((int(nz[0]), v))
    assert len(seen) == 1024


def test_q4_k_hand_built_blocks():
    """Blocks built by the encode-direction packing above decode to
    d sc q - dmin m exactly (rounded once to fp32), for every 6-bit scale and
    min value at every sub-block and every code at every position."""
    g = np.random.default_rng(1)
    for trial in range(64):
        sc = np.roll(np.arange(64), trial)[:8] if trial < 8 else g.integers(0, 64, 8)
        m = np.roll(np.arange(64), 3 * trial)[:8] if trial < 8 else g.integers(0, 64, 8)
        codes = g.integers(0, 16, 256)
        d_bits, dmin_bits = int(g.integers(0x0400, 0x7800)), int(g.integers(0x0400, 0x7800))
        got = _dq(Q4_K, _q4k_block(d_bits, dmin_bits, sc, m, codes))[0]
        d = Fraction(float(np.array([d_bits], np.uint16).view(np.float16)[0]))
        dmin = Fraction(float(np.array([dmin_bits], np.uint16).view(np.float16)[0]))
        for e in range(0, 256, 7):
            s = e // 32
            exact = d * int(sc[s]) * int(codes[e]) - dmin * int(m[s])
            assert got[e] == np.float32(float(exact)), (trial, e)
    # every 6-bit value in every scale and min position
    for v in range(64):
        for s in range(8):
            sc = np.zeros(8, int)
            m = np.zeros(8, int)
            sc[s] = v
            w = _dq(Q4_K, _q4k_block(HALF_ONE, 0, sc, m, np.ones(256, int)))[0].reshape(8, 32)
            expect = np.zeros((8, 32), np.float32)
            expect[s] = v
            assert np.array_equal(w, expect)
            m[s], sc[s] = v, 0
            w = _dq(Q4_K, _q4k_block(0, HALF_MINUS_ONE, sc, m, np.ones(256, int)))[0].reshape(8, 32)
            assert np.array_equal(w, expect)
    # every code at every position
    codes = np.arange(256) % 16
    for shift in range(16):
        c = np.roll(codes, shift)
        w = _dq(Q4_K, _q4k_block(HALF_ONE, 0, np.ones(8, int), np.zeros(8, int), c))[0]
        assert np.array_equal(w, c.astype(np.float32))


def test_q6_k_codes_are_a_bijection_and_centered():
    """Each of the 1536 code bits is one bit of exactly one element's 6-bit
    code, and the codes read as q - 32: with d = 1 and every scale 1 the all-zero
    code bytes give -32 everywhere, and every integer in [-32, 31] is reached."""
    base = _q6k_block(HALF_ONE, np.ones(16, np.int8), np.zeros(256, int))
    assert np.array_equal(base[:192], np.zeros(192, np.uint8))
    assert np.array_equal(_dq(Q6_K, base)[0], np.full(256, -32.0, np.float32))
    blocks = np.tile(base, (1536, 1))
    for t in range(1536):
        blocks[t, t // 8] = 1 << (t % 8)
    w = oracle.dequant_rows(Q6_K, blocks, 1536, 256).astype(np.float64) + 32.0
    seen = set()
    for t in range(1536):
        nz = np.flatnonzero(w[t])
        assert nz.size == 1
        v = int(w[t, nz[0]])
        assert v in (1, 2, 4, 8, 16, 32)
        seen.add((int(nz[0]), v))
    assert len(seen) == 1536
    g = np.random.default_rng(2)
    rnd = np.tile(base, (64, 1))
    rnd[:, :192] = g.integers(0, 256, (64, 192), dtype=np.uint8)
    vals = oracle.dequant_rows(Q6_K, rnd, 64, 256)
    assert set(np.unique(vals).astype(int)) == set(range(-32, 32))


def test_q6_k_scales_cover_runs_of_16():
    """Scale byte t multiplies exactly the 16 consecutive weights 16 t .. 16 t + 15."""
    for t in range(16):
        s = np.zeros(16, np.int8)
        s[t] = -3
        w = _dq(Q6_K, _q6k_block(HALF_ONE, s, np.zeros(256, int)))[0]
        expect = np.zeros(256, np.float32)
        expect[16 * t:16 * t + 16] = 96.0  # -3 * (0 - 32)
        assert np.array_equal(w, expect)


def test_q6_k_hand_built_blocks():
    """d scale (q - 32) exactly (rounded once), d the fp16 in the last two
    bytes: every code at every position, and random scales and d."""
    g = np.random.default_rng(3)
    for trial in range(32):
        codes = g.integers(0, 64, 256)
        scales = g.integers(-128, 128, 16).astype(np.int8)
        d_bits = int(g.integers(0x0400, 0x7800)) | (0x8000 if trial % 2 else 0)
        got = _dq(Q6_K, _q6k_block(d_bits, scales, codes))[0]
        d = Fraction(float(np.array([d_bits], np.uint16).view(np.float16)[0]))
        for e in range(256):
            exact = d * int(scales[e // 16]) * (int(codes[e]) - 32)
            assert got[e] == np.float32(float(exact)), (trial, e)
    codes = np.arange(256) % 64
    for shift in range(64):
        c = np.roll(codes, shift)
        w = _dq(Q6_K, _q6k_block(HALF_ONE, np.ones(16, np.int8), c))[0]
        assert np.array_equal(w, (c - 32).astype(np.float32))


@pytest.mark.parametrize("fmt", [Q4_K, Q6_K])
@pytest.mark.parametrize("k", [256, 512])
def test_kquant_gemv_against_exact_rationals(fmt, k):
    test_gemv_against_exact_rationals(fmt, k)


@pytest.mark.parametrize("fmt", [Q4_K, Q6_K])
def test_kquant_windows_equal_slices_of_the_whole(fmt):
    rows, k = 7, 256
    w = synth.blocks(fmt, rows, k, seed=9)
    x = synth.x_vec(k, 10)
    full, _ = oracle.gemv_rows(fmt, w, rows, k, x)
    for r0 in range(rows + 1):
        for r1 in range(r0, rows + 1):
            y, _ = oracle.gemv_rows(fmt, w, rows, k, x, r0, r1)
            assert np.array_equal(y, full[r0:r1])


def test_kquant_layout_is_row_major_out_by_in():
    """x = e_i returns column i of the decoded matrix, across super-block edges."""
    for fmt in (Q4_K, Q6_K):
        rows, k = 3, 512
        w = synth.blocks(fmt, rows, k, seed=5)
        dec = oracle.dequant_rows(fmt, w, rows, k)
        for i in (0, 31, 32, 255, 256, 300, 511):
            x = np.zeros(k, np.float32)
            x[i] = 1.0
            y, _ = oracle.gemv_rows(fmt, w, rows, k, x)
            assert np.array_equal(y, dec[:, i].astype(np.float64))


# --- router-weighted combine -------------------------------------------------------------

def test_combine_against_exact_rationals_and_special_cases():
    g = np.random.default_rng(8)
    y = g.standard_normal((4, 33))
    w = g.uniform(0.05, 1.0, 4)
    got = oracle.combine(y, w)
    for i in range(33):
        exact = sum(Fraction(float(w[s])) * Fraction(float(y[s, i])) for s in range(4))
        absum = sum(abs(Fraction(float(w[s])) * Fraction(float(y[s, i]))) for s in range(4))
        assert abs(Fraction(got[i]) - exact) <= 4 * Fraction(2) ** -53 * absum
    # one-hot weights select one expert's vector exactly; zero weights give zeros
    for s in range(4):
        e = np.zeros(4)
        e[s] = 1.0
        assert np.array_equal(oracle.combine(y, e), y[s])
    assert np.array_equal(oracle.combine(y, np.zeros(4)), np.zeros(33))
    assert np.array_equal(oracle.combine(np.zeros((0, 5)), np.zeros(0)), np.zeros(5))
    # the product w^T Y, as numpy's matrix product computes it
    assert np.allclose(got, w @ y, rtol=1e-14, atol=1e-14)
