"""The seeded input generators (no GPU): published SplitMix64, binary16
rounding, independence of row ranges and thread counts, and the stated
distributions."""
from __future__ import annotations

import numpy as np
import pytest

import synth

M64 = 2 ** 64 - 1


def splitmix64_py(seed, s, i):
    """SplitMix64's output function on the counter (Steele, Lea & Flood 2014)."""
    z = (seed + 0x9E3779B97F4A7C15 * (1 + ((s << 40) + i))) & M64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & M64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & M64
    return z ^ (z >> 31)


def test_counter_words_match_published_splitmix64():
    L = synth._load()
    for seed in (0, 1, 5003, 2 ** 63 + 11):
        for s in (0, 1, 2):
            for i in (0, 1, 77, 2 ** 35 + 3):
                assert L.synth_word(seed, s, i) == splitmix64_py(seed, s, i)
    # the plain SplitMix64 stream from state 0 begins with this published word
    assert splitmix64_py(0, 0, 0) == 0xE220A8397B1DCDAF


def test_half_rounding_matches_numpy():
    L = synth._load()
    v = np.random.default_rng(0).uniform(1e-3, 1e-2, 20000)
    v = np.concatenate([v, np.nextafter(np.float64(np.float16(0.005)), 1.0) + np.zeros(1)])
    for x in v:
        assert L.synth_half_bits(float(x)) == int(np.float16(x).view(np.uint16))


@pytest.mark.parametrize("fmt", [synth.Q8_0, synth.Q4_0, synth.MXFP4])
def test_row_ranges_and_threads_do_not_change_bytes(fmt):
    full = synth.blocks(fmt, 300, 2880, seed=42, threads=1)
    assert np.array_equal(full, synth.blocks(fmt, 300, 2880, seed=42, threads=7))
    for r0, r1 in [(0, 1), (17, 230), (299, 300), (5, 5)]:
        assert np.array_equal(synth.blocks(fmt, 300, 2880, seed=42, r0=r0, r1=r1), full[r0:r1])
    assert not np.array_equal(full, synth.blocks(fmt, 300, 2880, seed=43))


def test_distributions():
    b = synth.blocks(synth.Q8_0, 2000, 1024, seed=1).reshape(-1, 34)
    q = b[:, 2:].view(np.int8).astype(int)
    assert q.min() == -127 and q.max() == 127
    counts = np.bincount(q.ravel() + 127, minlength=255)
    assert counts.min() > 0.9 * counts.mean() and counts.max() < 1.1 * counts.mean()
    d = b[:, :2].copy().view(np.float16).astype(np.float64).ravel()
    assert np.all((np.abs(d) >= np.float16(1e-3)) & (np.abs(d) <= np.float16(1e-2)))
    assert 0.45 < (d < 0).mean() < 0.55
    b = synth.blocks(synth.Q4_0, 2000, 1024, seed=2).reshape(-1, 18)
    d = b[:, :2].copy().view(np.float16).astype(np.float64).ravel()
    assert np.all(d > 0)
    nib = np.concatenate([b[:, 2:] & 15, b[:, 2:] >> 4]).ravel()
    c = np.bincount(nib, minlength=16)
    assert c.min() > 0.95 * c.mean()
    b = synth.blocks(synth.MXFP4, 2000, 1024, seed=3).reshape(-1, 17)
    e = np.bincount(b[:, 0], minlength=256)
    assert set(np.nonzero(e)[0]) == set(range(118, 131))


def test_expert_ids_and_x():
    ids = synth.expert_ids(128, 4, 64, seed=4008)
    assert ids.shape == (64, 4) and ids.dtype == np.int32
    assert all(len(set(r)) == 4 and list(r) == sorted(r) for r in ids)
    assert np.array_equal(ids, synth.expert_ids(128, 4, 64, seed=4008))
    x = synth.x_vec(100000, 9)
    assert x.dtype == np.float32 and abs(x.mean()) < 0.02 and abs(x.std() - 1) < 0.02


def test_bad_arguments_rejected():
    with pytest.raises(ValueError):
        synth.blocks(synth.Q8_0, 4, 64, 1, scale_lo=0.0)
    with pytest.raises(AssertionError):
        synth.blocks(synth.Q8_0, 4, 48, 1)
