"""Parity gates shared by the GPU tests.

Gate 1 (normwise):       max_j |y_j - r_j| / max_j |r_j|        <= tol
Gate 2 (componentwise):  |y_j - r_j| <= tol * a_j,  a_j = sum_i |w_ji x_i|
with r the fp64 oracle result and tol = 1e-4.  Gate 2 bounds every row,
rows whose result cancels to nearly zero included; its scale a_j is what fp32
rounding error is proportional to.
"""
from __future__ import annotations

import numpy as np

TOL = 1e-4


def check(y, ref, a, tol=TOL, what=""):
    y = np.asarray(y, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    a = np.asarray(a, dtype=np.float64)
    assert y.shape == ref.shape, (y.shape, ref.shape)
    assert np.all(np.isfinite(y)), f"{what}: non-finite output"
    err = np.abs(y - ref)
    if ref.size == 0:
        return {}
    scale = np.abs(ref).max()
    g1 = err.max() / scale if scale > 0 else err.max()
    bad = err > tol * a
    assert g1 <= tol, f"{what}: normwise error {g1:.3e} > {tol}"
    assert not bad.any(), (f"{what}: componentwise gate failed in {bad.sum()} rows, worst "
                           f"{np.max(err / np.maximum(a, 1e-300)):.3e}")
    return {"normwise": float(g1), "componentwise": float(np.max(err / np.maximum(a, 1e-300)))}


def bits_equal(a, b) -> bool:
    """Bitwise equality of two float32 arrays (NaNs compared as NaN-ness)."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    b = np.ascontiguousarray(b, dtype=np.float32)
    if a.shape != b.shape:
        return False
    na, nb_ = np.isnan(a), np.isnan(b)
    if not np.array_equal(na, nb_):
        return False
    return np.array_equal(a.view(np.uint32)[~na], b.view(np.uint32)[~nb_])
