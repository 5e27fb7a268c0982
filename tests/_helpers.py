"""Comparison helpers shared by the tests (no collective arithmetic here)."""

from __future__ import annotations

import numpy as np


def bits_of(a: np.ndarray) -> np.ndarray:
    """Raw bit patterns: uint16 stays, float32 is viewed as uint32."""
    a = np.ascontiguousarray(a).reshape(-1)
    if a.dtype == np.uint16:
        return a
    if a.dtype == np.float32:
        return a.view(np.uint32)
    raise TypeError(a.dtype)


def is_nan_bits(b: np.ndarray) -> np.ndarray:
    if b.dtype == np.uint16:
        return ((b & 0x7F80) == 0x7F80) & ((b & 0x007F) != 0)
    return ((b & 0x7F800000) == 0x7F800000) & ((b & 0x007FFFFF) != 0)


def assert_bits_equal(got: np.ndarray, want: np.ndarray, what: str = "",
                      nan_by_class: bool = True):
    """Bitwise equality; NaNs match any NaN when ``nan_by_class``."""
    g, w = bits_of(got), bits_of(want)
    assert g.shape == w.shape, f"{what}: shape {g.shape} != {w.shape}"
    diff = g != w
    if nan_by_class:
        diff &= ~(is_nan_bits(g) & is_nan_bits(w))
    if diff.any():
        idx = np.flatnonzero(diff)
        raise AssertionError(
            f"{what}: {idx.size} of {g.size} differ; first at {idx[:8].tolist()}: "
            f"got {[hex(int(x)) for x in g[idx[:8]]]} want "
            f"{[hex(int(x)) for x in w[idx[:8]]]}")


def bf16_ulp_distance(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """|key(a) - key(b)| on the monotone integer line of bf16 patterns,
    where key maps -x below +x and both zeros to the same point."""
    def key(x):
        x = x.astype(np.int64)
        return np.where(x & 0x8000, 0x8000 - (x & 0x7FFF), 0x8000 + x)
    return np.abs(key(a) - key(b))


def assert_bf16_close(got: np.ndarray, want: np.ndarray, ulps: int = 1,
                      what: str = ""):
    g, w = bits_of(got), bits_of(want)
    assert g.dtype == np.uint16 and w.dtype == np.uint16
    both_nan = is_nan_bits(g) & is_nan_bits(w)
    d = np.where(both_nan, 0, bf16_ulp_distance(g, w))
    one_nan = is_nan_bits(g) ^ is_nan_bits(w)
    bad = (d > ulps) | one_nan
    if bad.any():
        idx = np.flatnonzero(bad)
        raise AssertionError(
            f"{what}: {idx.size} of {g.size} beyond {ulps} ulp; first at "
            f"{idx[:8].tolist()}: got {[hex(int(x)) for x in g[idx[:8]]]} want "
            f"{[hex(int(x)) for x in w[idx[:8]]]}")


def assert_f32_close(got: np.ndarray, want: np.ndarray, rel: float = 1e-6,
                     what: str = ""):
    g = np.ascontiguousarray(got).reshape(-1).astype(np.float64)
    w = np.ascontiguousarray(want).reshape(-1).astype(np.float64)
    both_nan = np.isnan(g) & np.isnan(w)
    same_inf = np.isinf(g) & np.isinf(w) & (g == w)
    with np.errstate(invalid="ignore"):
        ok = (np.abs(g - w) <= rel * np.abs(w)) | both_nan | same_inf
    if not ok.all():
        idx = np.flatnonzero(~ok)
        raise AssertionError(
            f"{what}: {idx.size} of {g.size} beyond rel {rel}; first at "
            f"{idx[:8].tolist()}: got {g[idx[:8]].tolist()} want {w[idx[:8]].tolist()}")
