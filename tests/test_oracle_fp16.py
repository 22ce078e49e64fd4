"""Pins of the oracle's own fp16 codec against NumPy's IEEE binary16 (library routine)."""
import numpy as np
import pytest

import oracle


def test_half_to_double_exhaustive():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    got = oracle.half_to_double(bits)
    ref = bits.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # signed zeros keep their sign
    assert np.signbit(got[0x8000]) and not np.signbit(got[0])


def _check_encode(f32: np.ndarray):
    got = oracle.float_to_half(f32)
    with np.errstate(over="ignore", invalid="ignore"):
        ref = f32.astype(np.float16).view(np.uint16)
    nan = np.isnan(f32)
    assert np.array_equal(np.isnan(got.view(np.float16)), nan)
    bad = np.nonzero((got != ref) & ~nan)[0]
    assert bad.size == 0, f"mismatch at {f32[bad[:5]]}: {got[bad[:5]]} vs {ref[bad[:5]]}"


def test_float_to_half_halfway_points():
    """Every point exactly halfway between two adjacent finite halves, and one
    float32 ulp either side: this is where round-to-nearest-even decides."""
    h = np.arange(0, 0x7C00, dtype=np.uint32).astype(np.uint16).view(np.float16).astype(np.float64)
    h = np.concatenate([h, [65536.0]])               # the would-be next step above 65504
    mid = ((h[:-1] + h[1:]) / 2).astype(np.float32)
    up = np.nextafter(mid, np.float32(np.inf))
    dn = np.nextafter(mid, np.float32(0))
    vals = np.concatenate([mid, up, dn, h[:-1].astype(np.float32)])
    _check_encode(np.concatenate([vals, -vals]))


def test_float_to_half_random_and_special():
    rng = np.random.default_rng(7)
    bits = rng.integers(0, 1 << 32, size=1 << 20, dtype=np.uint64).astype(np.uint32)
    f = bits.view(np.float32)
    spec = np.array([0.0, -0.0, np.inf, -np.inf, np.nan, 65504.0, 65519.996, 65520.0, 65536.0,
                     6.1035156e-05, 6.0975552e-05, 5.9604645e-08, 2.9802322e-08, 2.98023259e-08,
                     1e-10, 1e10, 1.0, -1.0, 0.1, 3.14159265], np.float32)
    _check_encode(np.concatenate([f, spec]))
    # values in the range the method actually produces
    g = (rng.standard_normal(1 << 20) * rng.choice([1e-4, 1e-2, 1.0, 30.0], 1 << 20)).astype(np.float32)
    _check_encode(g)
