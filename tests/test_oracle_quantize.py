"""Pins for the oracle's per-row signed-INT4 quantizer: brute force in exact
rationals on tiny rows, invariants, and the edge rows the pages test (zeros,
tiny and max-finite values, NaN/Inf, rounding boundaries, empty input)."""
from fractions import Fraction

import numpy as np
import pytest

import workloads
from tests.exact import rne

DTS = ["f32", "f16", "bf16"]
FLT_MIN = np.float32(2.0 ** -126)


def st(vals, dt):
    return workloads.f32_to_storage(np.asarray(vals, dtype=np.float32), dt)


def brute(yv):
    """Exact reference for one row of fp32-widened values."""
    yv = np.asarray(yv, dtype=np.float32)
    if np.isnan(yv).any():
        return None, [0] * len(yv)
    a = np.max(np.abs(yv)) if len(yv) else np.float32(0)
    s = np.float32(a) / np.float32(7.0)          # IEEE fp32 division (numpy)
    if s < FLT_MIN:
        s = FLT_MIN
    codes = []
    for v in yv:
        q = np.float32(v) / np.float32(s)
        if np.isnan(q):
            codes.append(0)
            continue
        # numpy's fp32 division is correctly rounded: pin that too
        if np.isfinite(q) and np.isfinite(s) and s != 0:
            exact = Fraction(float(v)) / Fraction(float(s))
            lo = np.nextafter(q, np.float32(-np.inf))
            hi = np.nextafter(q, np.float32(np.inf))
            assert abs(Fraction(float(q)) - exact) <= abs(Fraction(float(lo)) - exact)
            assert abs(Fraction(float(q)) - exact) <= abs(Fraction(float(hi)) - exact)
        c = rne(Fraction(float(q)))
        codes.append(max(-7, min(7, c)))
    return s, codes


@pytest.mark.parametrize("dt", DTS)
def test_brute_force_tiny_rows(orc, dt):
    rng = np.random.default_rng(21)
    for trial in range(40):
        M, K = rng.integers(1, 9), int(rng.integers(1, 17)) * 2
        scale = 10.0 ** rng.uniform(-6, 4)
        y = st(rng.standard_normal((M, K)) * scale, dt)
        codes, scales = orc.quantize(y, dt)
        yv = orc.decode(dt, y)
        for m in range(M):
            s, c = brute(yv[m])
            assert np.float32(scales[m]) == s
            assert list(codes[m]) == c


@pytest.mark.parametrize("dt", DTS)
def test_rounding_boundaries_half_even(orc, dt):
    # row max 7 -> s = 1 exactly; entries at k + 1/2 must round half-to-even
    vals = [7.0, 0.5, 1.5, 2.5, 3.5, -0.5, -1.5, -2.5, 6.5, -6.5, 4.5, 5.5, 0.0, -0.0, 3.0, -7.0]
    codes, scales = orc.quantize(st([vals], dt), dt)
    assert scales[0] == 1.0
    assert list(codes[0]) == [7, 0, 2, 2, 4, 0, -2, -2, 6, -6, 4, 6, 0, 0, 3, -7]


@pytest.mark.parametrize("dt", DTS)
def test_invariants_random(orc, dt):
    rng = np.random.default_rng(22)
    y = st(rng.standard_t(4, size=(64, 256)), dt)
    codes, scales = orc.quantize(y, dt)
    yv = orc.decode(dt, y)
    assert (scales > 0).all()
    assert (np.abs(codes).max(axis=1) == 7).all()        # the absmax maps to +-7
    err = np.abs(scales[:, None].astype(np.float64) * codes - yv)
    assert (err <= scales[:, None] * 0.5 * (1 + 1e-6)).all()
    neg = workloads.f32_to_storage(-orc.decode(dt, y).astype(np.float32), dt)
    c2, s2 = orc.quantize(neg, dt)
    assert np.array_equal(c2, -codes) and np.array_equal(s2, scales)


@pytest.mark.parametrize("dt", DTS)
def test_zero_row_uses_finite_minimum(orc, dt):
    codes, scales = orc.quantize(st(np.zeros((2, 32)), dt), dt)
    assert (codes == 0).all()
    assert (scales == FLT_MIN).all()


@pytest.mark.parametrize("dt", DTS)
def test_tiny_rows(orc, dt):
    # max |y| below 7 * 2^-126: the scale clamps to 2^-126 (codes may be < 7)
    tiny = {"f32": 1e-38, "f16": 6e-8, "bf16": 1e-38}[dt]
    row = np.array([tiny, -tiny / 2, tiny / 4, 0.0], dtype=np.float32)
    y = st([row], dt)
    codes, scales = orc.quantize(y, dt)
    yv = orc.decode(dt, y)[0]
    s, c = brute(yv)
    assert scales[0] == s and list(codes[0]) == c
    if dt == "f16":
        assert scales[0] == FLT_MIN or scales[0] > 0


@pytest.mark.parametrize("dt", DTS)
def test_max_finite_rows(orc, dt):
    big = {"f32": np.finfo(np.float32).max, "f16": 65504.0, "bf16": 3.3895313892515355e+38}[dt]
    y = st([[big, -big, big / 2, 1.0]], dt)
    codes, scales = orc.quantize(y, dt)
    assert np.isfinite(scales[0])
    assert list(codes[0][:3]) == [7, -7, 4]   # 3.5 -> 4 (half-even)
    assert codes[0][3] == 0


@pytest.mark.parametrize("dt", DTS)
def test_nan_and_inf_rows(orc, dt):
    y = st([[1.0, np.nan, 2.0, 3.0], [1.0, np.inf, -2.0, 3.0], [1.0, 2.0, 3.0, 7.0]], dt)
    codes, scales = orc.quantize(y, dt)
    assert np.isnan(scales[0]) and (codes[0] == 0).all()
    assert np.isinf(scales[1]) and (codes[1] == 0).all()  # finite/inf = 0, inf/inf = NaN -> 0
    assert scales[2] == 1.0 and list(codes[2]) == [1, 2, 3, 7]


def test_empty(orc):
    codes, scales = orc.quantize(np.zeros((0, 16), dtype=np.float32), "f32")
    assert codes.shape == (0, 16) and scales.shape == (0,)
