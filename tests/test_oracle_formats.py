"""Pins for the oracle's number formats: its own round-to-nearest-even
conversions are checked against numpy/torch library casts and against an
exact-rational brute force over every finite 16-bit value."""
from fractions import Fraction

import numpy as np
import pytest
import torch

from tests.exact import round_exact


def _probe_values(rng, n):
    # Wide exponent spread incl. subnormal and overflow regions, plus exact ties.
    mags = np.exp2(rng.uniform(-150, 130, size=n))
    v = mags * rng.choice([-1.0, 1.0], size=n)
    specials = [0.0, -0.0, 1.0, 65504.0, 65519.999, 65520.0, 1e-8, 5.9604644775390625e-08,
                2.9802322387695312e-08, 3.0e-8, 3.3895313892515355e+38, 3.3961e38, 3.5e38,
                1.00390625, 1.01171875, 1.0009765625, 1.0029296875, np.inf, -np.inf]
    return np.concatenate([v, np.array(specials)])


def test_f16_matches_numpy_cast(orc):
    rng = np.random.default_rng(1)
    v = _probe_values(rng, 20000)
    vals, bits = orc.round_to("f16", v)
    ref = v.astype(np.float16)
    assert np.array_equal(bits.view(np.uint16), ref.view(np.uint16))
    assert np.array_equal(vals, ref.astype(np.float64))


def test_bf16_matches_torch_cast_on_fp32_values(orc):
    rng = np.random.default_rng(2)
    v = _probe_values(rng, 20000).astype(np.float32).astype(np.float64)
    vals, bits = orc.round_to("bf16", v)
    ref = torch.from_numpy(v.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy()
    assert np.array_equal(bits.view(np.int16), ref)


def test_f32_matches_numpy_cast(orc):
    rng = np.random.default_rng(3)
    v = _probe_values(rng, 20000)
    v = v[np.abs(v) < 1e300]
    vals, bits = orc.round_to("f32", v)
    with np.errstate(over="ignore"):
        ref = v.astype(np.float32)
    assert np.array_equal(bits.view(np.uint32), ref.view(np.uint32))


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
def test_round_matches_exact_rational_brute_force(orc, fmt):
    # Doubles that are not fp32 values (so no library cast is involved) vs the
    # nearest-even search over every finite value of the format.
    rng = np.random.default_rng(4)
    lo, hi = (-26, 17) if fmt == "f16" else (-135, 129)
    v = np.exp2(rng.uniform(lo, hi, size=3000)) * rng.choice([-1.0, 1.0], size=3000)
    # add exact midpoints between neighbours (tie cases)
    keys = np.array([0.0])
    vals, bits = orc.round_to(fmt, v)
    for x, got in zip(v, vals):
        assert got == round_exact(Fraction(float(x)), fmt), (fmt, x, got)


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
def test_ties_go_to_even(orc, fmt):
    from tests.exact import finite_values
    keys, even = finite_values(fmt)
    rng = np.random.default_rng(5)
    idx = rng.integers(0, len(keys) - 1, size=2000)
    for i in idx:
        a, b = keys[i], keys[i + 1]
        mid = (a + b) / 2
        if float(mid) != mid:  # midpoint not a double -> skip
            continue
        got = orc.round_to(fmt, [float(mid)])[0][0]
        want = float(a) if even[i] else float(b)
        assert got == want


def test_decode_exhaustive(orc):
    allb = np.arange(1 << 16, dtype=np.uint16)
    d16 = orc.decode("f16", allb)
    ref16 = allb.view(np.float16).astype(np.float64)
    assert np.array_equal(np.isnan(d16), np.isnan(ref16))
    ok = ~np.isnan(ref16)
    assert np.array_equal(d16[ok], ref16[ok])
    db = orc.decode("bf16", allb)
    refb = (allb.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    assert np.array_equal(np.isnan(db), np.isnan(refb))
    ok = ~np.isnan(refb)
    assert np.array_equal(db[ok], refb[ok])
