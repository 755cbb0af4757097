"""Pins for the oracle's INT8 mode (qmax = 127) of the per-row quantizer and
for the dynamic INT8 linear built on it ("[Feat][Ascend] Add fused RotateQuant
backend", "What this PR does / why we need it": the fused rotate + per-token
INT8 quantization feeding the ConvRot INT8 linear).  Brute force in exact
rationals on tiny rows, half-even boundaries at an exact unit scale,
invariants, the special rows, and an independent integer GEMM with the full
INT8 weight range."""
from fractions import Fraction

import numpy as np
import pytest

import workloads
from tests.exact import rne

DTS = ["f32", "f16", "bf16"]
FLT_MIN = np.float32(2.0 ** -126)
Q = 127


def st(vals, dt):
    return workloads.f32_to_storage(np.asarray(vals, dtype=np.float32), dt)


def brute(yv, qmax=Q):
    """Exact reference for one row of fp32-widened values."""
    yv = np.asarray(yv, dtype=np.float32)
    if np.isnan(yv).any():
        return None, [0] * len(yv)
    a = np.max(np.abs(yv)) if len(yv) else np.float32(0)
    s = np.float32(a) / np.float32(qmax)          # IEEE fp32 division (numpy)
    if s < FLT_MIN:
        s = FLT_MIN
    codes = []
    for v in yv:
        q = np.float32(v) / np.float32(s)
        if np.isnan(q):
            codes.append(0)
            continue
        if np.isfinite(q) and np.isfinite(s):
            exact = Fraction(float(v)) / Fraction(float(s))
            lo = np.nextafter(q, np.float32(-np.inf))
            hi = np.nextafter(q, np.float32(np.inf))
            assert abs(Fraction(float(q)) - exact) <= abs(Fraction(float(lo)) - exact)
            assert abs(Fraction(float(q)) - exact) <= abs(Fraction(float(hi)) - exact)
        c = rne(Fraction(float(q)))
        codes.append(max(-qmax, min(qmax, c)))
    return s, codes


@pytest.mark.parametrize("dt", DTS)
def test_brute_force_tiny_rows(orc, dt):
    rng = np.random.default_rng(31)
    for trial in range(40):
        M, K = rng.integers(1, 9), int(rng.integers(1, 17)) * 2
        scale = 10.0 ** rng.uniform(-6, 4)
        y = st(rng.standard_normal((M, K)) * scale, dt)
        codes, scales = orc.quantize(y, dt, qmax=Q)
        yv = orc.decode(dt, y)
        for m in range(M):
            s, c = brute(yv[m])
            assert np.float32(scales[m]) == s
            assert list(codes[m]) == c


@pytest.mark.parametrize("dt", DTS)
def test_rounding_boundaries_half_even(orc, dt):
    # row max 127 -> s = 1 exactly; entries at k + 1/2 round half to even
    vals = [127.0, 0.5, 1.5, 2.5, 126.5, -126.5, 63.5, 64.5, -0.5, -63.5, 100.0, -127.0, 0.0, 3.0, 7.5, 8.5]
    codes, scales = orc.quantize(st([vals], dt), dt, qmax=Q)
    assert scales[0] == 1.0
    assert list(codes[0]) == [127, 0, 2, 2, 126, -126, 64, 64, 0, -64, 100, -127, 0, 3, 8, 8]


@pytest.mark.parametrize("dt", DTS)
def test_invariants_random(orc, dt):
    rng = np.random.default_rng(32)
    y = st(rng.standard_t(4, size=(64, 256)), dt)
    codes, scales = orc.quantize(y, dt, qmax=Q)
    yv = orc.decode(dt, y)
    assert (scales > 0).all()
    assert (np.abs(codes.astype(np.int32)).max(axis=1) == Q).all()   # the absmax maps to +-127
    assert codes.min() >= -Q                                          # -128 never appears
    # |y/s - c| <= 1/2 up to the rounding of the quotient (|q| <= 127, so within
    # 127 * 2^-24 of y/s)
    err = np.abs(scales[:, None].astype(np.float64) * codes - yv)
    assert (err <= scales[:, None].astype(np.float64) * (0.5 + Q * 2.0 ** -23)).all()
    # odd symmetry
    neg = workloads.f32_to_storage(-orc.decode(dt, y).astype(np.float32), dt)
    c2, s2 = orc.quantize(neg, dt, qmax=Q)
    assert np.array_equal(c2, -codes) and np.array_equal(s2, scales)


@pytest.mark.parametrize("dt", DTS)
def test_special_rows(orc, dt):
    big = {"f32": 3.0e38, "f16": 65504.0, "bf16": 3.0e38}[dt]
    rows = [
        [0.0] * 8,
        [1e-30, -1e-30, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0] if dt != "f16" else [6e-8, 0.0, 0, 0, 0, 0, 0, 0],
        [big, -big, big / 2, 1.0, 0.0, 0.0, 0.0, 0.0],
        [np.nan, 1.0, 0, 0, 0, 0, 0, 0],
        [np.inf, 1.0, -2.0, 0, 0, 0, 0, 0],
    ]
    y = st(rows, dt)
    codes, scales = orc.quantize(y, dt, qmax=Q)
    yv = orc.decode(dt, y)
    assert scales[0] == FLT_MIN and (codes[0] == 0).all()
    for m in (1, 2):
        s, c = brute(yv[m])
        assert scales[m] == s and list(codes[m]) == c
    assert np.isnan(scales[3]) and (codes[3] == 0).all()
    assert np.isinf(scales[4]) and list(codes[4][:3]) == [0, 0, 0]


def test_qmax_is_not_seven(orc):
    # the same row gives different codes in the two modes
    y = st([[7.0, 3.5, 1.0, -2.0]], "f32")
    c7, s7 = orc.quantize(y, "f32")
    c127, s127 = orc.quantize(y, "f32", qmax=Q)
    assert list(c7[0]) == [7, 4, 1, -2] and s7[0] == 1.0
    assert list(c127[0]) == [127, 64, 18, -36]
    assert s127[0] == np.float32(7.0) / np.float32(127.0)


def test_other_qmax_rejected(orc):
    with pytest.raises(ValueError):
        orc.quantize(st([[1.0, 2.0]], "f32"), "f32", qmax=15)


def test_int8_gemm_full_range(orc):
    # the integer product with INT8 weights over the whole range, against an
    # independent int64 matmul
    rng = np.random.default_rng(33)
    c = rng.integers(-127, 128, size=(9, 96)).astype(np.int8)
    w = rng.integers(-128, 128, size=(13, 96)).astype(np.int8)
    w[0, :] = -128
    c[0, :] = -127
    acc = orc.gemm(c, w)
    ref = c.astype(np.int64) @ w.astype(np.int64).T
    assert np.array_equal(acc, ref)
    assert acc[0, 0] == 127 * 128 * 96


def test_linear_int8_composition(orc):
    # the INT8 linear is rotation -> INT8 codes -> integer product -> E-B
    # epilogue; checked against an op-by-op numpy float32 evaluation
    rng = np.random.default_rng(34)
    M, K, N, g = 6, 128, 10, 64
    x = st(rng.standard_normal((M, K)), "bf16")
    h = np.ones((1, 1))
    while h.shape[0] < g:
        h = np.block([[h, h], [h, -h]])
    R = h / np.sqrt(g)
    w = rng.integers(-127, 128, size=(N, K)).astype(np.int8)
    s_w = st(rng.uniform(0.001, 0.01, N), "bf16")
    bias = st(rng.normal(0, 0.1, N), "bf16")
    res = orc.linear_int8(x, R, g, w, s_w, "bf16", "bf16", bias=bias)
    y = orc.rotate(x, R, g, "bf16")
    codes, scales = orc.quantize(y, "bf16", qmax=Q)
    assert np.array_equal(res["codes"], codes) and np.array_equal(res["scales"], scales)
    acc = codes.astype(np.int64) @ w.astype(np.int64).T
    swf = orc.decode("bf16", s_w).astype(np.float32)
    bf = orc.decode("bf16", bias).astype(np.float32)
    t = (acc.astype(np.float32) * scales[:, None]).astype(np.float32)
    t = (t * swf[None, :]).astype(np.float32)
    t = (t + bf[None, :]).astype(np.float32)
    _, expect = orc.round_to("bf16", t.astype(np.float64))
    assert np.array_equal(res["out"].view(np.uint16), expect.view(np.uint16))
    # rows / cols subsets give the same entries
    sub = orc.linear_int8(x, R, g, w, s_w, "bf16", "bf16", bias=bias, rows=[1, 4], cols=[2, 7, 9])
    assert np.array_equal(sub["out"].view(np.uint16), res["out"][np.ix_([1, 4], [2, 7, 9])].view(np.uint16))
