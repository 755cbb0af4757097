"""Pins for the oracle's SVDQuant-variant steps (source page
comfy_kitchen/tensor/svdquant_w4a4.py: the ``_w4a4_forward`` docstring (the
act_unsigned shift 0.171875 onto the unsigned [0, 15] grid, the low-rank
branch on the raw activation) and the module docstring (INT4 group size 64)):

* the shift against numpy / torch float conversions of an fp32 add;
* the quantizer on both grids, per row and per 64-group, by brute force in
  exact rationals; group independence (a NaN or a large value in one group
  leaves the other groups alone); half-even ties on an exact unit scale;
* the epilogue with per-group activation scales against an independent
  float32 evaluation in the stated order, and exactly (rationals) where every
  product is exact;
* the layer composition, including that the low-rank branch sees the raw x."""
from fractions import Fraction

import numpy as np
import pytest
import torch

import workloads
from tests.exact import rne

FLT_MIN = np.float32(2.0 ** -126)
DTS = ["f32", "f16", "bf16"]


def st(vals, dt):
    return workloads.f32_to_storage(np.asarray(vals, dtype=np.float32), dt)


def brute_block(yv, unsigned):
    """Exact reference for one block of fp32-widened values."""
    yv = np.asarray(yv, dtype=np.float32)
    qmax = 15 if unsigned else 7
    lo = 0 if unsigned else -7
    if np.isnan(yv).any():
        return None, [0] * len(yv)
    a = np.max(np.abs(yv)) if len(yv) else np.float32(0)
    s = np.float32(a) / np.float32(qmax)
    if s < FLT_MIN:
        s = FLT_MIN
    codes = []
    for v in yv:
        q = np.float32(v) / np.float32(s)
        if np.isnan(q):
            codes.append(0)
            continue
        c = rne(Fraction(float(q))) if np.isfinite(q) else (qmax if q > 0 else lo)
        codes.append(max(lo, min(qmax, c)))
    return s, codes


@pytest.mark.parametrize("dt", DTS)
def test_shift_is_one_fp32_add_rounded_to_T(orc, dt):
    rng = np.random.default_rng(41)
    vals = np.concatenate([rng.standard_normal(200) * 3, [-0.171875, -0.17, 0.0, -0.0, 1e-8, -1e-8],
                           [60000.0, -65504.0] if dt == "f16" else [3.0e38, -3.0e38, 1e-40]])
    x = st([vals], dt)
    got = orc.shift(x, dt)
    xf = workloads.storage_to_f32(x, dt)
    with np.errstate(over="ignore"):
        summed = (xf + np.float32(0.171875)).astype(np.float32)
    if dt == "f32":
        ref = summed
    elif dt == "f16":
        ref = summed.astype(np.float16)
    else:
        ref = torch.from_numpy(summed).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(np.asarray(got).view(np.uint8), np.asarray(ref).view(np.uint8))


@pytest.mark.parametrize("dt", DTS)
@pytest.mark.parametrize("unsigned", [False, True])
@pytest.mark.parametrize("group", [0, 64])
def test_quantizer_brute_force(orc, dt, unsigned, group):
    rng = np.random.default_rng(42 + group + unsigned)
    for trial in range(12):
        M, K = int(rng.integers(1, 4)), 128
        scale = 10.0 ** rng.uniform(-5, 3)
        raw = rng.standard_normal((M, K)) * scale
        if unsigned:
            raw = np.abs(raw) - 0.05 * scale        # a few slightly negative entries
        y = st(raw, dt)
        codes, scales = orc.quantize_groups(y, dt, unsigned, group)
        yv = orc.decode(dt, y)
        glen = group or K
        for m in range(M):
            for gi in range(K // glen):
                blk = slice(gi * glen, (gi + 1) * glen)
                s, c = brute_block(yv[m, blk], unsigned)
                got_s = scales[m, gi] if group else scales[m]
                assert np.float32(got_s) == s
                assert list(codes[m, blk]) == c


@pytest.mark.parametrize("dt", DTS)
def test_unsigned_grid_ties_and_negatives(orc, dt):
    # block max 15 -> s = 1 exactly: k + 1/2 rounds to even, negatives give 0
    vals = [15.0, 0.5, 1.5, 2.5, 14.5, 13.5, 7.5, 8.5, -0.25, -3.0, 0.0, 3.0, 9.0, 10.5, 11.5, 12.5]
    codes, scales = orc.quantize_groups(st([vals], dt), dt, True, 0)
    assert scales[0] == 1.0
    assert list(codes[0]) == [15, 0, 2, 2, 14, 14, 8, 8, 0, 0, 0, 3, 9, 10, 12, 12]


@pytest.mark.parametrize("unsigned", [False, True])
def test_groups_are_independent_and_special_blocks(orc, unsigned):
    dt = "bf16"
    rng = np.random.default_rng(43)
    base = np.abs(rng.standard_normal((1, 256))) + 0.1
    y = base.copy()
    y[0, 70] = np.nan          # group 1 only
    y[0, 130] = 1000.0         # group 2 only
    y[0, 192:256] = 0.0        # group 3 all zero
    codes, scales = orc.quantize_groups(st(y, dt), dt, unsigned, 64)
    c0, s0 = orc.quantize_groups(st(base[:, :64], dt), dt, unsigned, 0)
    assert np.array_equal(codes[0, :64], c0[0]) and scales[0, 0] == s0[0]
    assert np.isnan(scales[0, 1]) and (codes[0, 64:128] == 0).all()
    assert scales[0, 2] == np.float32(np.float32(1000.0) / np.float32(15 if unsigned else 7))
    assert scales[0, 3] == FLT_MIN and (codes[0, 192:] == 0).all()
    # the same row quantized whole has one NaN scale for everything
    cr, sr = orc.quantize_groups(st(y, dt), dt, unsigned, 0)
    assert np.isnan(sr[0]) and (cr == 0).all()


def test_signed_whole_row_is_the_w4a4_quantizer(orc):
    rng = np.random.default_rng(44)
    y = st(rng.standard_t(4, size=(16, 192)), "f16")
    c1, s1 = orc.quantize_groups(y, "f16", False, 0)
    c2, s2 = orc.quantize(y, "f16")
    assert np.array_equal(c1, c2) and np.array_equal(s1, s2)


def _epilogue_ag_numpy(acc, sa, sw, sw_group, bias):
    """Independent float32 evaluation in the order of reading R19."""
    M, G, N = acc.shape
    out = np.empty((M, N), dtype=np.float32)
    for m in range(M):
        for n in range(N):
            t = np.float32(0)
            for g in range(G):
                p = np.float32(np.float32(acc[m, g, n]) * sa[m, g])
                if sw_group:
                    p = np.float32(p * sw[g, n])
                t = np.float32(t + p)
            if not sw_group:
                t = np.float32(t * sw[n])
            if bias is not None:
                t = np.float32(t + bias[n])
            out[m, n] = t
    return out


@pytest.mark.parametrize("sw_group", [0, 64])
def test_epilogue_group_activation_scales_order(orc, sw_group):
    rng = np.random.default_rng(45)
    M, G, N = 5, 4, 7
    acc = rng.integers(-5000, 5000, size=(M, G, N)).astype(np.int64)
    sa = rng.uniform(0.01, 0.3, size=(M, G)).astype(np.float32)
    sw = rng.uniform(0.001, 0.02, size=(G, N) if sw_group else (N,)).astype(np.float32)
    bias = rng.normal(0, 0.1, size=N).astype(np.float32)
    got = orc.epilogue_ag(acc, sa, sw, "f32", "f32", sw_group, bias=bias, bias_dtype="f32")
    ref = _epilogue_ag_numpy(acc, sa, sw, sw_group, bias)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))
    # the test tells the stated order from a plausible other one: the two
    # scales multiplied together first (group weight scales), or the
    # per-channel weight scale applied inside the sum
    other = np.empty_like(ref)
    for m in range(M):
        for n in range(N):
            t = np.float32(0)
            for g in range(G):
                if sw_group:
                    sc = np.float32(sa[m, g] * sw[g, n])
                    t = np.float32(t + np.float32(np.float32(acc[m, g, n]) * sc))
                else:
                    p = np.float32(np.float32(acc[m, g, n]) * sa[m, g])
                    t = np.float32(t + np.float32(p * sw[n]))
            other[m, n] = np.float32(t + bias[n])
    assert not np.array_equal(other.view(np.uint32), ref.view(np.uint32))


def test_epilogue_group_activation_scales_exact(orc):
    # power-of-two scales: every product is exact; the sum of 4 small exact
    # terms is exact in fp32, so the result is the rational value rounded once
    rng = np.random.default_rng(46)
    M, G, N = 3, 4, 5
    acc = rng.integers(-1000, 1000, size=(M, G, N)).astype(np.int64)
    sa = (2.0 ** rng.integers(-6, 0, size=(M, G))).astype(np.float32)
    sw = (2.0 ** rng.integers(-8, -2, size=(G, N))).astype(np.float32)
    got = orc.epilogue_ag(acc, sa, sw, "f32", "bf16", 64)
    for m in range(M):
        for n in range(N):
            exact = sum(Fraction(int(acc[m, g, n])) * Fraction(float(sa[m, g])) * Fraction(float(sw[g, n]))
                        for g in range(G))
            ref = orc.round_to("bf16", np.array([float(exact)]))[1][0]
            assert got[m, n] == ref


def test_linear_svdquant_composition(orc):
    rng = np.random.default_rng(47)
    M, K, N, R = 6, 256, 9, 4
    dt = "bf16"
    x = st(rng.standard_normal((M, K)), dt)
    wq = rng.integers(-8, 8, size=(N, K)).astype(np.int8)
    wp = orc.pack(wq)
    sw = st(rng.uniform(0.005, 0.02, size=(K // 64, N)), "bf16")
    sm = st(rng.uniform(0.5, 2.0, size=K), dt)
    down = st(rng.standard_normal((K, R)) / 16, dt)
    up = st(rng.normal(0, 0.1, size=(N, R)), dt)
    bias = st(rng.normal(0, 0.1, size=N), dt)
    res = orc.linear_svdquant(x, wp, sw, dt, "bf16", 64, sm, bias, down, up, act_unsigned=True, act_group=64)
    xm = orc.shift(x, dt)
    codes, scales = orc.quantize_groups(orc.smooth(xm, sm, dt), dt, True, 64)
    assert codes.min() >= 0 and np.array_equal(res["codes"], codes)
    L = orc.lowrank_down(x, down, dt)                      # the raw x, not the shifted one
    assert np.array_equal(res["L"], L)
    assert not np.array_equal(orc.lowrank_down(xm, down, dt), L)
    acc = orc.gemm(codes, wq, 64)
    ref = orc.epilogue_ag(acc, scales, sw, "bf16", dt, 64, bias=bias, bias_dtype=dt, L=L, proj_up=up,
                          up_dtype=dt)
    assert np.array_equal(res["out"], ref)
    # rows / cols subsets give the same entries
    sub = orc.linear_svdquant(x, wp, sw, dt, "bf16", 64, sm, bias, down, up, act_unsigned=True, act_group=64,
                              rows=[1, 4], cols=[0, 5, 8])
    assert np.array_equal(sub["out"], res["out"][np.ix_([1, 4], [0, 5, 8])])
    # per-row activation scales (act_group 0) go through the W4A4 epilogue
    r0 = orc.linear_svdquant(x, wp, sw, dt, "bf16", 64, sm, bias, down, up, act_unsigned=False, act_group=0)
    c0, s0 = orc.quantize(orc.smooth(x, sm, dt), dt)
    ref0 = orc.epilogue(orc.gemm(c0, wq, 64), s0, sw, "bf16", dt, bias=bias, bias_dtype=dt, group=64, L=L,
                        proj_up=up, up_dtype=dt)
    assert np.array_equal(r0["out"], ref0)
