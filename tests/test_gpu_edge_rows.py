"""Edge rows through the rotate-quant kernels the benchmark times, with the
rotation on.

The pages test all-zero rows ("[Feat][Ascend] Add fused RotateQuant backend",
section "How was this patch tested?") and zeros, tiny and maximum finite
values and NaN/Inf ("[Perf][Ascend] Avoid activation pack/unpack in ConvRot
W4A4", section "Correctness and tests").  Each case below plants such rows
among ordinary ones, in a shape and layout for which the plan query confirms
the kernel under test is the one that runs:
  * "row":      contiguous rows, K=3840, g=64, M >= 2048 (the prefill kernel),
                with and without smoothing;
  * "wave":     contiguous rows, K=3840, g=64, 1536 <= M < 2048;
  * "g256":     contiguous rows, g=256, with and without smoothing (the
                low-rank layer's kernel);
  * "colmajor": a transposed view with M % 8 == 0 (the wide-K kernel);
  * "reg":      few contiguous rows, g=64 (the decode kernel);
  * "generic":  16-bit g=16 (exact fp64 sums).
Checks: the plan names the kernel; the oracle's quantizer reproduces the
GPU's codes and scales bit for bit from the GPU's exported rotated values;
those values agree with the oracle's rotation (NaN where it has NaN, equal
infinities, finite values within one unit in the last place of T or within
the fp32 summation bound of the group's products); and the
codes and scales do not depend on whether the rotated values are exported.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.gpu_util import bits, dev, host, need_gpu, rotated_close

pytestmark = pytest.mark.gpu

import bit_quantized_linear_rotate_amd as w4  # noqa: E402

MAXF = {"bf16": 3.3895313892515355e38, "f16": 65504.0}


def edge_rows(dt, K, g, rng):
    """A dict name -> (K,) fp32 row of edge patterns (representable in dt)."""
    nb = K // g
    rows = {}
    rows["zero"] = np.zeros(K)
    rows["neg_zero"] = np.full(K, -0.0)
    base = rng.standard_t(4, size=K)
    r = base.copy(); r[K // 3] = np.nan; rows["nan"] = r
    r = base.copy(); r[5] = np.inf; rows["pinf"] = r
    r = base.copy(); r[K - 1] = -np.inf; rows["ninf"] = r
    r = base.copy(); r[g + 1] = np.inf; r[g + 2] = -np.inf; rows["inf_minus_inf"] = r
    r = np.zeros(K); r[7] = np.inf; rows["inf_in_zeros"] = r
    mx = MAXF[dt]
    # one maximal entry per group (no overflow inside the rotation), signs mixed
    r = np.zeros(K); r[np.arange(nb) * g + (np.arange(nb) % g)] = mx * np.where(np.arange(nb) % 2, -1, 1)
    rows["max_one_hot"] = r
    rows["big_spread"] = rng.uniform(-1, 1, size=K) * (mx / g)
    if dt == "f16":
        rows["all_max"] = np.full(K, mx)          # rotated column 0 overflows to Inf
        rows["subnormal"] = rng.integers(-1023, 1024, size=K) * 2.0 ** -24
        rows["tiny_normal"] = rng.uniform(-1, 1, size=K) * 2.0 ** -13
    else:
        rows["subnormal"] = rng.integers(-127, 128, size=K) * 2.0 ** -133
        rows["tiny_normal"] = rng.uniform(-1, 1, size=K) * 1e-37   # scale clamped to 2^-126
        rows["tiny_mixed"] = np.where(rng.random(K) < 0.5, rng.uniform(-1, 1, size=K) * 1e-38, 0.0)
    # exact ties: one-hot groups whose rotated values are exact multiples of
    # the row's absmax; with a = 8*2^k/sqrt(g) the scale a/7 is inexact, with
    # a = 7*2^k/sqrt(g) it is exact, and the quotients sit on half-integers
    for name, top in (("ties_inexact_scale", 8.0), ("ties_exact_scale", 7.0)):
        r = np.zeros(K)
        vals = [top] + [h for h in (0.5, 1.5, 2.5, 3.5, 4.5, 5.5, 6.5, 4.0, 1.0, 2.0, 3.0)]
        for b in range(nb):
            r[b * g + (b * 5) % g] = vals[b % len(vals)] * 2.0 ** 3 * (1 if b % 3 else -1)
        rows[name] = r
    r = base.copy(); r[::17] *= 20.0; rows["outliers"] = r
    return rows


def build_matrix(dt, M, K, g, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_t(4, size=(M, K))
    er = edge_rows(dt, K, g, rng)
    names = list(er)
    # spread the edge rows: first and last rows, neighbours, the middle,
    # then every third row
    assert M >= 2 * len(names)
    slots = [0, 1, M - 1, M - 2, M // 2, M // 2 + 1] + list(range(3, M, 3))
    where, used = {}, set()
    for name in names:
        m = next(r for r in slots if r not in used)
        used.add(m)
        x[m] = er[name]
        where[name] = m
    with np.errstate(over="ignore", invalid="ignore"):
        xs = workloads.f32_to_storage(x.astype(np.float32), dt)
    return xs, where


def scales_equal(a, b):
    return np.array_equal(np.isnan(a), np.isnan(b)) and np.array_equal(
        bits(a[~np.isnan(a)]), bits(b[~np.isnan(b)]))


def run_case(dt, M, K, g, x_dev, x_host, kernel, smooth=None, rot_seed=3):
    R = workloads.asymmetric_rotation(g, seed=rot_seed)
    rot = torch.from_numpy(np.ascontiguousarray(R, dtype=np.float32)).cuda()
    sm_dev = dev(smooth, dt) if smooth is not None else None
    assert w4.w4a4_rotate_quant_plan(x_dev, rot, g, smooth=sm_dev) == kernel
    assert w4.w4a4_rotate_quant_plan(x_dev, rot, g, smooth=sm_dev, return_rotated=True) == kernel
    c, s, yg = w4.w4a4_rotate_quant_rowwise(x_dev, rot, g, smooth=sm_dev, return_rotated=True)
    c2, s2 = w4.w4a4_rotate_quant_rowwise(x_dev, rot, g, smooth=sm_dev)
    c, s, yg, c2, s2 = host(c), host(s), host(yg), host(c2), host(s2)
    # the timed configuration (no export) gives the same codes and scales
    assert np.array_equal(c, c2) and scales_equal(s, s2)
    # the oracle's quantizer reproduces codes and scales from the GPU's values
    oc, os_ = oracle.quantize(yg, dt)
    assert np.array_equal(c, oc), "codes differ from the oracle quantizer on the GPU's rotated values"
    assert scales_equal(s, os_), "scales differ from the oracle quantizer on the GPU's rotated values"
    # the rotated values agree with the oracle's rotation
    xs = oracle.smooth(x_host, smooth, dt) if smooth is not None else x_host
    yo = oracle.rotate(xs, R, g, dt)
    frac, beyond = rotated_close(yg, yo, xs, R, g, dt)
    # end to end: codes within one of the oracle's, scales equal unless the
    # rotated absmax element itself sits one ulp away
    _, rc, rs = oracle.rotate_quant(x_host, R, g, dt, smooth)
    same = np.array([scales_equal(s[i:i + 1], rs[i:i + 1]) for i in range(M)])
    dc = np.abs(c.astype(np.int32) - rc)
    assert dc.max(initial=0) <= 1
    print(f"{kernel} {dt} M={M} K={K} g={g}: {frac:.2e} of rotated values differ from the oracle "
          f"({beyond} beyond 1 ulp, within the fp32 summation bound), "
          f"{(~same).sum()} rows with another scale, {(dc > 0).sum()} code flips")
    return c, s


@pytest.mark.parametrize("dt", ["bf16", "f16"])
@pytest.mark.parametrize("smoothing", [False, True])
def test_row_kernel_edge_rows(dt, smoothing):
    # K=3840, g=64, M >= 2048: one wave per row -> the prefill kernel
    need_gpu()
    M, K, g = 2048, 3840, 64
    x, where = build_matrix(dt, M, K, g, seed=41)
    sm = None
    if smoothing:
        sm = workloads.f32_to_storage(np.random.default_rng(6).uniform(0.5, 2.0, size=K), dt)
    c, s = run_case(dt, M, K, g, dev(x, dt), x, "row", smooth=sm)
    assert (c[where["zero"]] == 0).all() and s[where["zero"]] == np.float32(2.0 ** -126)
    assert np.isnan(s[where["nan"]]) and (c[where["nan"]] == 0).all()


@pytest.mark.parametrize("dt", ["bf16", "f16"])
def test_wave_kernel_edge_rows(dt):
    # K=3840, g=64, 1536 <= M < 2048 row blocks -> the wave-per-row-block kernel
    need_gpu()
    M, K, g = 1600, 3840, 64
    x, where = build_matrix(dt, M, K, g, seed=40)
    c, s = run_case(dt, M, K, g, dev(x, dt), x, "wave")
    assert (c[where["zero"]] == 0).all() and s[where["zero"]] == np.float32(2.0 ** -126)
    assert np.isnan(s[where["nan"]]) and (c[where["nan"]] == 0).all()


@pytest.mark.parametrize("dt", ["bf16", "f16"])
@pytest.mark.parametrize("smoothing", [False, True])
def test_g256_kernel_edge_rows(dt, smoothing):
    need_gpu()
    M, K, g = 96, 4096, 256
    x, where = build_matrix(dt, M, K, g, seed=42)
    sm = None
    if smoothing:
        sm = workloads.f32_to_storage(np.random.default_rng(5).uniform(0.5, 2.0, size=K), dt)
    c, s = run_case(dt, M, K, g, dev(x, dt), x, "g256", smooth=sm)
    assert (c[where["zero"]] == 0).all()


@pytest.mark.parametrize("dt,g", [("f16", 256), ("bf16", 256), ("f16", 64), ("bf16", 128)])
def test_colmajor_kernel_edge_rows(dt, g):
    need_gpu()
    M, K = 256, 2048
    x, where = build_matrix(dt, M, K, g, seed=43 + g)
    xt = dev(np.ascontiguousarray(x.T), dt).t()     # (M, K) view of a (K, M) buffer
    assert xt.stride() == (1, M)
    c, s = run_case(dt, M, K, g, xt, x, "colmajor")
    assert (c[where["zero"]] == 0).all()


@pytest.mark.parametrize("dt", ["bf16", "f16"])
def test_reg_kernel_edge_rows(dt):
    need_gpu()
    M, K, g = 40, 3840, 64
    x, _ = build_matrix(dt, M, K, g, seed=44)
    run_case(dt, M, K, g, dev(x, dt), x, "reg")


@pytest.mark.parametrize("dt", ["bf16", "f16"])
def test_g16_edge_rows_exact(dt):
    # 16-bit g=16 sums each group on its own (no zero padding that an Inf
    # could meet); the rotated values are then the oracle's exactly
    need_gpu()
    M, K, g = 40, 1024, 16
    x, where = build_matrix(dt, M, K, g, seed=45)
    xd = dev(x, dt)
    run_case(dt, M, K, g, xd, x, "generic")
    R = workloads.asymmetric_rotation(g, seed=3)
    _, s, yg = w4.w4a4_rotate_quant_rowwise(xd, torch.from_numpy(np.ascontiguousarray(R, dtype=np.float32)).cuda(), g,
                                            return_rotated=True)
    yo = oracle.rotate(x, R, g, dt)
    assert np.array_equal(oracle.decode(dt, host(yg)), oracle.decode(dt, yo), equal_nan=True)
    assert s[where["pinf"]].item() == float("inf")
