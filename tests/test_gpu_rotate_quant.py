"""GPU parity of the fused rotate + quantize kernel against the oracle.

Protocol: codes and scales must be bit-exact in both directions when both
sides quantize the same rotated values; the rotated values themselves must
agree to 1e-5 (group-normwise, fp32) or within 1 ulp (fp16/bf16); end to end,
codes may differ only by +-1 on at most 1e-4 of the entries."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.gpu_util import bits, dev, host, need_gpu, rotated_close, same_values, ulp_distance

pytestmark = pytest.mark.gpu

import bit_quantized_linear_rotate_amd as w4  # noqa: E402


def _rot_dev(R):
    return torch.from_numpy(np.ascontiguousarray(R, dtype=np.float32)).cuda()


def _draw(dt, M, K, seed, scale=1.0):
    rng = np.random.default_rng(seed)
    return workloads.f32_to_storage(rng.standard_t(4, size=(M, K)) * scale, dt)


def _quant_both_ways(dt, y_np, g_codes, g_scales):
    oc, os_ = oracle.quantize(y_np, dt)
    assert np.array_equal(oc, g_codes), "codes differ from the oracle on the same rotated values"
    assert np.array_equal(bits(os_), bits(g_scales)) or np.array_equal(
        np.isnan(os_), np.isnan(g_scales)) and np.array_equal(os_[~np.isnan(os_)],
                                                              g_scales[~np.isnan(g_scales)])


CASES = [
    # dtype, M, K, g  (ragged M, several tiles, all group sizes)
    ("bf16", 37, 3840, 64), ("f16", 21, 1024, 256), ("bf16", 9, 4096, 256), ("f16", 40, 512, 16),
    ("bf16", 17, 768, 32), ("f16", 5, 1024, 128), ("f32", 13, 256, 16), ("f32", 6, 512, 64),
    ("f32", 3, 1024, 256), ("bf16", 1, 96, 16),
]


@pytest.mark.parametrize("dt,M,K,g", CASES)
def test_codes_bit_exact_on_identical_rotated_input(dt, M, K, g):
    need_gpu()
    x = _draw(dt, M, K, seed=M * 7 + K)
    R = workloads.asymmetric_rotation(g, seed=g)
    y = oracle.rotate(x, R, g, dt)
    # direction 1: the GPU quantizes the oracle's rotated values (no rotation)
    c, s = w4.w4a4_rotate_quant_rowwise(dev(y, dt), None, 0)
    oc, os_ = oracle.quantize(y, dt)
    assert np.array_equal(host(c), oc)
    assert np.array_equal(bits(host(s)), bits(os_))
    # direction 2: the oracle quantizes the GPU's exported rotated values
    c2, s2, yg = w4.w4a4_rotate_quant_rowwise(dev(x, dt), _rot_dev(R), g, return_rotated=True)
    oc2, os2 = oracle.quantize(host(yg), dt)
    assert np.array_equal(host(c2), oc2)
    assert np.array_equal(bits(host(s2)), bits(os2))


@pytest.mark.parametrize("dt,M,K,g", CASES)
def test_rotated_values_within_tolerance(dt, M, K, g):
    need_gpu()
    x = _draw(dt, M, K, seed=M + K + g)
    R = workloads.asymmetric_rotation(g, seed=g + 1)
    yo = oracle.rotate(x, R, g, dt)
    _, _, yg = w4.w4a4_rotate_quant_rowwise(dev(x, dt), _rot_dev(R), g, return_rotated=True)
    yg = host(yg)
    if dt == "f32":
        a = yo.reshape(M, K // g, g).astype(np.float64)
        b = yg.reshape(M, K // g, g).astype(np.float64)
        err = np.abs(a - b).max(axis=2)
        ref = np.abs(a).max(axis=2)
        assert (err <= 1e-5 * ref).all()
    else:
        frac, beyond = rotated_close(yg, yo, x, R, g, dt)
        print(f"{dt} M={M} K={K} g={g}: {frac:.2e} of rotated values differ from the oracle, "
              f"{beyond} by more than 1 ulp (within the fp32 summation bound)")


@pytest.mark.parametrize("dt,M,K,g", CASES)
def test_end_to_end_code_flips(dt, M, K, g):
    need_gpu()
    x = _draw(dt, M, K, seed=3 * M + K)
    R = workloads.hadamard(g)
    yo, oc, os_ = oracle.rotate_quant(x, R, g, dt)
    c, s = w4.w4a4_rotate_quant_rowwise(dev(x, dt), _rot_dev(R), g)
    c, s = host(c), host(s)
    _, _, yg = w4.w4a4_rotate_quant_rowwise(dev(x, dt), _rot_dev(R), g, return_rotated=True)
    yg = host(yg)
    same_scale = bits(s) == bits(os_)
    # a row with another scale must be the oracle quantizer's result on the
    # GPU's own rotated row, whose values are within 1 ulp of the oracle's
    # (or the fp32 summation bound)
    other = np.flatnonzero(~same_scale)
    if other.size:
        qc, qs = oracle.quantize(yg[other], dt)
        assert np.array_equal(qc, c[other]) and np.array_equal(bits(qs), bits(s[other]))
        if dt != "f32":
            rotated_close(yg[other], yo[other], x[other], R, g, dt)
    d = np.abs(c.astype(np.int32) - oc)
    assert d.max(initial=0) <= 1
    assert (d > 0).sum() <= 1e-4 * M * K


@pytest.mark.parametrize("dt,M,K,g", [("bf16", 7, 48, 16), ("f16", 5, 80, 16), ("f32", 9, 272, 16),
                                      ("f32", 4, 512, 256), ("bf16", 3, 1040, 16)])
def test_fp64_sum_path_is_bit_exact(dt, M, K, g):
    # fp32 activations, and 16-bit widths the MFMA tiling does not cover
    # (K = 16 * odd with g = 16), take the path that sums the exact products in
    # fp64 in index order and rounds once: identical to the oracle.
    need_gpu()
    x = _draw(dt, M, K, seed=K)
    R = workloads.asymmetric_rotation(g, seed=1)
    c, s, yg = w4.w4a4_rotate_quant_rowwise(dev(x, dt), _rot_dev(R), g, return_rotated=True)
    yo, oc, os_ = oracle.rotate_quant(x, R, g, dt)
    assert np.array_equal(bits(host(yg)), bits(yo))
    assert np.array_equal(host(c), oc)
    assert np.array_equal(bits(host(s)), bits(os_))


@pytest.mark.parametrize("dt", ["f32", "f16", "bf16"])
def test_edge_rows(dt):
    need_gpu()
    K = 64
    big = {"f32": 3.0e38, "f16": 65504.0, "bf16": 3.3e38}[dt]
    tiny = {"f32": 1e-38, "f16": 6e-8, "bf16": 1e-38}[dt]
    rows = np.zeros((8, K), dtype=np.float32)
    rows[1, :] = np.linspace(-big, big, K)
    rows[2, :] = np.linspace(-tiny, tiny, K)
    rows[3, 5] = np.nan
    rows[4, 7] = np.inf
    rows[5, :] = np.arange(K) - 31.5        # exact half-integers at scale 1 after /s
    rows[6, :4] = [7.0, 0.5, 1.5, 2.5]
    rows[7, :] = -0.0
    y = workloads.f32_to_storage(rows, dt)
    c, s = w4.w4a4_rotate_quant_rowwise(dev(y, dt), None, 0)
    oc, os_ = oracle.quantize(y, dt)
    assert np.array_equal(host(c), oc)
    gs = host(s)
    assert np.array_equal(np.isnan(gs), np.isnan(os_))
    ok = ~np.isnan(os_)
    assert np.array_equal(bits(gs[ok]), bits(os_[ok]))


@pytest.mark.parametrize("dt,g", [("f16", 256), ("bf16", 64), ("f32", 16)])
def test_transposed_and_strided_views(dt, g):
    need_gpu()
    M, K = 33, 4 * g
    buf = _draw(dt, K, M, seed=5)                     # (K, M) buffer
    xt = dev(buf, dt).t()                            # (M, K) view, strides (1, M)
    R = workloads.hadamard(g)
    c, s, yg = w4.w4a4_rotate_quant_rowwise(xt, _rot_dev(R), g, return_rotated=True)
    oc, os2 = oracle.quantize(host(yg), dt)
    assert np.array_equal(host(c), oc) and np.array_equal(bits(host(s)), bits(os2))
    # and the same as on a contiguous copy of the same values
    c1, s1, y1 = w4.w4a4_rotate_quant_rowwise(xt.contiguous(), _rot_dev(R), g, return_rotated=True)
    assert np.array_equal(host(c1), host(c)) and np.array_equal(bits(host(s1)), bits(host(s)))
    assert np.array_equal(bits(host(y1)), bits(host(yg)))


@pytest.mark.parametrize("dt", ["bf16", "f16"])
def test_smoothing(dt):
    need_gpu()
    M, K, g = 7, 1024, 256
    x = _draw(dt, M, K, seed=9)
    sm = workloads.f32_to_storage(np.random.default_rng(3).uniform(0.5, 2.0, size=K), dt)
    R = workloads.hadamard(g)
    # smoothing alone is exact (one IEEE division, one rounding)
    c0, s0, y0 = w4.w4a4_rotate_quant_rowwise(dev(x, dt), None, 0, smooth=dev(sm, dt),
                                              return_rotated=True)
    assert np.array_equal(bits(host(y0)), bits(oracle.smooth(x, sm, dt)))
    c, s, yg = w4.w4a4_rotate_quant_rowwise(dev(x, dt), _rot_dev(R), g, smooth=dev(sm, dt),
                                            return_rotated=True)
    xs = oracle.smooth(x, sm, dt)
    yo = oracle.rotate(xs, R, g, dt)
    rotated_close(host(yg), yo, xs, R, g, dt)


def test_empty_and_rejections():
    need_gpu()
    x = torch.zeros((0, 64), dtype=torch.bfloat16, device="cuda")
    c, s = w4.w4a4_rotate_quant_rowwise(x, None, 0)
    assert c.shape == (0, 64) and s.shape == (0,)
    with pytest.raises(ValueError):
        w4.w4a4_rotate_quant_rowwise(torch.zeros((2, 63), dtype=torch.bfloat16, device="cuda"),
                                     None, 0)
    R = _rot_dev(workloads.hadamard(64))
    with pytest.raises(ValueError):
        w4.w4a4_rotate_quant_rowwise(torch.zeros((2, 96), dtype=torch.bfloat16, device="cuda"), R, 64)


@pytest.mark.parametrize("dt,g,M,K", [("f16", 256, 64, 1024), ("bf16", 256, 96, 2560),
                                      ("f16", 128, 40, 512), ("bf16", 64, 256, 192),
                                      ("f16", 256, 32, 256)])
def test_column_major_views_match_contiguous(dt, g, M, K):
    # a transposed view with M % 8 == 0 takes the column-major kernel (two
    # passes over 32-row blocks); the rotated bits, scales and codes must equal
    # those of a contiguous copy, and the codes those of the oracle quantizer
    need_gpu()
    buf = _draw(dt, K, M, seed=M + g)
    xt = dev(buf, dt).t()
    assert xt.stride() == (1, M)
    R = workloads.asymmetric_rotation(g, g)
    c, s, yg = w4.w4a4_rotate_quant_rowwise(xt, _rot_dev(R), g, return_rotated=True)
    c1, s1, y1 = w4.w4a4_rotate_quant_rowwise(xt.contiguous(), _rot_dev(R), g, return_rotated=True)
    assert np.array_equal(bits(host(yg)), bits(host(y1)))
    assert np.array_equal(bits(host(s)), bits(host(s1)))
    assert np.array_equal(host(c), host(c1))
    oc, os2 = oracle.quantize(host(yg), dt)
    assert np.array_equal(host(c), oc) and np.array_equal(bits(host(s)), bits(os2))
    # without the rotated export the codes are the same
    c2, s2 = w4.w4a4_rotate_quant_rowwise(xt, _rot_dev(R), g)
    assert np.array_equal(host(c2), host(c)) and np.array_equal(bits(host(s2)), bits(host(s)))


@pytest.mark.parametrize("dt,M,K,edge", [
    ("f16", 48, 1024, False), ("bf16", 48, 1024, False),
    # about a million smoothed values: a few hundred products land near a
    # rounding boundary of T, where the row-major kernel divides instead
    ("bf16", 64, 16384, False), ("f16", 128, 8192, False),
    # zeros in x, subnormal and huge smoothing factors
    ("bf16", 48, 2048, True), ("f16", 48, 2048, True),
])
def test_column_major_with_smoothing(dt, M, K, edge):
    """The contiguous copy takes the row-major kernel (product with a reciprocal,
    division near rounding boundaries), the transposed view the column-major one
    (IEEE division everywhere): the same bits."""
    need_gpu()
    g = 256
    buf = _draw(dt, K, M, seed=21)
    sm = np.random.default_rng(4).uniform(0.5, 2.0, size=K)
    if edge:
        buf = buf.copy()
        buf[::7, ::5] = 0
        tiny, huge = (1e-40, 2.0 ** 120) if dt == "bf16" else (3e-7, 6e4)
        sm[::11] = tiny          # (buf is x transposed: its row k is column k of x)
        buf[::11, :] = 0         # 0 / tiny = 0, with no overflow into the rotation
        sm[5::13] = huge
    sm = workloads.f32_to_storage(sm, dt)
    xt = dev(buf, dt).t()
    R = workloads.hadamard(g)
    c, s, yg = w4.w4a4_rotate_quant_rowwise(xt, _rot_dev(R), g, smooth=dev(sm, dt), return_rotated=True)
    c1, s1, y1 = w4.w4a4_rotate_quant_rowwise(xt.contiguous(), _rot_dev(R), g, smooth=dev(sm, dt),
                                              return_rotated=True)
    assert np.array_equal(bits(host(yg)), bits(host(y1)))
    assert np.array_equal(host(c), host(c1)) and np.array_equal(bits(host(s)), bits(host(s1)))


@pytest.mark.parametrize("dt,M,K,sm", [
    ("bf16", 1, 64, 64),          # one row, one group: TW 1, eight rows per block
    ("f16", 9, 512, 512),         # two rows per block, odd M: a partial block
    ("bf16", 67, 1024, 1024),     # 16 groups per row: TW 1, one row per block
    ("f16", 33, 1536, 1536),      # TW 2
    ("bf16", 130, 4096, 4096),    # 64 groups per row: every lane of TW 4
    ("bf16", 1600, 3840, 3840),   # more row blocks than waves: each wave takes several
    ("bf16", 2600, 3840, 3840),   # the row-streaming kernel (one wave per row)
    ("f16", 4100, 2560, 2560),    # row-streaming, two tiles a row, ragged last wave
    ("bf16", 2048, 3840, 4096),   # row-streaming with strided rows
    ("f16", 300, 3840, 4160),     # strided rows (a column slice of a wider buffer)
])
def test_row_major_g64_shapes(dt, M, K, sm):
    # row-major 16-bit rows with g = 64 (one to four 16-group tiles per row,
    # one to eight rows per wave, strided rows): the oracle's quantizer must reproduce codes and scales bit for bit from
    # the exported rotated values, which stay within 1 ulp of the oracle's,
    # and the codes must not depend on whether the rotated values are exported
    need_gpu()
    g = 64
    buf = _draw(dt, M, sm, seed=M + K)
    x = dev(buf, dt)[:, :K]
    assert x.stride() == (sm, 1)
    R = workloads.asymmetric_rotation(g, seed=5)
    c, s, yg = w4.w4a4_rotate_quant_rowwise(x, _rot_dev(R), g, return_rotated=True)
    oc, os2 = oracle.quantize(host(yg), dt)
    assert np.array_equal(host(c), oc) and np.array_equal(bits(host(s)), bits(os2))
    xk = np.ascontiguousarray(buf[:, :K])
    yo = oracle.rotate(xk, R, g, dt)
    frac, beyond = rotated_close(host(yg), yo, xk, R, g, dt)
    print(f"{dt} M={M} K={K}: {frac:.2e} of rotated values differ, {beyond} beyond 1 ulp")
    c2, s2 = w4.w4a4_rotate_quant_rowwise(x, _rot_dev(R), g)
    assert np.array_equal(host(c2), host(c)) and np.array_equal(bits(host(s2)), bits(host(s)))


@pytest.mark.parametrize("dt,M", [("bf16", 50), ("f16", 50), ("bf16", 2100), ("f16", 2100)])
def test_row_major_g64_with_smoothing(dt, M):
    need_gpu()
    K, g = 2048, 64
    x = _draw(dt, M, K, seed=13)
    sm = workloads.f32_to_storage(np.random.default_rng(6).uniform(0.5, 2.0, size=K), dt)
    R = workloads.hadamard(g)
    c, s, yg = w4.w4a4_rotate_quant_rowwise(dev(x, dt), _rot_dev(R), g, smooth=dev(sm, dt),
                                            return_rotated=True)
    xs = oracle.smooth(x, sm, dt)
    yo = oracle.rotate(xs, R, g, dt)
    rotated_close(host(yg), yo, xs, R, g, dt)
    oc, os2 = oracle.quantize(host(yg), dt)
    assert np.array_equal(host(c), oc) and np.array_equal(bits(host(s)), bits(os2))
