"""Pins for nibble unpacking (exhaustive), the exact integer GEMM (brute
force) and the fp32 epilogue (an independent numpy float32 implementation)."""
import numpy as np
import pytest
import torch

import workloads


def test_unpack_exhaustive_table(orc):
    wp = np.arange(256, dtype=np.uint8).reshape(1, 256)
    w = orc.unpack(wp, 512)
    for b in range(256):
        lo, hi = b & 15, b >> 4
        assert w[0, 2 * b] == (lo - 16 if lo >= 8 else lo)
        assert w[0, 2 * b + 1] == (hi - 16 if hi >= 8 else hi)
    # spot values of the convention: low nibble = even k, 0x8 = -8
    assert list(orc.unpack(np.array([[0x78, 0x8F, 0xF1]], dtype=np.uint8), 6)[0]) == \
        [-8, 7, -1, -8, 1, -1]


def test_pack_unpack_round_trip_all_pairs(orc):
    codes = np.array([[a, b] for a in range(-8, 8) for b in range(-8, 8)], dtype=np.int8)
    codes = codes.reshape(1, -1)
    assert np.array_equal(orc.unpack(orc.pack(codes), codes.shape[1]), codes)
    with pytest.raises(ValueError):
        orc.pack(np.array([[8, 0]], dtype=np.int8))


def test_generated_weights_never_use_minus_8(orc):
    rng = np.random.default_rng(1)
    wp = workloads.random_packed_weights(rng, 64, 512)
    w = orc.unpack(wp, 512)
    assert w.min() == -7 and w.max() == 7
    assert len(np.unique(w)) == 15


def test_gemm_brute_force(orc):
    rng = np.random.default_rng(31)
    M, N, K = 5, 7, 34
    c = rng.integers(-7, 8, size=(M, K)).astype(np.int8)
    w = rng.integers(-8, 8, size=(N, K)).astype(np.int8)
    acc = orc.gemm(c, w)
    for m in range(M):
        for n in range(N):
            assert acc[m, n] == sum(int(c[m, k]) * int(w[n, k]) for k in range(K))


def test_gemm_matches_float64_dot_and_group_partials(orc):
    rng = np.random.default_rng(32)
    M, N, K = 33, 65, 640
    c = rng.integers(-7, 8, size=(M, K)).astype(np.int8)
    w = rng.integers(-8, 8, size=(N, K)).astype(np.int8)
    acc = orc.gemm(c, w)
    assert np.array_equal(acc, (c.astype(np.float64) @ w.astype(np.float64).T).astype(np.int64))
    parts = orc.gemm(c, w, group=64)
    assert parts.shape == (M, K // 64, N)
    assert np.array_equal(parts.sum(axis=1), acc)
    assert np.array_equal(parts[:, 3, :], orc.gemm(c[:, 192:256], w[:, 192:256]))


def test_gemm_extreme_codes_no_overflow(orc):
    K = 1 << 16
    c = np.full((1, K), 7, dtype=np.int8)
    w = np.full((1, K), -8, dtype=np.int8)
    assert orc.gemm(c, w)[0, 0] == -56 * K


def _bf16_bits(f32):
    return torch.from_numpy(np.asarray(f32, np.float32)).to(torch.bfloat16).view(torch.int16) \
        .numpy().view(np.uint16)


def _to_out(t, dt):
    if dt == "f32":
        return t.view(np.uint32)
    if dt == "f16":
        with np.errstate(over="ignore"):
            return t.astype(np.float16).view(np.uint16)
    return _bf16_bits(t)


def _out_bits(out, dt):
    return out.view(np.uint32) if dt == "f32" else out.view(np.uint16)


@pytest.mark.parametrize("odt", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("with_bias", [False, True])
def test_epilogue_matches_numpy_float32_op_by_op(orc, odt, with_bias):
    rng = np.random.default_rng(41)
    M, N = 37, 29
    acc = rng.integers(-600000, 600000, size=(M, N)).astype(np.int64)
    sa = rng.uniform(1e-3, 3.0, size=M).astype(np.float32)
    sw = workloads.f32_to_storage(rng.uniform(0.005, 0.02, size=N), odt)
    bias = workloads.f32_to_storage(rng.normal(0, 0.1, size=N), odt) if with_bias else None
    out = orc.epilogue(acc, sa, sw, odt, odt, bias=bias, bias_dtype=odt if with_bias else None)
    t = acc.astype(np.float32)                       # exact: |acc| < 2^24
    t = t * sa[:, None]
    t = t * workloads.storage_to_f32(sw, odt)[None, :]
    if with_bias:
        t = t + workloads.storage_to_f32(bias, odt)[None, :]
    assert np.array_equal(_out_bits(out, odt), _to_out(t.astype(np.float32), odt))


def test_epilogue_group_scales_and_lowrank(orc):
    rng = np.random.default_rng(42)
    M, N, G, R = 9, 11, 6, 4
    acc = rng.integers(-3584, 3585, size=(M, G, N)).astype(np.int64)
    sa = rng.uniform(1e-3, 1.0, size=M).astype(np.float32)
    sw = workloads.f32_to_storage(rng.uniform(0.005, 0.02, size=(G, N)), "bf16")
    L = rng.standard_normal((M, R)).astype(np.float32)
    up = workloads.f32_to_storage(rng.normal(0, 0.1, size=(N, R)), "bf16")
    out = orc.epilogue(acc, sa, sw, "bf16", "bf16", group=64, L=L, proj_up=up, up_dtype="bf16")
    swf = workloads.storage_to_f32(sw, "bf16")
    upf = workloads.storage_to_f32(up, "bf16").astype(np.float64)
    t = np.zeros((M, N), dtype=np.float32)
    for gi in range(G):
        t = t + acc[:, gi, :].astype(np.float32) * swf[gi][None, :]
    t = t * sa[:, None]
    ell = (L.astype(np.float64) @ upf.T).astype(np.float32)
    t = t + ell
    assert np.array_equal(_out_bits(out, "bf16"), _bf16_bits(t))


@pytest.mark.parametrize("odt", ["f32", "f16", "bf16"])
def test_epilogue_special_cases(orc, odt):
    N = 8
    bias = workloads.f32_to_storage(np.linspace(-1, 1, N), odt)
    zero = np.zeros((1, N), dtype=np.int64)
    sw = workloads.f32_to_storage(np.full(N, 0.01), odt)
    out = orc.epilogue(zero, np.ones(1, np.float32), sw, odt, odt, bias=bias, bias_dtype=odt)
    assert np.array_equal(_out_bits(out, odt), _out_bits(bias.reshape(1, N), odt))
    acc = np.array([[1, -2, 3, 2 ** 24 + 1, -(2 ** 24) - 3, 100000, 7, 0]], dtype=np.int64)
    one = workloads.f32_to_storage(np.ones(N), odt)
    out = orc.epilogue(acc, np.ones(1, np.float32), one, odt, odt)
    assert np.array_equal(_out_bits(out, odt), _to_out(acc.astype(np.float32), odt))


def test_epilogue_f16_overflow_and_nan(orc):
    acc = np.array([[100000, -100000, 5]], dtype=np.int64)
    sa = np.array([1.0], dtype=np.float32)
    sw = workloads.f32_to_storage(np.array([1.0, 1.0, 1.0]), "f16")
    out = orc.epilogue(acc, sa, sw, "f16", "f16")
    assert np.isposinf(out[0, 0]) and np.isneginf(out[0, 1]) and out[0, 2] == 5
    out = orc.epilogue(acc, np.array([np.nan], dtype=np.float32), sw, "f16", "f16")
    assert np.isnan(out.astype(np.float32)).all()
