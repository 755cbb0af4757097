"""GPU parity of the W4A4 GEMM + epilogue against the oracle.

Given identical codes and scales: the INT32 sums are bit-exact, and the
outputs are bit-exact under the epilogue order fp32(acc) * s_a * s_w + bias
(each operation rounded separately).  With a low-rank term the GPU sums the
rank terms in fp32 while the oracle sums them in fp64, so the bound is one
ulp of the output dtype plus the fp32 rounding of that short sum."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.gpu_util import bits, dev, host, need_gpu, ulp_distance

pytestmark = pytest.mark.gpu

import bit_quantized_linear_rotate_amd as w4  # noqa: E402


def _operands(M, K, N, odt, sw_dt, group=0, bias=True, seed=0):
    rng = np.random.default_rng(seed)
    codes = rng.integers(-7, 8, size=(M, K)).astype(np.int8)
    scales = rng.uniform(0.01, 0.5, size=M).astype(np.float32)
    wp = workloads.random_packed_weights(rng, N, K)
    if group:
        sw = workloads.f32_to_storage(rng.uniform(0.005, 0.02, size=(K // group, N)), sw_dt)
    else:
        sw = workloads.f32_to_storage(rng.uniform(0.005, 0.02, size=N), sw_dt)
    b = workloads.f32_to_storage(rng.normal(0, 0.1, size=N), odt) if bias else None
    return codes, scales, wp, sw, b


SHAPES = [  # (M, K, N): tiles of 128 x 128 x 64 plus ragged tails
    (1, 256, 256), (32, 3840, 384), (130, 640, 200), (257, 1024, 129), (64, 96, 64),
    (200, 2048, 300), (5, 160, 17), (128, 64, 128),
    # 64 < M <= 128 with K % 64 == 0: the 128 x 128 kernel's buffer-load
    # staging, rows past M and columns past N reading zeros
    (100, 192, 130), (77, 1024, 40),
]


@pytest.mark.parametrize("M,K,N", SHAPES)
@pytest.mark.parametrize("odt", ["f32", "bf16", "f16"])
def test_acc_and_output_bit_exact(M, K, N, odt):
    need_gpu()
    codes, sa, wp, sw, b = _operands(M, K, N, odt, odt, seed=M + K + N)
    out, acc = w4.w4a4_gemm_from_codes(dev(codes), dev(sa), dev(wp), dev(sw, odt), bias=dev(b, odt),
                                       out_dtype={"f32": torch.float32, "f16": torch.float16,
                                                  "bf16": torch.bfloat16}[odt], return_acc=True)
    oacc = oracle.gemm(codes, oracle.unpack(wp, K))
    assert np.array_equal(host(acc).astype(np.int64), oacc)
    oout = oracle.epilogue(oacc, sa, sw, odt, odt, bias=b, bias_dtype=odt)
    assert np.array_equal(bits(host(out)), bits(oout))


@pytest.mark.parametrize("sw_dt", ["f32", "bf16", "f16"])
def test_no_bias_and_mixed_dtypes(sw_dt):
    need_gpu()
    M, K, N = 70, 512, 96
    codes, sa, wp, sw, _ = _operands(M, K, N, "bf16", sw_dt, bias=False, seed=3)
    out = w4.w4a4_gemm_from_codes(dev(codes), dev(sa), dev(wp), dev(sw, sw_dt),
                                  out_dtype=torch.float32)
    oout = oracle.epilogue(oracle.gemm(codes, oracle.unpack(wp, K)), sa, sw, sw_dt, "f32")
    assert np.array_equal(bits(host(out)), bits(oout))


@pytest.mark.parametrize("M,K,N", [(33, 1024, 130), (128, 4096, 256), (300, 2048, 260)])
def test_forced_k_chunks_are_exact(M, K, N):
    need_gpu()
    codes, sa, wp, sw, b = _operands(M, K, N, "bf16", "bf16", seed=11)
    ref, racc = w4.w4a4_gemm_from_codes(dev(codes), dev(sa), dev(wp), dev(sw, "bf16"),
                                        bias=dev(b, "bf16"), return_acc=True)
    for kc in (64, 192, 1024):
        out, acc = w4.w4a4_gemm_from_codes(dev(codes), dev(sa), dev(wp), dev(sw, "bf16"),
                                           bias=dev(b, "bf16"), return_acc=True, k_chunk=kc)
        assert torch.equal(acc, racc)
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16))


def test_extreme_codes_int32_range():
    need_gpu()
    M, N, K = 16, 16, 16384
    codes = np.full((M, K), 7, dtype=np.int8)
    codes[1::2] = -7
    wq = np.full((N, K), -8, dtype=np.int8)
    wq[::3] = 7
    wp = oracle.pack(wq)
    sa = np.ones(M, np.float32)
    sw = np.ones(N, np.float32)
    out, acc = w4.w4a4_gemm_from_codes(dev(codes), dev(sa), dev(wp), dev(sw),
                                       out_dtype=torch.float32, return_acc=True)
    oacc = oracle.gemm(codes, wq)
    assert np.array_equal(host(acc).astype(np.int64), oacc)
    assert np.abs(oacc).max() == 56 * K


@pytest.mark.parametrize("M,K,N", [(40, 1024, 96), (129, 2048, 200)])
def test_group_scales_and_lowrank(M, K, N):
    need_gpu()
    codes, sa, wp, sw, _ = _operands(M, K, N, "bf16", "bf16", group=64, bias=False, seed=5)
    rng = np.random.default_rng(6)
    R = 32
    L = rng.standard_normal((M, R)).astype(np.float32)
    up = workloads.f32_to_storage(rng.normal(0, 0.1, size=(N, R)), "bf16")
    parts = oracle.gemm(codes, oracle.unpack(wp, K), group=64)
    # without the low-rank term: bit-exact
    out = w4.w4a4_gemm_from_codes(dev(codes), dev(sa), dev(wp), dev(sw, "bf16"), w_scale_group=64,
                                  out_dtype=torch.bfloat16)
    oout = oracle.epilogue(parts, sa, sw, "bf16", "bf16", group=64)
    assert np.array_equal(bits(host(out)), bits(oout))
    # with it: within one bf16 ulp
    out = w4.w4a4_gemm_from_codes(dev(codes), dev(sa), dev(wp), dev(sw, "bf16"), w_scale_group=64,
                                  lora_act=dev(L), proj_up=dev(up, "bf16"), out_dtype=torch.bfloat16)
    oout = oracle.epilogue(parts, sa, sw, "bf16", "bf16", group=64, L=L, proj_up=up, up_dtype="bf16")
    assert ulp_distance(host(out), oout, "bf16").max() <= 1


@pytest.mark.parametrize("sw_dt", ["f32", "bf16", "f16"])
def test_group_scales_every_scale_dtype(sw_dt):
    need_gpu()
    M, K, N = 150, 1024, 260
    codes, sa, wp, sw, b = _operands(M, K, N, "f32", sw_dt, group=64, seed=21)
    out = w4.w4a4_gemm_from_codes(dev(codes), dev(sa), dev(wp), dev(sw, sw_dt), w_scale_group=64,
                                  bias=dev(b, "f32"), out_dtype=torch.float32)
    parts = oracle.gemm(codes, oracle.unpack(wp, K), group=64)
    oout = oracle.epilogue(parts, sa, sw, sw_dt, "f32", group=64, bias=b, bias_dtype="f32")
    assert np.array_equal(bits(host(out)), bits(oout))


def test_group_scales_below_2_pow_minus_122():
    """fp32 group scales so small that scale / 16 is not exact: the workgroups
    that meet one redo their K loop in the exact form; results stay bit-exact."""
    need_gpu()
    M, K, N = 150, 1024, 260
    codes, sa, wp, sw, _ = _operands(M, K, N, "f32", "f32", group=64, seed=22)
    rng = np.random.default_rng(23)
    sw = sw.copy()
    sw[:, 7] = rng.uniform(1e-40, 1e-37, size=K // 64).astype(np.float32)  # one whole column
    sw[5, 200] = np.float32(3.3e-39)                                      # one entry elsewhere
    parts = oracle.gemm(codes, oracle.unpack(wp, K), group=64)
    # the planted scales do make float(16 s) * (scale / 16) differ from s * scale
    s7 = parts[:, :, 7].astype(np.float32)
    q7 = (sw[:, 7] * np.float32(0.0625)).astype(np.float32)
    assert not np.array_equal((s7 * np.float32(16)) * q7[None, :], s7 * sw[:, 7][None, :])
    out = w4.w4a4_gemm_from_codes(dev(codes), dev(sa), dev(wp), dev(sw, "f32"), w_scale_group=64,
                                  out_dtype=torch.float32)
    oout = oracle.epilogue(parts, sa, sw, "f32", "f32", group=64)
    assert np.array_equal(bits(host(out)), bits(oout))


@pytest.mark.parametrize("sw_dt", ["bf16", "f16"])
def test_group_scales_16bit_special_values(sw_dt):
    """16-bit group scales take the fast path that starts each group's INT32
    sum from the pattern of 1.5 * 2^23 and folds the conversion into one fma.
    Zero, negative and subnormal scales stay on it (the sums of zero terms
    cannot change a sum that starts at +0); Inf, NaN and scales whose
    1.5 * 2^23 * scale / 16 overflows send their workgroup to the exact path.
    All of it bit-exact, with zero code rows and extreme codes mixed in."""
    need_gpu()
    M, K, N = 300, 1024, 384
    codes, sa, wp, sw, _ = _operands(M, K, N, "f32", sw_dt, group=64, seed=24)
    codes[3] = 0                 # zero rows: every group sum is 0
    codes[4] = 7
    codes[5] = -7
    swf = workloads.storage_to_f32(sw, sw_dt).copy()
    swf[:, 10] = 0.0
    swf[:, 11] = -swf[:, 11]
    swf[2, 12] = -0.0
    swf[:, 13] = 2.0 ** -20 if sw_dt == "f16" else 2.0 ** -130   # subnormal in the scale's format
    swf[0, 140] = np.inf         # (a tile of its own column block)
    swf[1, 300] = np.nan
    swf[7, 290] = 6.0e4 if sw_dt == "f16" else 3.0e38             # large, finite
    sw = workloads.f32_to_storage(swf, sw_dt)
    parts = oracle.gemm(codes, oracle.unpack(wp, K), group=64)
    for odt, tdt in (("f32", torch.float32), ("bf16", torch.bfloat16)):
        out = w4.w4a4_gemm_from_codes(dev(codes), dev(sa), dev(wp), dev(sw, sw_dt), w_scale_group=64,
                                      out_dtype=tdt)
        oout = oracle.epilogue(parts, sa, sw, sw_dt, odt, group=64)
        go = host(out)
        # bit-exact, signed zeros included; a NaN is any NaN (the pages fix no
        # NaN payload: the oracle stores one canonical NaN, the GPU's
        # conversion keeps the f32 NaN's sign)
        nan = np.isnan(oracle.decode(odt, oout))
        assert nan[:, 300].all() and np.array_equal(np.isnan(oracle.decode(odt, go)), nan)
        assert np.array_equal(bits(go)[~nan], bits(oout)[~nan]), (odt, sw_dt)


def test_lowrank_down_matches_oracle():
    need_gpu()
    rng = np.random.default_rng(8)
    # ranks 16/32/64 take the sixteen-wave kernel (K slices of 32, four in
    # flight per wave; K = 2080 leaves a ragged last round), other ranks the
    # four-wave one, fp32 the plain loop
    for dt, M, K, R in [("bf16", 37, 2048, 32), ("f16", 16, 512, 16), ("f32", 5, 256, 8),
                        ("bf16", 100, 2080, 64), ("f16", 33, 16384, 32), ("bf16", 20, 96, 16),
                        ("bf16", 40, 1024, 20), ("f16", 17, 544, 48)]:
        x = workloads.f32_to_storage(rng.standard_normal((M, K)), dt)
        down = workloads.f32_to_storage(rng.standard_normal((K, R)) / np.sqrt(K), dt)
        L = host(w4.w4a4_lowrank_down(dev(x, dt), dev(down, dt)))
        Lo = oracle.lowrank_down(x, down, dt)
        xa = np.abs(oracle.decode(dt, x)) @ np.abs(oracle.decode(dt, down))
        # recursive fp32 summation bound: |err| <= (K + 2) u sum |x d|, u = 2^-24
        assert (np.abs(L.astype(np.float64) - Lo) <= (K + 2) * 2.0 ** -24 * xa + 1e-30).all()


def test_empty_shapes():
    need_gpu()
    z = torch.zeros((0, 64), dtype=torch.int8, device="cuda")
    out = w4.w4a4_gemm_from_codes(z, torch.zeros(0, device="cuda"),
                                  torch.zeros((8, 32), dtype=torch.uint8, device="cuda"),
                                  torch.ones(8, device="cuda"), out_dtype=torch.float32)
    assert out.shape == (0, 8)


@pytest.mark.parametrize("M,K,N", [(300, 2048, 520), (513, 1024, 257), (256, 3840, 256),
                                   (1000, 640, 1000), (300, 2048, 528), (1000, 640, 1008)])
@pytest.mark.parametrize("odt", ["f32", "bf16", "f16"])
def test_output_bit_exact_without_acc_export(M, K, N, odt):
    # the large-tile kernels run only when the INT32 sums are not exported
    need_gpu()
    codes, sa, wp, sw, b = _operands(M, K, N, odt, odt, seed=M * 3 + N)
    out = w4.w4a4_gemm_from_codes(dev(codes), dev(sa), dev(wp), dev(sw, odt), bias=dev(b, odt),
                                  out_dtype={"f32": torch.float32, "f16": torch.float16,
                                             "bf16": torch.bfloat16}[odt])
    oacc = oracle.gemm(codes, oracle.unpack(wp, K))
    oout = oracle.epilogue(oacc, sa, sw, odt, odt, bias=b, bias_dtype=odt)
    assert np.array_equal(bits(host(out)), bits(oout))
    # forced K-chunks through the same kernels give the same bits
    out2 = w4.w4a4_gemm_from_codes(dev(codes), dev(sa), dev(wp), dev(sw, odt), bias=dev(b, odt),
                                   out_dtype=out.dtype, k_chunk=128)
    assert np.array_equal(bits(host(out2)), bits(oout))


@pytest.mark.parametrize("M,K,N", [(4100, 256, 4130), (4352, 384, 4112), (4100, 256, 4128)])
def test_several_tiles_per_workgroup(M, K, N):
    # more 256 x 256 tiles than CUs: the persistent kernel walks several tiles
    # per workgroup and prefetches the next tile during the last steps; ragged
    # M and N on the last tiles, K at two and three 128-steps
    need_gpu()
    codes, sa, wp, sw, b = _operands(M, K, N, "bf16", "bf16", seed=M + K + N)
    out = w4.w4a4_gemm_from_codes(dev(codes), dev(sa), dev(wp), dev(sw, "bf16"),
                                  bias=dev(b, "bf16"), out_dtype=torch.bfloat16)
    oacc = oracle.gemm(codes, oracle.unpack(wp, K))
    oout = oracle.epilogue(oacc, sa, sw, "bf16", "bf16", bias=b, bias_dtype="bf16")
    assert np.array_equal(bits(host(out)), bits(oout))


@pytest.mark.parametrize("sw_dt", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("b_dt", [None, "f32", "bf16", "f16"])
def test_pingpong_scale_and_bias_dtypes(sw_dt, b_dt):
    # the ping-pong kernel stages the scales and bias in LDS as stored and
    # widens them in the epilogue: every dtype pair, with and without bias,
    # on a ragged 2 x 2 tile grid
    need_gpu()
    M, K, N = 300, 512, 272
    assert w4.w4a4_gemm_plan(M, K, N) == "pingpong"
    codes, sa, wp, sw, _ = _operands(M, K, N, "f32", sw_dt, bias=False, seed=7)
    rng = np.random.default_rng(8)
    b = workloads.f32_to_storage(rng.normal(0, 0.1, size=N), b_dt) if b_dt else None
    for odt, tdt in (("bf16", torch.bfloat16), ("f32", torch.float32)):
        out = w4.w4a4_gemm_from_codes(dev(codes), dev(sa), dev(wp), dev(sw, sw_dt),
                                      bias=dev(b, b_dt) if b_dt else None, out_dtype=tdt)
        oout = oracle.epilogue(oracle.gemm(codes, oracle.unpack(wp, K)), sa, sw, sw_dt, odt, bias=b,
                               bias_dtype=b_dt)
        assert np.array_equal(bits(host(out)), bits(oout)), (odt, sw_dt, b_dt)


SKINNY = [  # (M, K, N): decode-sized M takes the skinny kernel (K % 64 == 0)
    (1, 64, 16), (16, 192, 200), (17, 3840, 384), (32, 3840, 3840), (33, 640, 129), (64, 4096, 272),
    (48, 128, 1),
]


@pytest.mark.parametrize("M,K,N", SKINNY)
@pytest.mark.parametrize("odt", ["f32", "bf16", "f16"])
def test_skinny_m_bit_exact(M, K, N, odt):
    # one workgroup per 16 columns, K steps split over 16 waves and summed in
    # LDS: the INT32 sums and the outputs must still be the oracle's exactly
    need_gpu()
    codes, sa, wp, sw, b = _operands(M, K, N, odt, "bf16", seed=M * 3 + K + N)
    out, acc = w4.w4a4_gemm_from_codes(dev(codes), dev(sa), dev(wp), dev(sw, "bf16"), bias=dev(b, odt),
                                       out_dtype={"f32": torch.float32, "f16": torch.float16,
                                                  "bf16": torch.bfloat16}[odt], return_acc=True)
    oacc = oracle.gemm(codes, oracle.unpack(wp, K))
    assert np.array_equal(host(acc).astype(np.int64), oacc)
    oout = oracle.epilogue(oacc, sa, sw, "bf16", odt, bias=b, bias_dtype=odt)
    assert np.array_equal(bits(host(out)), bits(oout))
    # without the INT32 export and without bias
    out2 = w4.w4a4_gemm_from_codes(dev(codes), dev(sa), dev(wp), dev(sw, "bf16"),
                                   out_dtype={"f32": torch.float32, "f16": torch.float16,
                                              "bf16": torch.bfloat16}[odt])
    oout2 = oracle.epilogue(oacc, sa, sw, "bf16", odt)
    assert np.array_equal(bits(host(out2)), bits(oout2))


def test_skinny_m_with_lowrank_term():
    need_gpu()
    M, K, N, R = 24, 1024, 96, 32
    codes, sa, wp, sw, _ = _operands(M, K, N, "bf16", "bf16", bias=False, seed=8)
    rng = np.random.default_rng(9)
    L = rng.standard_normal((M, R)).astype(np.float32)
    up = workloads.f32_to_storage(rng.normal(0, 0.1, size=(N, R)), "bf16")
    oacc = oracle.gemm(codes, oracle.unpack(wp, K))
    out = w4.w4a4_gemm_from_codes(dev(codes), dev(sa), dev(wp), dev(sw, "bf16"),
                                  lora_act=dev(L), proj_up=dev(up, "bf16"), out_dtype=torch.bfloat16)
    oout = oracle.epilogue(oacc, sa, sw, "bf16", "bf16", L=L, proj_up=up, up_dtype="bf16")
    assert ulp_distance(host(out), oout, "bf16").max() <= 1


def test_skinny_m_equals_large_m_rows():
    # the first rows of a large-M GEMM (256 x 256 tiles) and the same rows
    # alone (skinny kernel) are the same bits
    need_gpu()
    M, K, N = 512, 3840, 384
    codes, sa, wp, sw, b = _operands(M, K, N, "bf16", "bf16", seed=21)
    big = w4.w4a4_gemm_from_codes(dev(codes), dev(sa), dev(wp), dev(sw, "bf16"), bias=dev(b, "bf16"))
    small = w4.w4a4_gemm_from_codes(dev(codes[:40]), dev(sa[:40]), dev(wp), dev(sw, "bf16"),
                                    bias=dev(b, "bf16"))
    assert torch.equal(big[:40].view(torch.int16), small.view(torch.int16))


def _full_range_weights(rng, N, K):
    """Packed weights over all 16 nibble patterns, -8 (0x8) included."""
    w = rng.integers(-8, 8, size=(N, K)).astype(np.int8)
    w[:, ::7] = -8
    return w, oracle.pack(w)


@pytest.mark.parametrize("M,K,N,kernel", [
    (300, 1024, 260, "ring3"), (4100, 256, 300, "ring3"), (300, 1024, 272, "pingpong"),
    (4100, 256, 304, "pingpong"),
    (100, 192, 130, "tile128"), (77, 1024, 40, "tile128"),
    (32, 3840, 384, "skinny"), (5, 160, 17, "tile128")])
def test_minus_eight_nibble_every_kernel(M, K, N, kernel):
    need_gpu()
    assert w4.w4a4_gemm_plan(M, K, N) == kernel
    rng = np.random.default_rng(M + N)
    codes = rng.integers(-7, 8, size=(M, K)).astype(np.int8)
    wq, wp = _full_range_weights(rng, N, K)
    sa = rng.uniform(0.01, 0.5, size=M).astype(np.float32)
    sw = workloads.f32_to_storage(rng.uniform(0.005, 0.02, size=N), "bf16")
    out = w4.w4a4_gemm_from_codes(dev(codes), dev(sa), dev(wp), dev(sw, "bf16"),
                                  out_dtype=torch.float32)
    oacc = oracle.gemm(codes, wq)
    assert np.array_equal(bits(host(out)), bits(oracle.epilogue(oacc, sa, sw, "bf16", "f32")))
    # per-64-group scales (the 128 x 128 kernel's group loop)
    if K % 64 == 0:
        swg = workloads.f32_to_storage(rng.uniform(0.005, 0.02, size=(K // 64, N)), "bf16")
        assert w4.w4a4_gemm_plan(M, K, N, 64) == "tile128"
        outg = w4.w4a4_gemm_from_codes(dev(codes), dev(sa), dev(wp), dev(swg, "bf16"), w_scale_group=64,
                                       out_dtype=torch.float32)
        parts = oracle.gemm(codes, wq, group=64)
        assert np.array_equal(bits(host(outg)), bits(oracle.epilogue(parts, sa, swg, "bf16", "f32",
                                                                     group=64)))


@pytest.mark.parametrize("N,kernel", [(256, "pingpong"), (264, "ring3")])
def test_extreme_codes_ring_kernel(N, kernel):
    # +-7 codes against -8 / 7 weights at K = 16384 through the persistent
    # kernels (no INT32 export there): unit scales and fp32 output give
    # f32(acc), exact below 2^24
    need_gpu()
    M, K = 512, 16384
    assert w4.w4a4_gemm_plan(M, K, N) == kernel
    codes = np.full((M, K), 7, dtype=np.int8)
    codes[1::2] = -7
    codes[2::5, ::3] = 0
    wq = np.full((N, K), -8, dtype=np.int8)
    wq[::3] = 7
    wp = oracle.pack(wq)
    out = w4.w4a4_gemm_from_codes(dev(codes), dev(np.ones(M, np.float32)), dev(wp),
                                  dev(np.ones(N, np.float32)), out_dtype=torch.float32)
    oacc = oracle.gemm(codes, wq)
    assert np.abs(oacc).max() == 56 * K
    assert np.array_equal(host(out), oacc.astype(np.float32))
