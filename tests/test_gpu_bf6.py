"""GPU parity of the FP6 GEMM path ("[Feat][Ascend] Consolidate INT8,
RotateQuant, RoPE and ConvRot W4A4 backends", "W4A4 correctness and
performance scope": the exact integer accumulation of the same codes and
weights, here on gfx950's f8f6f4 matrix cores with bf6 operands).

* the encoders: the GPU's bf6 blocks decode (host decoder from the format's
  definition, pinned in test_bf6_format) to the int8 codes / the unpacked INT4
  weights, pad bytes zero;
* the GEMM: bit-exact against the oracle's integer GEMM and epilogue, and
  bit-identical to the INT8 path, on ragged shapes, several tiles per
  workgroup, the smallest K and a K near the exact-accumulation limit with
  the extreme products;
* the linear at full prefill size: bit-identical to w4a4_linear."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.bf6 import decode_blocks
from tests.gpu_util import bits, dev, host, need_gpu

pytestmark = pytest.mark.gpu

import bit_quantized_linear_rotate_amd as w4  # noqa: E402


def test_encoders_decode_to_the_integers():
    need_gpu()
    rng = np.random.default_rng(81)
    codes = rng.integers(-8, 9, size=(67, 640)).astype(np.int8)
    c6 = host(w4.w4a4_codes_to_bf6(dev(codes)))
    vals, pad = decode_blocks(c6)
    assert np.array_equal(vals, codes.astype(np.float64)) and not pad.any()
    wq = rng.integers(-8, 8, size=(33, 640)).astype(np.int8)
    w6 = host(w4.w4a4_pack_weights_bf6(dev(oracle.pack(wq))))
    vals, pad = decode_blocks(w6)
    assert np.array_equal(vals, wq.astype(np.float64)) and not pad.any()


def _gemm_case(M, K, N, odt, rng, extreme=False):
    codes = rng.integers(-7, 8, size=(M, K)).astype(np.int8)
    wq = rng.integers(-8, 8, size=(N, K)).astype(np.int8)
    if extreme:
        codes[0] = -7
        wq[0] = -8
        codes[1] = 7
        wq[1] = 7
    sa = rng.uniform(0.001, 0.1, size=M).astype(np.float32)
    sw = workloads.f32_to_storage(rng.uniform(0.001, 0.01, size=N).astype(np.float32), odt)
    b = workloads.f32_to_storage(rng.normal(0, 0.1, size=N).astype(np.float32), odt)
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[odt]
    cd, wpd = dev(codes), dev(oracle.pack(wq))
    out6 = w4.w4a4_gemm_bf6(w4.w4a4_codes_to_bf6(cd), dev(sa), w4.w4a4_pack_weights_bf6(wpd), dev(sw, odt),
                            bias=dev(b, odt), out_dtype=tdt)
    out8 = w4.w4a4_gemm_from_codes(cd, dev(sa), wpd, dev(sw, odt), bias=dev(b, odt), out_dtype=tdt)
    assert torch.equal(out6.view(torch.uint8), out8.view(torch.uint8)), "FP6 and INT8 paths differ"
    return codes, wq, sa, sw, b, host(out6)


@pytest.mark.parametrize("M,K,N", [(300, 2048, 520), (513, 1024, 257), (64, 256, 64), (1000, 640, 1000),
                                   (2560, 384, 2304)])
@pytest.mark.parametrize("odt", ["bf16", "f16", "f32"])
def test_gemm_bf6_bit_exact(M, K, N, odt):
    need_gpu()
    rng = np.random.default_rng(M + K + N)
    codes, wq, sa, sw, b, out = _gemm_case(M, K, N, odt, rng, extreme=True)
    ref = oracle.epilogue(oracle.gemm(codes, wq), sa, sw, odt, odt, bias=b, bias_dtype=odt)
    assert np.array_equal(bits(out), bits(ref))


def test_gemm_bf6_near_the_exact_accumulation_limit():
    # 56 K just below 2^24: the extreme rows' sums reach 16.7 million and stay exact
    need_gpu()
    rng = np.random.default_rng(82)
    M, K, N = 256, 299520, 128
    codes, wq, sa, sw, b, out = _gemm_case(M, K, N, "f32", rng, extreme=True)
    rows = np.array([0, 1, 2, 255])
    acc = oracle.gemm(codes[rows], wq)
    assert acc[0, 0] == 56 * K and acc[0, 0] < 2 ** 24
    ref = oracle.epilogue(acc, sa[rows], sw, "f32", "f32", bias=b, bias_dtype="f32")
    assert np.array_equal(bits(out[rows]), bits(ref))


def test_gemm_bf6_rejects_unsupported_shapes():
    need_gpu()
    c6 = torch.zeros((64, 192), dtype=torch.uint8, device="cuda")
    w6 = torch.zeros((64, 192), dtype=torch.uint8, device="cuda")
    with pytest.raises(NotImplementedError):
        w4.w4a4_gemm_bf6(c6, torch.ones(64, device="cuda"), w6, torch.ones(64, device="cuda"))


def test_linear_bf6_full_prefill_equals_int8_path():
    need_gpu()
    w = workloads.WORKLOADS["prefill"]
    inp = workloads.generate(w)
    x = dev(inp["x"], w.dtype)
    rot = torch.from_numpy(inp["rot"].astype(np.float32)).cuda()
    wp = dev(inp["w_packed"])
    sw = dev(inp["s_w"], w.sw_dtype)
    out6 = w4.w4a4_linear_bf6(x, rot, w.g, w4.w4a4_pack_weights_bf6(wp), sw)
    out8 = w4.w4a4_linear(x, rot, w.g, wp, sw)
    assert torch.equal(out6.view(torch.int16), out8.view(torch.int16))
    rows = np.array([0, 17, 4095, 8191])
    ref = oracle.linear(inp, w.dtype, w.g, w.sw_dtype, w.sw_group, rows=rows)
    go = host(out6)[rows]
    codes, scales = w4.w4a4_rotate_quant_rowwise(x, rot, w.g)
    same = (host(codes)[rows] == ref["codes"]).all(axis=1) & (host(scales)[rows] == ref["scales"])
    assert np.array_equal(bits(go[same]), bits(ref["out"][same])) and same.sum() >= 2
