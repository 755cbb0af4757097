"""GPU parity of the INT8 mode (qmax = 127) and the dynamic INT8 linear
against the oracle ("[Feat][Ascend] Add fused RotateQuant backend", "What this
PR does / why we need it"; the shapes of its "Performance and memory" table).

* rotate-quant: the oracle's quantizer on the GPU's exported rotated values
  reproduces codes and scales bit for bit, the rotated values are within the
  rotation tolerance, and end to end every row's codes are within one of the
  oracle's (equal on rows with the oracle's scale), through every kernel the
  INT8 mode takes (row, g = 256, generic), with the edge rows planted;
* the INT8-weight GEMM: exact INT32 sums through the epilogue, bit-exact, on
  aligned and ragged shapes and on the INT64 K-chunk path;
* the linear: bit-exact against the oracle's epilogue on the GPU's own codes,
  and on every row whose codes match the oracle's."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.gpu_util import bits, dev, host, need_gpu, rotated_close
from tests.test_gpu_edge_rows import build_matrix, scales_equal

pytestmark = pytest.mark.gpu

import bit_quantized_linear_rotate_amd as w4  # noqa: E402

Q = 127


def _rq_case(dt, x_host, x_dev, R, g, kernel, smooth=None):
    rot = torch.from_numpy(np.ascontiguousarray(R, dtype=np.float32)).cuda()
    sm_dev = dev(smooth, dt) if smooth is not None else None
    assert w4.w8a8_rotate_quant_plan(x_dev, rot, g, smooth=sm_dev) == kernel
    c, s, yg = w4.w8a8_rotate_quant_rowwise(x_dev, rot, g, smooth=sm_dev, return_rotated=True)
    c2, s2 = w4.w8a8_rotate_quant_rowwise(x_dev, rot, g, smooth=sm_dev)
    c, s, yg, c2, s2 = host(c), host(s), host(yg), host(c2), host(s2)
    assert np.array_equal(c, c2) and scales_equal(s, s2)
    assert c.min() >= -Q
    oc, os_ = oracle.quantize(yg, dt, qmax=Q)
    assert np.array_equal(c, oc), "codes differ from the oracle quantizer on the GPU's rotated values"
    assert scales_equal(s, os_), "scales differ from the oracle quantizer on the GPU's rotated values"
    xs = oracle.smooth(x_host, smooth, dt) if smooth is not None else x_host
    yo = oracle.rotate(xs, R, g, dt)
    frac, beyond = rotated_close(yg, yo, xs, R, g, dt)
    _, rc, rs = oracle.rotate_quant(x_host, R, g, dt, smooth, qmax=Q)
    M = x_host.shape[0]
    same = np.array([scales_equal(s[i:i + 1], rs[i:i + 1]) for i in range(M)])
    dc = np.abs(c.astype(np.int32) - rc)
    assert dc.max(initial=0) <= 1
    eq = (dc == 0).all(axis=1)
    print(f"INT8 {kernel} {dt} M={M} K={x_host.shape[1]} g={g}: {frac:.2e} rotated values differ "
          f"({beyond} beyond 1 ulp), {(~same).sum()} rows with another scale, "
          f"{(dc > 0).sum()} code flips, {(~eq).sum()} rows not identical")
    return c, s


@pytest.mark.parametrize("dt", ["bf16", "f16"])
def test_int8_row_kernel_edge_rows(dt):
    need_gpu()
    M, K, g = 2048, 3840, 64
    x, where = build_matrix(dt, M, K, g, seed=51)
    R = workloads.asymmetric_rotation(g, seed=5)
    c, s = _rq_case(dt, x, dev(x, dt), R, g, "row")
    assert (c[where["zero"]] == 0).all() and s[where["zero"]] == np.float32(2.0 ** -126)
    assert np.isnan(s[where["nan"]]) and (c[where["nan"]] == 0).all()


@pytest.mark.parametrize("dt", ["bf16", "f16"])
@pytest.mark.parametrize("smoothing", [False, True])
def test_int8_g256_kernel_edge_rows(dt, smoothing):
    need_gpu()
    M, K, g = 96, 4096, 256
    x, where = build_matrix(dt, M, K, g, seed=52)
    R = workloads.asymmetric_rotation(g, seed=6)
    sm = None
    if smoothing:
        sm = workloads.f32_to_storage(np.random.default_rng(7).uniform(0.5, 2.0, size=K), dt)
    _rq_case(dt, x, dev(x, dt), R, g, "g256", smooth=sm)


@pytest.mark.parametrize("dt,g,transposed", [("f32", 16, False), ("bf16", 64, True), ("f16", 128, False)])
def test_int8_generic_kernel(dt, g, transposed):
    need_gpu()
    M, K = 40, 512
    rng = np.random.default_rng(53)
    x = workloads.f32_to_storage(rng.standard_t(4, size=(M, K)).astype(np.float32), dt)
    R = workloads.asymmetric_rotation(g, seed=8)
    if transposed:
        xd = dev(np.ascontiguousarray(x.T), dt).t()
    else:
        xd = dev(x, dt)
    _rq_case(dt, x, xd, R, g, "generic")


def test_int8_exact_ties_half_even():
    # a row whose absmax is 127 * 2^e: s = 2^e exactly, so every k + 1/2 entry
    # is a tie the quotient meets exactly; the row kernel must round it to even
    need_gpu()
    M, K, g = 2048, 3840, 64
    rng = np.random.default_rng(54)
    x = workloads.f32_to_storage(rng.standard_t(4, size=(M, K)).astype(np.float32), "bf16")
    R = np.eye(g)
    vals = np.zeros(K, np.float32)
    vals[0] = 127.0
    vals[1:64] = np.arange(63) + 0.5
    vals[64:127] = -(np.arange(63) + 0.5)
    x[7] = workloads.f32_to_storage(vals / 4.0, "bf16")
    c, s = _rq_case("bf16", x, dev(x, "bf16"), R, g, "row")
    assert s[7] == np.float32(0.25)
    k = np.arange(63)
    assert np.array_equal(c[7, 1:64], (k + 1) // 2 * 2)        # half to even
    assert np.array_equal(c[7, 64:127], -((k + 1) // 2 * 2))


@pytest.mark.parametrize("M,K,N,kernel", [(300, 2048, 520, "ring3"), (513, 1024, 257, "ring3"),
                                          (260, 192, 300, "ring3"), (1000, 640, 1000, "ring3"),
                                          (64, 256, 64, "tile128"), (5, 96, 17, "tile128"),
                                          (200, 100, 40, "tile128")])
@pytest.mark.parametrize("odt", ["bf16", "f16", "f32"])
def test_int8_gemm_bit_exact(M, K, N, kernel, odt):
    need_gpu()
    assert w4.w8a8_gemm_plan(M, K, N) == kernel
    rng = np.random.default_rng(M + K + N)
    codes = rng.integers(-127, 128, size=(M, K)).astype(np.int8)
    w = rng.integers(-128, 128, size=(N, K)).astype(np.int8)
    w[0] = -128
    codes[0] = 127
    sa = rng.uniform(0.001, 0.1, size=M).astype(np.float32)
    sw = workloads.f32_to_storage(rng.uniform(0.001, 0.01, size=N).astype(np.float32), odt)
    b = workloads.f32_to_storage(rng.normal(0, 0.1, size=N).astype(np.float32), odt)
    out = w4.w8a8_gemm_from_codes(dev(codes), dev(sa), dev(w), dev(sw, odt), bias=dev(b, odt),
                                  out_dtype={"f32": torch.float32, "f16": torch.float16,
                                             "bf16": torch.bfloat16}[odt])
    acc = oracle.gemm(codes, w)
    ref = oracle.epilogue(acc, sa, sw, odt, odt, bias=b, bias_dtype=odt)
    assert np.array_equal(bits(host(out)), bits(ref))


@pytest.mark.parametrize("odt", ["bf16", "f32"])
def test_int8_gemm_ring3_many_tiles(odt):
    # more 256 x 256 tiles than workgroups (each walks several, the operand
    # ring running across them), ragged in M and N; sampled rows, every column
    need_gpu()
    M, K, N = 4500, 256, 3900
    assert w4.w8a8_gemm_plan(M, K, N) == "ring3"
    rng = np.random.default_rng(57)
    codes = rng.integers(-127, 128, size=(M, K)).astype(np.int8)
    w = rng.integers(-128, 128, size=(N, K)).astype(np.int8)
    sa = rng.uniform(0.001, 0.1, size=M).astype(np.float32)
    sw = workloads.f32_to_storage(rng.uniform(0.001, 0.01, size=N).astype(np.float32), odt)
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16}[odt]
    out = host(w4.w8a8_gemm_from_codes(dev(codes), dev(sa), dev(w), dev(sw, odt), out_dtype=tdt))
    rows = np.unique(np.concatenate([np.arange(4352, M), rng.choice(M, 150, replace=False), [0, 255, 256]]))
    ref = oracle.epilogue(oracle.gemm(codes[rows], w), sa[rows], sw, odt, odt)
    assert np.array_equal(bits(out[rows]), bits(ref))


def test_int8_gemm_int64_chunks():
    # K past the INT32-safe length: the sums are taken in K-chunks and combined
    # exactly in int64; the extreme products make the INT32 range matter
    need_gpu()
    M, K, N = 8, 132160, 16
    assert w4.w8a8_gemm_workspace_size(M, N, K) > 0
    rng = np.random.default_rng(55)
    codes = np.full((M, K), 127, np.int8)
    codes[1:] = rng.integers(-127, 128, size=(M - 1, K))
    w = np.full((N, K), -128, np.int8)
    w[1:] = rng.integers(-128, 128, size=(N - 1, K))
    sa = np.ones(M, np.float32)
    sw = np.ones(N, np.float32)
    out = w4.w8a8_gemm_from_codes(dev(codes), dev(sa), dev(w), dev(sw), out_dtype=torch.float32)
    acc = oracle.gemm(codes, w)
    assert acc[0, 0] == -127 * 128 * K and abs(int(acc[0, 0])) > 2 ** 31
    ref = oracle.epilogue(acc, sa, sw, "f32", "f32")
    assert np.array_equal(bits(host(out)), bits(ref))


def _linear_case(dt, x, R, g, w, sw, b, rows, cols, kernel, transposed=False):
    xd = dev(np.ascontiguousarray(x.T), dt).t() if transposed else dev(x, dt)
    rot = torch.from_numpy(np.ascontiguousarray(R, dtype=np.float32)).cuda()
    assert w4.w8a8_rotate_quant_plan(xd, rot, g) == kernel
    out = w4.w8a8_linear(xd, rot, g, dev(w), dev(sw, dt), bias=dev(b, dt))
    c, s = w4.w8a8_rotate_quant_rowwise(xd, rot, g)
    torch.cuda.synchronize()
    gc, gs = host(c), host(s)
    # codes and scales of the sampled rows: within one of the oracle's
    _, rc, rs = oracle.rotate_quant(x[rows], R, g, dt, qmax=Q)
    dc = np.abs(gc[rows].astype(np.int32) - rc)
    assert dc.max(initial=0) <= 1
    same = np.array([scales_equal(gs[i:i + 1], rs[k:k + 1]) for k, i in enumerate(rows)])
    # the output: the oracle's epilogue on the GPU's own codes, and the
    # oracle's output on rows whose codes match
    go = host(out)[np.ix_(rows, cols)]
    acc = oracle.gemm(gc[rows], w[cols])
    own = oracle.epilogue(acc, gs[rows], sw[cols], dt, dt, bias=b[cols], bias_dtype=dt)
    assert np.array_equal(bits(go), bits(own))
    ref = oracle.linear_int8(x, R, g, w, sw, dt, dt, bias=b, rows=rows, cols=cols)
    exact = same & (dc.max(axis=1) == 0)
    assert np.array_equal(bits(go[exact]), bits(ref["out"][exact]))
    assert exact.sum() >= len(rows) // 4
    print(f"INT8 linear {dt} M={x.shape[0]} K={x.shape[1]} N={w.shape[0]} g={g}: rows with another "
          f"scale {(~same).sum()}, code flips {(dc > 0).sum()}, output rows {len(rows)} x {len(cols)}, "
          f"exact rows {int(exact.sum())}")


@pytest.mark.parametrize("M,K,N,g,dt,kernel", [(2304, 3840, 256, 64, "bf16", "row"),
                                                (96, 10240, 200, 256, "f16", "g256"),
                                                (48, 3840, 130, 64, "bf16", "generic")])
def test_int8_linear_reduced(M, K, N, g, dt, kernel):
    need_gpu()
    rng = np.random.default_rng(M + N)
    x = workloads.f32_to_storage(rng.standard_t(4, size=(M, K)).astype(np.float32), dt)
    w = rng.integers(-127, 128, size=(N, K)).astype(np.int8)
    sw = workloads.f32_to_storage(rng.uniform(0.0005, 0.002, size=N).astype(np.float32), dt)
    b = workloads.f32_to_storage(rng.normal(0, 0.1, size=N).astype(np.float32), dt)
    rows = np.arange(M) if M <= 400 else np.sort(rng.choice(M, 300, replace=False))
    _linear_case(dt, x, workloads.hadamard(g), g, w, sw, b, rows, np.arange(N), kernel)


@pytest.mark.parametrize("name,K,g,kernel", [("prefill", 3840, 64, "row"), ("widek", 10240, 256, "g256")])
def test_int8_linear_full_size(name, K, g, kernel):
    # the shapes of the RotateQuant page's timing table, [8192, 3840] and
    # [8192, 10240], with the config's activations (contiguous rows)
    need_gpu()
    wl = workloads.WORKLOADS[name]
    inp = workloads.generate(wl)
    x = np.ascontiguousarray(inp["x"])
    assert x.shape == (8192, K)
    N = 3840
    rng = np.random.default_rng(56)
    w = rng.integers(-127, 128, size=(N, K)).astype(np.int8)
    sw = workloads.f32_to_storage(rng.uniform(0.0005, 0.002, size=N).astype(np.float32), wl.dtype)
    b = workloads.f32_to_storage(rng.normal(0, 0.1, size=N).astype(np.float32), wl.dtype)
    rows = np.unique(np.concatenate([[0, 8191], rng.choice(8192, 62, replace=False)]))
    cols = np.unique(np.concatenate([[0, N - 1], rng.choice(N, 254, replace=False)]))
    _linear_case(wl.dtype, x, workloads.hadamard(g), g, w, sw, b, rows, cols, kernel)
