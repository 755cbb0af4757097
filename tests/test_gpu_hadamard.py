"""GPU parity of the structured-rotation path (fast Walsh-Hadamard transform;
at g = 64 on many contiguous rows, the row-streaming kernel with R built
in-kernel) against the oracle with the same rotation written out as a dense R.

The rotation is R = diag(sign_in) . H_g . diag(sign_out) / sqrt(g) (group
sizes and asymmetric rotations of "[Feat][Ascend] Add fused RotateQuant
backend", section "How was this patch tested?"); with random signs on both
sides R is not symmetric, so a transposed R would fail.  The kernel sums the
same exact products as the dense kernels in another order, so the parity rule
is the dense kernels' own:
  * the oracle's quantizer on the GPU's exported rotated values gives the
    GPU's codes and scales bit for bit (both code ranges);
  * those rotated values are within one ulp of T of the oracle's rotation, or
    within the fp32 summation bound; NaN where it has NaN;
  * end to end, codes within 1 of the oracle's; rows with another scale are
    explained by the rotated row (first point);
  * the whole layer (w4a4_linear_hadamard, w8a8_linear_hadamard) at reduced
    and full size through the same checks as the dense layer.
Edge rows (zeros, NaN, Inf, tiny, max-finite, exact ties) are planted among
ordinary ones, and shapes include a partial last 512-element chunk."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.gpu_util import bits, dev, host, need_gpu, rotated_close
from tests.test_gpu_edge_rows import build_matrix, scales_equal

pytestmark = pytest.mark.gpu

import bit_quantized_linear_rotate_amd as w4  # noqa: E402


def _signs(g, seed):
    if seed is None:
        return None, None
    rng = np.random.default_rng(seed)
    si = rng.choice(np.array([-1, 1], np.int8), size=g)
    so = rng.choice(np.array([-1, 1], np.int8), size=g)
    return si, so


def _dense(g, si, so):
    h = workloads.hadamard(g)
    if si is not None:
        h = si.astype(np.float64)[:, None] * h
    if so is not None:
        h = h * so.astype(np.float64)[None, :]
    return h


def _hadamard(g, si, so):
    return w4.Hadamard(g, None if si is None else torch.from_numpy(si).cuda(),
                       None if so is None else torch.from_numpy(so).cuda())


def _rq_case(dt, x, g, si, so, qmax, smooth=None, x_dev=None, plan="hadamard"):
    h = _hadamard(g, si, so)
    R = _dense(g, si, so)
    # the binding's dense form is the same matrix
    assert np.array_equal(h.dense().cpu().numpy(), R.astype(np.float32))
    xd = dev(x, dt) if x_dev is None else x_dev
    sm = dev(smooth, dt) if smooth is not None else None
    assert w4.w4a4_rotate_quant_hadamard_plan(xd, g, qmax, smooth=sm, return_rotated=True) == plan
    c, s, yg = w4.w4a4_rotate_quant_hadamard(xd, h, qmax, smooth=sm, return_rotated=True)
    c2, s2 = w4.w4a4_rotate_quant_hadamard(xd, h, qmax, smooth=sm)
    c, s, yg, c2, s2 = host(c), host(s), host(yg), host(c2), host(s2)
    assert np.array_equal(c, c2) and scales_equal(s, s2)
    oc, os_ = oracle.quantize(yg, dt, qmax=qmax)
    assert np.array_equal(c, oc), "codes differ from the oracle quantizer on the GPU's rotated values"
    assert scales_equal(s, os_), "scales differ from the oracle quantizer on the GPU's rotated values"
    xs = oracle.smooth(x, smooth, dt) if smooth is not None else x
    yo = oracle.rotate(xs, R, g, dt)
    frac, beyond = rotated_close(yg, yo, xs, R, g, dt)
    _, rc, rs = oracle.rotate_quant(x, R, g, dt, smooth, qmax=qmax)
    M = x.shape[0]
    same = np.array([scales_equal(s[i:i + 1], rs[i:i + 1]) for i in range(M)])
    dc = np.abs(c.astype(np.int32) - rc)
    assert dc.max(initial=0) <= 1
    print(f"{plan} g={g} {dt} qmax={qmax} M={M} K={x.shape[1]} signs={si is not None}: "
          f"{frac:.2e} rotated values differ ({beyond} beyond 1 ulp), {(~same).sum()} rows with "
          f"another scale, {(dc > 0).sum()} code flips")
    return c, s


@pytest.mark.parametrize("g", [16, 32, 64, 128, 256])
@pytest.mark.parametrize("dt", ["bf16", "f16"])
@pytest.mark.parametrize("qmax", [7, 127])
def test_hadamard_all_group_sizes(g, dt, qmax):
    need_gpu()
    M, K = 64, 4096
    x, where = build_matrix(dt, M, K, g, seed=61 + g)
    si, so = _signs(g, seed=g)
    c, s = _rq_case(dt, x, g, si, so, qmax)
    assert (c[where["zero"]] == 0).all() and s[where["zero"]] == np.float32(2.0 ** -126)
    assert np.isnan(s[where["nan"]]) and (c[where["nan"]] == 0).all()


@pytest.mark.parametrize("g,K", [(256, 2304), (16, 1040), (64, 3840), (32, 96), (256, 16384)])
@pytest.mark.parametrize("signs", [None, 5])
def test_hadamard_partial_chunks_and_widths(g, K, signs):
    # K not a multiple of 512 (a partial last chunk; for g = 16 half of a
    # 32-element piece), the smallest widths and the largest supported one
    need_gpu()
    rng = np.random.default_rng(K + g)
    M = 40
    x = workloads.f32_to_storage(rng.standard_t(4, size=(M, K)).astype(np.float32), "bf16")
    si, so = _signs(g, signs)
    _rq_case("bf16", x, g, si, so, 7)


@pytest.mark.parametrize("dt", ["bf16", "f16"])
def test_hadamard_smoothing_and_strided_rows(dt):
    # smoothing (the low-rank layer's activations) and a row stride larger
    # than K (a view of every other 4096-wide block)
    need_gpu()
    g, M, K = 256, 48, 4096
    rng = np.random.default_rng(62)
    big = workloads.f32_to_storage(rng.standard_normal((M, 2 * K)).astype(np.float32), dt)
    x = np.ascontiguousarray(big[:, :K])
    xd = dev(big, dt)[:, :K]
    sm = workloads.f32_to_storage(rng.uniform(0.5, 2.0, size=K).astype(np.float32), dt)
    si, so = _signs(g, 7)
    _rq_case(dt, x, g, si, so, 7, smooth=sm, x_dev=xd)
    _rq_case(dt, x, g, si, so, 127, smooth=sm, x_dev=xd)


@pytest.mark.parametrize("dt,K", [("bf16", 4096), ("f16", 1152)])
@pytest.mark.parametrize("qmax", [7, 127])
@pytest.mark.parametrize("signs", [None, 11])
def test_hadamard_g64_row_kernel(dt, K, qmax, signs):
    # g = 64 on many contiguous rows: the row-streaming kernel, which builds
    # the fragments of diag(sign_in) H_64 diag(sign_out) / 8 itself.  The
    # oracle's checks, and bit-identity with the same kernel given that R as
    # a dense matrix (the same fp32 products, summed in the same order)
    need_gpu()
    g, M = 64, 2048
    x, where = build_matrix(dt, M, K, g, seed=65 + K + qmax)
    si, so = _signs(g, signs)
    sm = None
    if signs is not None:
        sm = workloads.f32_to_storage(np.random.default_rng(66).uniform(0.5, 2.0, size=K).astype(np.float32), dt)
    c, s = _rq_case(dt, x, g, si, so, qmax, smooth=sm, plan="row")
    xd = dev(x, dt)
    smd = dev(sm, dt) if sm is not None else None
    R = torch.from_numpy(_dense(g, si, so).astype(np.float32)).cuda()
    c1, s1, y1 = w4.w4a4_rotate_quant_hadamard(xd, _hadamard(g, si, so), qmax, smooth=smd, return_rotated=True)
    if qmax == 7:
        assert w4.w4a4_rotate_quant_plan(xd, R, g, smooth=smd) == "row"
        c2, s2, y2 = w4.w4a4_rotate_quant_rowwise(xd, R, g, smooth=smd, return_rotated=True)
    else:
        c2, s2, y2 = w4.w8a8_rotate_quant_rowwise(xd, R, g, smooth=smd, return_rotated=True)
    assert torch.equal(c1, c2) and torch.equal(s1.view(torch.int32), s2.view(torch.int32))
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
    assert (c[where["zero"]] == 0).all() and s[where["zero"]] == np.float32(2.0 ** -126)
    assert np.isnan(s[where["nan"]]) and (c[where["nan"]] == 0).all()


def test_hadamard_unsupported_layouts_are_refused():
    need_gpu()
    h = w4.Hadamard(256)
    x = torch.zeros((64, 4096), dtype=torch.bfloat16, device="cuda")
    # unsupported layouts (W4A4_UNSUPPORTED), then an invalid code range
    with pytest.raises(NotImplementedError):
        w4.w4a4_rotate_quant_hadamard(x.t().contiguous().t(), h)       # column-major view
    with pytest.raises(NotImplementedError):
        w4.w4a4_rotate_quant_hadamard(x.float(), h)                     # fp32
    with pytest.raises(NotImplementedError):
        w4.w4a4_rotate_quant_hadamard(torch.zeros((4, 16640), dtype=torch.bfloat16, device="cuda"), h)
    with pytest.raises(ValueError):
        w4.w4a4_rotate_quant_hadamard(x, h, qmax=15)
    with pytest.raises(ValueError):
        w4.Hadamard(8)


def test_hadamard_matches_dense_kernel_codes_on_exact_rows():
    # with g = 16 and 16-bit inputs whose group sums are exact in fp32 (small
    # integers), both kernels compute the exact rotation: identical results
    need_gpu()
    g, M, K = 16, 64, 1024
    rng = np.random.default_rng(63)
    x = workloads.f32_to_storage(rng.integers(-64, 65, size=(M, K)).astype(np.float32), "bf16")
    xd = dev(x, "bf16")
    c1, s1, y1 = w4.w4a4_rotate_quant_hadamard(xd, w4.Hadamard(g), return_rotated=True)
    R = torch.from_numpy(workloads.hadamard(g).astype(np.float32)).cuda()
    c2, s2, y2 = w4.w4a4_rotate_quant_rowwise(xd, R, g, return_rotated=True)
    assert torch.equal(c1, c2) and torch.equal(s1.view(torch.int32), s2.view(torch.int32))
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))


# ---- the whole layer ----------------------------------------------------------

from tests.test_gpu_linear import _check, _device_inputs  # noqa: E402


def _run_h(w, d):
    h = w4.Hadamard(w.g)
    out = w4.w4a4_linear_hadamard(d["x"], h, d["w_packed"], d["w_scale"], w_scale_group=w.sw_group,
                                  bias=d["bias"], smooth=d["smooth"], proj_down=d["proj_down"],
                                  proj_up=d["proj_up"])
    codes, scales, y = w4.w4a4_rotate_quant_hadamard(d["x"], h, smooth=d["smooth"], return_rotated=True)
    L = w4.w4a4_lowrank_down(d["x"], d["proj_down"]) if d["proj_down"] is not None else None
    torch.cuda.synchronize()
    return out, codes, scales, y, L


@pytest.mark.parametrize("name,M,N", [("lowrank", 100, 200), ("prefill", 300, 256), ("widek", 96, 200)])
def test_hadamard_linear_reduced(name, M, N):
    need_gpu()
    w = dataclasses.replace(workloads.WORKLOADS[name].scaled(M=M, N=N), transposed=False)
    inp = workloads.generate(w)
    d = _device_inputs(w, inp)
    assert w4.w4a4_rotate_quant_hadamard_plan(d["x"], w.g, smooth=d["smooth"]) == "hadamard"
    out, codes, scales, y, L = _run_h(w, d)
    _check(w, inp, out, codes, scales, y, L, np.arange(w.M), np.arange(w.N), full=False)


@pytest.mark.parametrize("name", ["lowrank", "widek"])
def test_hadamard_linear_full_size(name):
    # the low-rank layer as configured; the wide-K shape with contiguous rows
    need_gpu()
    w = dataclasses.replace(workloads.WORKLOADS[name], transposed=False)
    inp = workloads.generate(w)
    d = _device_inputs(w, inp)
    out, codes, scales, y, L = _run_h(w, d)
    rng = np.random.default_rng(98)
    rows = np.unique(np.concatenate([[0, w.M - 1], rng.choice(w.M, 160, replace=False)]))
    cols = np.unique(np.concatenate([[0, w.N - 1], rng.choice(w.N, 300, replace=False)]))
    _check(w, inp, out, codes, scales, y, L, rows, cols, full=True)


def test_hadamard_int8_linear():
    need_gpu()
    dt, g, M, K, N = "f16", 256, 256, 10240, 200
    rng = np.random.default_rng(64)
    x = workloads.f32_to_storage(rng.standard_normal((M, K)).astype(np.float32), dt)
    w = rng.integers(-127, 128, size=(N, K)).astype(np.int8)
    sw = workloads.f32_to_storage(rng.uniform(0.0005, 0.002, size=N).astype(np.float32), dt)
    b = workloads.f32_to_storage(rng.normal(0, 0.1, size=N).astype(np.float32), dt)
    si, so = _signs(g, 9)
    h = _hadamard(g, si, so)
    xd = dev(x, dt)
    out = host(w4.w8a8_linear_hadamard(xd, h, dev(w), dev(sw, dt), bias=dev(b, dt)))
    gc, gs = (host(t) for t in w4.w4a4_rotate_quant_hadamard(xd, h, 127))
    R = _dense(g, si, so)
    _, rc, rs = oracle.rotate_quant(x, R, g, dt, qmax=127)
    dc = np.abs(gc.astype(np.int32) - rc)
    assert dc.max(initial=0) <= 1
    own = oracle.epilogue(oracle.gemm(gc, w), gs, sw, dt, dt, bias=b, bias_dtype=dt)
    assert np.array_equal(bits(out), bits(own))
    ref = oracle.linear_int8(x, R, g, w, sw, dt, dt, bias=b)
    exact = np.array([scales_equal(gs[i:i + 1], rs[i:i + 1]) for i in range(M)]) & (dc.max(axis=1) == 0)
    assert exact.sum() >= M // 2
    assert np.array_equal(bits(out[exact]), bits(ref["out"][exact]))
