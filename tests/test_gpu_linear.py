"""End-to-end GPU parity of the whole W4A4 linear on the five workloads.

For each workload, at a reduced size and at its full size, in the launch
configuration the benchmark times (the plan queries confirm the kernels):
  * codes and scales of EVERY row are compared with the oracle's.  A row
    whose scale differs is accepted only when the GPU's exported rotated row
    explains it: the oracle's quantizer, run on that row, reproduces the GPU's
    codes and scale bit for bit, and the rotated values are within one unit in
    the last place of the oracle's (or the fp32 summation bound).  Codes differ by at most 1 anywhere, and
    on at most 1e-4 of all entries (rows with another scale included);
  * the output (all entries at reduced size; 256 rows x 512 columns at full
    size, zero rows and rows with another scale among them) equals the
    oracle's epilogue applied to the GPU's own codes and scales bit for bit
    (within 1 ulp with the low-rank term), and rows whose codes and scales
    match the oracle's give the oracle's output.
The counts (rows with another scale, code flips) are printed per workload."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.gpu_util import TORCH_DT, bits, dev, host, need_gpu, rotated_close, ulp_distance

pytestmark = pytest.mark.gpu

import bit_quantized_linear_rotate_amd as w4  # noqa: E402

# kernels the benchmark's configuration of each workload takes
PLAN = {"tiny": ("generic", "skinny"), "decode": ("reg", "skinny"), "prefill": ("row", "pingpong"),
        "widek": ("colmajor", "pingpong"), "lowrank": ("g256", "tile128")}


def _device_inputs(w, inp):
    dt = w.dtype
    if w.transposed:
        x = dev(inp["x_buffer"], dt).t()
    else:
        x = dev(inp["x"], dt)
    return dict(
        x=x,
        rot=torch.from_numpy(inp["rot"].astype(np.float32)).cuda(),
        w_packed=dev(inp["w_packed"]),
        w_scale=dev(inp["s_w"], w.sw_dtype),
        bias=dev(inp["bias"], dt) if inp["bias"] is not None else None,
        smooth=dev(inp["smooth"], dt) if inp["smooth"] is not None else None,
        proj_down=dev(inp["proj_down"], dt) if inp["proj_down"] is not None else None,
        proj_up=dev(inp["proj_up"], dt) if inp["proj_up"] is not None else None,
    )


def _run_gpu(w, d):
    out = w4.w4a4_linear(d["x"], d["rot"], w.g, d["w_packed"], d["w_scale"],
                         w_scale_group=w.sw_group, bias=d["bias"], smooth=d["smooth"],
                         proj_down=d["proj_down"], proj_up=d["proj_up"])
    codes, scales = w4.w4a4_rotate_quant_rowwise(d["x"], d["rot"], w.g, smooth=d["smooth"])
    c2, s2, y = w4.w4a4_rotate_quant_rowwise(d["x"], d["rot"], w.g, smooth=d["smooth"],
                                             return_rotated=True)
    L = w4.w4a4_lowrank_down(d["x"], d["proj_down"]) if d["proj_down"] is not None else None
    torch.cuda.synchronize()
    assert torch.equal(codes, c2) and torch.equal(scales.view(torch.int32), s2.view(torch.int32))
    return out, codes, scales, y, L


def _scale_same(a, b):
    return (bits(a) == bits(b)) | (np.isnan(a) & np.isnan(b))


def _check(w, inp, out, codes, scales, y, L, gemm_rows, cols, full):
    dt = w.dtype
    M = w.M
    # --- rotate-quant, every row
    ref_y, ref_c, ref_s = oracle.rotate_quant(inp["x"], inp["rot"], w.g, dt, inp.get("smooth"))
    gc, gs, gy = host(codes), host(scales), host(y)
    same = _scale_same(gs, ref_s)
    other = np.flatnonzero(~same)
    if other.size:
        qc, qs = oracle.quantize(gy[other], dt)
        assert np.array_equal(qc, gc[other]), "a row with another scale is not the oracle " \
                                              "quantizer's result on the GPU's rotated row"
        assert np.array_equal(_scale_same(qs, gs[other]), np.ones(other.size, bool))
        xs = oracle.smooth(inp["x"], inp["smooth"], dt) if inp.get("smooth") is not None else inp["x"]
        rotated_close(gy[other], ref_y[other], xs[other], inp["rot"], w.g, dt)
    dc = np.abs(gc.astype(np.int32) - ref_c)
    assert dc.max(initial=0) <= 1
    flips = int((dc > 0).sum())
    assert flips <= 1e-4 * M * w.K, flips
    # --- GEMM + epilogue on sampled rows and columns
    lowrank = w.rank > 0
    rows = gemm_rows
    if full:
        # include rows with another scale and (wide-K) zero rows
        zero_rows = np.flatnonzero((gc == 0).all(axis=1))[:8]
        rows = np.unique(np.concatenate([rows, other[:16], zero_rows]))
    ref = oracle.linear(inp, dt, w.g, w.sw_dtype, w.sw_group, rows=rows, cols=cols)
    go = host(out)[np.ix_(rows, cols)]
    wq = oracle.unpack(inp["w_packed"][cols], w.K)
    acc = oracle.gemm(gc[rows], wq, w.sw_group)
    s_w = inp["s_w"][..., cols]
    bias = inp["bias"][cols] if inp["bias"] is not None else None
    up = inp["proj_up"][cols] if lowrank else None
    Lr = host(L)[rows] if lowrank else None
    own = oracle.epilogue(acc, gs[rows], s_w, w.sw_dtype, dt, bias=bias,
                          bias_dtype=dt if bias is not None else None, group=w.sw_group,
                          L=Lr, proj_up=up, up_dtype=dt if lowrank else None)
    exact_rows = same[rows] & (dc[rows].max(axis=1) == 0)
    if lowrank:
        assert ulp_distance(go, own, dt).max() <= 1
        assert ulp_distance(go[exact_rows], ref["out"][exact_rows], dt).max(initial=0) <= 1
    else:
        assert np.array_equal(bits(go), bits(own))
        assert np.array_equal(bits(go[exact_rows]), bits(ref["out"][exact_rows]))
    print(f"{w.name}: M={M} K={w.K} N={w.N}: rows with another scale {other.size}, "
          f"code flips {flips} ({flips / (M * w.K):.2e}), output rows compared {len(rows)} "
          f"x {len(cols)} cols, exact rows {int(exact_rows.sum())}")


def _plan_ok(w, d):
    rq, gm = PLAN[w.name.replace("-scaled", "")]
    assert w4.w4a4_rotate_quant_plan(d["x"], d["rot"], w.g, smooth=d["smooth"]) == rq
    if gm == "pingpong" and w.N % 16:
        gm = "ring3"   # the ping-pong kernel writes whole 16-column pieces
    assert w4.w4a4_gemm_plan(w.M, w.K, w.N, w.sw_group, lowrank=w.rank > 0) == gm


# reduced sizes: widek keeps M % 8 == 0 so that its transposed view takes the
# column-major kernel (and meets its zero rows); prefill keeps enough rows for
# the row-streaming kernel.  Prefill's N is a multiple of 16 (the ping-pong
# GEMM), widek's is not (the ring GEMM).
REDUCED = {"tiny": None, "decode": None, "prefill": (2304, 208), "widek": (304, 200),
           "lowrank": (100, 200)}


@pytest.mark.parametrize("name", list(REDUCED))
def test_linear_reduced_all_entries(name):
    need_gpu()
    w = workloads.WORKLOADS[name]
    if REDUCED[name]:
        M, N = REDUCED[name]
        w = w.scaled(M=M, N=N)
    inp = workloads.generate(w)
    d = _device_inputs(w, inp)
    _plan_ok(w, d)
    out, codes, scales, y, L = _run_gpu(w, d)
    rows = np.arange(w.M) if w.M <= 400 else np.random.default_rng(5).choice(w.M, 300, replace=False)
    _check(w, inp, out, codes, scales, y, L, np.sort(rows), np.arange(w.N), full=False)


@pytest.mark.parametrize("name", ["prefill", "widek", "lowrank"])
def test_linear_full_size(name):
    need_gpu()
    w = workloads.WORKLOADS[name]
    inp = workloads.generate(w)
    d = _device_inputs(w, inp)
    _plan_ok(w, d)
    out, codes, scales, y, L = _run_gpu(w, d)
    rng = np.random.default_rng(99)
    rows = np.unique(np.concatenate([[0, w.M - 1], rng.choice(w.M, 230, replace=False)]))
    cols = np.unique(np.concatenate([[0, w.N - 1], rng.choice(w.N, 510, replace=False)]))
    _check(w, inp, out, codes, scales, y, L, rows, cols, full=True)


def test_linear_equals_composition_of_entry_points():
    need_gpu()
    w = workloads.WORKLOADS["decode"]
    inp = workloads.generate(w)
    d = _device_inputs(w, inp)
    out = w4.w4a4_linear(d["x"], d["rot"], w.g, d["w_packed"], d["w_scale"], bias=d["bias"])
    c, s = w4.w4a4_rotate_quant_rowwise(d["x"], d["rot"], w.g)
    out2 = w4.w4a4_gemm_from_codes(c, s, d["w_packed"], d["w_scale"], bias=d["bias"],
                                   out_dtype=TORCH_DT[w.dtype])
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16))


def test_batched_input_shape():
    need_gpu()
    w = workloads.WORKLOADS["tiny"]
    inp = workloads.generate(w)
    d = _device_inputs(w, inp)
    x3 = d["x"].view(4, 8, w.K)
    out = w4.w4a4_linear(x3, d["rot"], w.g, d["w_packed"], d["w_scale"], bias=d["bias"])
    out2 = w4.w4a4_linear(d["x"], d["rot"], w.g, d["w_packed"], d["w_scale"], bias=d["bias"])
    assert out.shape == (4, 8, w.N)
    assert torch.equal(out.reshape(-1, w.N), out2)


def test_linear_rejects_on_device_bad_layouts():
    # with device tensors: a wrong-shaped output or weight is refused before
    # anything is enqueued
    need_gpu()
    w = workloads.WORKLOADS["decode"]
    inp = workloads.generate(w)
    d = _device_inputs(w, inp)
    with pytest.raises(ValueError):
        w4.w4a4_linear(d["x"], d["rot"], w.g, d["w_packed"], d["w_scale"], bias=d["bias"],
                       out=torch.empty((w.M, w.N - 1), dtype=torch.bfloat16, device="cuda"))
    with pytest.raises(ValueError):
        w4.w4a4_linear(d["x"], d["rot"], w.g, d["w_packed"][:, :-1], d["w_scale"], bias=d["bias"])
    with pytest.raises(ValueError):
        w4.w4a4_linear(d["x"], d["rot"], w.g, d["w_packed"], d["w_scale"], bias=d["bias"].cpu())
