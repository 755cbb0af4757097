"""End-to-end GPU parity of the whole W4A4 linear on the five workloads.

For each workload, at a reduced size (all rows and columns compared) and at
its full size (sampled rows and columns, in the launch configuration the
benchmark times):
  * activation codes differ from the oracle's by at most 1, on at most 1e-4 of
    the entries (rows whose scale differs are counted, at most 5%);
  * the output equals the oracle's epilogue applied to the GPU's own codes and
    scales bit for bit (within 1 ulp with the low-rank term);
  * rows whose codes and scales match the oracle's give the oracle's output
    (bit-exact, or 1 ulp with the low-rank term)."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.gpu_util import TORCH_DT, bits, dev, host, need_gpu, ulp_distance

pytestmark = pytest.mark.gpu

import bit_quantized_linear_rotate_amd as w4  # noqa: E402


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
    L = w4.w4a4_lowrank_down(d["x"], d["proj_down"]) if d["proj_down"] is not None else None
    torch.cuda.synchronize()
    return out, codes, scales, L


def _check(w, inp, out, codes, scales, L, rows, cols):
    dt = w.dtype
    ref = oracle.linear(inp, dt, w.g, w.sw_dtype, w.sw_group, rows=rows, cols=cols)
    gc = host(codes)[rows]
    gs = host(scales)[rows]
    go = host(out)[np.ix_(rows, cols)]
    lowrank = w.rank > 0
    # codes: +-1 flips only, rarely
    same_scale = bits(gs) == bits(ref["scales"])
    assert (~same_scale).sum() <= max(1, 0.05 * len(rows))
    dc = np.abs(gc.astype(np.int32) - ref["codes"])
    assert dc[same_scale].max(initial=0) <= 1
    flips = (dc[same_scale] > 0).mean() if same_scale.any() else 0.0
    assert flips <= 1e-4, flips
    # the output is the oracle's epilogue of the GPU's own codes
    wq = oracle.unpack(inp["w_packed"][cols], w.K)
    acc = oracle.gemm(gc, wq, w.sw_group)
    s_w = inp["s_w"][..., cols]
    bias = inp["bias"][cols] if inp["bias"] is not None else None
    up = inp["proj_up"][cols] if lowrank else None
    Lr = host(L)[rows] if lowrank else None
    own = oracle.epilogue(acc, gs, s_w, w.sw_dtype, dt, bias=bias,
                          bias_dtype=dt if bias is not None else None, group=w.sw_group,
                          L=Lr, proj_up=up, up_dtype=dt if lowrank else None)
    exact_rows = same_scale & (dc.max(axis=1) == 0)
    if lowrank:
        assert ulp_distance(go, own, dt).max() <= 1
        assert ulp_distance(go[exact_rows], ref["out"][exact_rows], dt).max(initial=0) <= 1
    else:
        assert np.array_equal(bits(go), bits(own))
        assert np.array_equal(bits(go[exact_rows]), bits(ref["out"][exact_rows]))
    print(f"{w.name}: rows={len(rows)} cols={len(cols)} code flips={flips:.2e} "
          f"rows with other scale={(~same_scale).sum()} exact rows={exact_rows.sum()}")


REDUCED = {"tiny": None, "decode": None, "prefill": (300, 200), "widek": (300, 200),
           "lowrank": (100, 200)}


@pytest.mark.parametrize("name", list(REDUCED))
def test_linear_reduced_all_entries(name):
    need_gpu()
    w = workloads.WORKLOADS[name]
    if REDUCED[name]:
        M, N = REDUCED[name]
        w = w.scaled(M=M, N=N)
    inp = workloads.generate(w)
    out, codes, scales, L = _run_gpu(w, _device_inputs(w, inp))
    _check(w, inp, out, codes, scales, L, np.arange(w.M), np.arange(w.N))


@pytest.mark.parametrize("name", ["prefill", "widek", "lowrank"])
def test_linear_full_size_sampled(name):
    need_gpu()
    w = workloads.WORKLOADS[name]
    inp = workloads.generate(w)
    out, codes, scales, L = _run_gpu(w, _device_inputs(w, inp))
    rng = np.random.default_rng(99)
    rows = np.unique(np.concatenate([[0, w.M - 1], rng.choice(w.M, 46, replace=False)]))
    cols = np.unique(np.concatenate([[0, w.N - 1], rng.choice(w.N, 254, replace=False)]))
    _check(w, inp, out, codes, scales, L, rows, cols)


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
