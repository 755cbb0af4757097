"""The no-allocation entry point (w4a4_linear_noalloc) against w4a4_linear.

Two calls in a row through the C ABI, the second on a smaller layer (the
scratch keeps the first call's contents), each compared bit for bit with
w4a4_linear on the same inputs with its own workspace; a low-rank layer
with smoothing and per-64-group weight scales (codes, scales and low-rank
activations all in the scratch); the size limit refused before anything is
enqueued; and the same results with the scratch reused after other work."""
import ctypes

import numpy as np
import pytest
import torch

import workloads
from tests.gpu_util import dev, need_gpu

pytestmark = pytest.mark.gpu

import bit_quantized_linear_rotate_amd as w4  # noqa: E402
from bit_quantized_linear_rotate_amd import _binding as b  # noqa: E402


def _device(w, inp):
    dt = w.dtype
    return dict(
        x=dev(inp["x"], dt),
        rot=torch.from_numpy(inp["rot"].astype(np.float32)).cuda(),
        w_packed=dev(inp["w_packed"]),
        w_scale=dev(inp["s_w"], w.sw_dtype),
        bias=dev(inp["bias"], dt) if inp["bias"] is not None else None,
        smooth=dev(inp["smooth"], dt) if inp["smooth"] is not None else None,
        proj_down=dev(inp["proj_down"], dt) if inp["proj_down"] is not None else None,
        proj_up=dev(inp["proj_up"], dt) if inp["proj_up"] is not None else None,
    )


def _reference(w, d):
    return w4.w4a4_linear(d["x"], d["rot"], w.g, d["w_packed"], d["w_scale"], w_scale_group=w.sw_group,
                          bias=d["bias"], smooth=d["smooth"], proj_down=d["proj_down"],
                          proj_up=d["proj_up"])


def _noalloc_raw(w, d, out):
    """Straight through the C ABI (ctypes), no binding logic."""
    x = d["x"]
    M, K = x.shape
    N = d["w_packed"].shape[0]
    rank = d["proj_down"].shape[1] if d["proj_down"] is not None else 0
    p = lambda t: None if t is None else t.data_ptr()  # noqa: E731
    rc = w4.lib().w4a4_linear_noalloc(
        p(x), b._dt(x), M, K, x.stride(0), x.stride(1), p(d["rot"]), w.g, p(d["smooth"]),
        p(d["w_packed"]), N, p(d["w_scale"]), b._dt(d["w_scale"]), w.sw_group, p(d["bias"]),
        p(d["proj_down"]), p(d["proj_up"]), rank, p(out), b._DT[out.dtype],
        torch.cuda.current_stream().cuda_stream)
    assert rc == 0, w4.lib().w4a4_last_error()
    return out


def _bits_equal(a, c):
    return torch.equal(a.view(torch.int16), c.view(torch.int16))


def test_noalloc_two_calls_second_smaller():
    need_gpu()
    big = workloads.WORKLOADS["prefill"].scaled(M=2304, N=384)
    small = workloads.WORKLOADS["decode"]
    cases = []
    for w in (big, small):
        d = _device(w, workloads.generate(w))
        out = torch.full((w.M, w.N), float("nan"), dtype=d["x"].dtype, device="cuda")
        cases.append((w, d, out))
    # both calls back to back on one stream, then both references
    for w, d, out in cases:
        _noalloc_raw(w, d, out)
    torch.cuda.synchronize()
    for w, d, out in cases:
        ref = _reference(w, d)
        torch.cuda.synchronize()
        assert _bits_equal(out, ref), w.name


def test_noalloc_lowrank_layer_and_binding():
    need_gpu()
    w = workloads.WORKLOADS["lowrank"].scaled(M=96, N=256)
    d = _device(w, workloads.generate(w))
    out = torch.empty((w.M, w.N), dtype=d["x"].dtype, device="cuda")
    w4.w4a4_linear_noalloc(d["x"], d["rot"], w.g, d["w_packed"], d["w_scale"], out,
                           w_scale_group=w.sw_group, bias=d["bias"], smooth=d["smooth"],
                           proj_down=d["proj_down"], proj_up=d["proj_up"])
    ref = _reference(w, d)
    torch.cuda.synchronize()
    assert _bits_equal(out, ref)
    # a second, smaller call after unrelated allocations and work
    junk = torch.randn(1 << 20, device="cuda") * 3
    w2 = workloads.WORKLOADS["tiny"]
    d2 = _device(w2, workloads.generate(w2))
    out2 = torch.empty((w2.M, w2.N), dtype=d2["x"].dtype, device="cuda")
    _noalloc_raw(w2, d2, out2)
    ref2 = _reference(w2, d2)
    torch.cuda.synchronize()
    assert torch.equal(out2.view(torch.int32), ref2.view(torch.int32))
    del junk


def test_noalloc_refuses_layers_beyond_the_scratch():
    need_gpu()
    # codes alone need M*K bytes: one row more than the scratch holds
    K = 4096
    M = w4.NOALLOC_SCRATCH_BYTES // K + 1
    x = torch.zeros((M, K), dtype=torch.bfloat16, device="cuda")
    rot = torch.eye(64, dtype=torch.float32, device="cuda")
    wp = torch.zeros((64, K // 2), dtype=torch.uint8, device="cuda")
    sw = torch.ones((64,), dtype=torch.float32, device="cuda")
    out = torch.full((M, 64), 7.0, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError, match="scratch"):
        w4.w4a4_linear_noalloc(x, rot, 64, wp, sw, out)
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())   # nothing was enqueued


def test_noalloc_declared_in_header():
    import os
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    with open(os.path.join(root, "include", "w4a4.h")) as f:
        text = f.read()
    assert "int w4a4_linear_noalloc(" in text and "W4A4_NOALLOC_SCRATCH_BYTES" in text
    assert w4.NOALLOC_SCRATCH_BYTES == 128 << 20
    assert isinstance(w4.lib().w4a4_linear_noalloc, ctypes._CFuncPtr)
