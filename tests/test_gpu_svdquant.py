"""GPU parity of the SVDQuant variant against the oracle (source page
comfy_kitchen/tensor/svdquant_w4a4.py: ``_w4a4_forward`` (act_unsigned shift,
low-rank branch on the raw x), ``svdquant_w4a4_grouped_linear`` (one
activation quantization shared by split projections),
``svdquant_w4a4_fuse_linear_weights`` (runtime N-fusion), module docstring
(INT4 group size 64)).

The quantizer has no rotation, so every step is an elementwise IEEE operation
or an exact maximum: codes and scales are compared bit for bit on every row.
The GEMM's integer sums are exact and its epilogue follows the oracle's
order, so outputs are bit-exact without the low-rank term.  With it, the
GPU's L = x . proj_down and l = L . proj_up are fp32 sums where the oracle
rounds exact sums once: an output is accepted within one ulp of T, or within
the fp32 summation bounds of those two sums (which matter where t + l nearly
cancels): R 2^-23 sum_r |L_r up_r| against the oracle's epilogue on the GPU's
own L, plus sum_r K 2^-24 (sum_k |x_k down_kr|) |up_r| against the oracle's L."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.gpu_util import bits, dev, host, need_gpu, ulp_distance
from tests.test_gpu_edge_rows import build_matrix, scales_equal

pytestmark = pytest.mark.gpu

import bit_quantized_linear_rotate_amd as w4  # noqa: E402


def _lowrank_close(go, ref, dt, x, down, up, L, with_l_error):
    """go within one ulp of ref, or within the fp32 summation bounds of the
    low-rank term (see the module docstring)."""
    gv, rv = oracle.decode(dt, go), oracle.decode(dt, ref)
    Lv = np.abs(np.asarray(L, np.float64))
    upv = np.abs(oracle.decode(dt, up))
    K, R = oracle.decode(dt, down).shape
    bound = R * 2.0 ** -23 * (Lv @ upv.T)
    if with_l_error:
        S = np.abs(oracle.decode(dt, x)) @ np.abs(oracle.decode(dt, down))     # (M, R)
        bound = bound + (K * 2.0 ** -24 * S) @ upv.T
    ok = (ulp_distance(go, ref, dt) <= 1) | (np.abs(gv - rv) <= bound + 2.0 ** -133)
    assert ok.all(), f"{int((~ok).sum())} outputs beyond one ulp and the low-rank summation bound"


def _oracle_quant(x, dt, smooth, unsigned, group):
    xm = oracle.shift(x, dt) if unsigned else x
    xs = oracle.smooth(xm, smooth, dt) if smooth is not None else xm
    return oracle.quantize_groups(xs, dt, unsigned, group)


@pytest.mark.parametrize("dt", ["bf16", "f16"])
@pytest.mark.parametrize("unsigned", [False, True])
@pytest.mark.parametrize("group", [0, 64])
@pytest.mark.parametrize("smoothing", [False, True])
def test_quantizer_bit_exact_with_edge_rows(dt, unsigned, group, smoothing):
    need_gpu()
    M, K = 96, 4096
    x, where = build_matrix(dt, M, K, 64, seed=71 + unsigned + 2 * group)
    if unsigned:
        # post-GELU-like rows: GELU's minimum is about -0.17
        xf = workloads.storage_to_f32(x, dt)
        xf = np.where(np.isfinite(xf), np.maximum(xf, -0.17), xf)
        x = workloads.f32_to_storage(xf, dt)
    sm = workloads.f32_to_storage(np.random.default_rng(8).uniform(0.5, 2.0, size=K), dt) if smoothing else None
    c, s = w4.w4a4_quantize_svdquant(dev(x, dt), dev(sm, dt) if sm is not None else None, unsigned, group)
    c, s = host(c), host(s)
    rc, rs = _oracle_quant(x, dt, sm, unsigned, group)
    assert np.array_equal(c, rc)
    assert scales_equal(s.reshape(-1), rs.reshape(-1))
    if unsigned:
        assert c.min() >= 0 and c.max() <= 15


@pytest.mark.parametrize("K", [64, 192, 1088, 16384])
def test_quantizer_widths(K):
    # one group, a partial last 512-element chunk, the widest row
    need_gpu()
    rng = np.random.default_rng(K)
    x = workloads.f32_to_storage(rng.standard_t(4, size=(37, K)).astype(np.float32), "bf16")
    for group in (0, 64):
        for unsigned in (False, True):
            c, s = w4.w4a4_quantize_svdquant(dev(x, "bf16"), None, unsigned, group)
            rc, rs = _oracle_quant(x, "bf16", None, unsigned, group)
            assert np.array_equal(host(c), rc) and scales_equal(host(s).reshape(-1), rs.reshape(-1))


@pytest.mark.parametrize("sw_group", [0, 64])
@pytest.mark.parametrize("unsigned", [False, True])
@pytest.mark.parametrize("odt", ["bf16", "f32"])
@pytest.mark.parametrize("M,K,N", [(200, 1024, 300), (7, 64, 17), (129, 2048, 128)])
def test_gemm_group_activation_scales_bit_exact(sw_group, unsigned, odt, M, K, N):
    need_gpu()
    rng = np.random.default_rng(M + K + N + sw_group)
    codes = (rng.integers(0, 16, size=(M, K)) if unsigned else rng.integers(-7, 8, size=(M, K))).astype(np.int8)
    codes[0] = 15 if unsigned else -7
    wq = rng.integers(-8, 8, size=(N, K)).astype(np.int8)
    wq[0] = -8
    sa = rng.uniform(0.001, 0.1, size=(M, K // 64)).astype(np.float32)
    sw = workloads.f32_to_storage(rng.uniform(0.001, 0.01, size=(K // 64, N) if sw_group else (N,)), odt)
    b = workloads.f32_to_storage(rng.normal(0, 0.1, size=N).astype(np.float32), odt)
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16}[odt]
    out = w4.w4a4_gemm_svdquant(dev(codes), dev(sa), dev(oracle.pack(wq)), dev(sw, odt), 64, unsigned,
                                w_scale_group=sw_group, bias=dev(b, odt), out_dtype=tdt)
    acc = oracle.gemm(codes, wq, 64)
    ref = oracle.epilogue_ag(acc, sa, sw, odt, odt, sw_group, bias=b, bias_dtype=odt)
    assert np.array_equal(bits(host(out)), bits(ref))


def test_gemm_per_row_unsigned_is_the_w4a4_epilogue():
    # act_group 0 with unsigned codes: the W4A4 epilogue, bit for bit
    need_gpu()
    rng = np.random.default_rng(72)
    M, K, N = 150, 512, 200
    codes = rng.integers(0, 16, size=(M, K)).astype(np.int8)
    wq = rng.integers(-8, 8, size=(N, K)).astype(np.int8)
    sa = rng.uniform(0.001, 0.1, size=M).astype(np.float32)
    sw = workloads.f32_to_storage(rng.uniform(0.001, 0.01, size=N), "bf16")
    out = w4.w4a4_gemm_svdquant(dev(codes), dev(sa), dev(oracle.pack(wq)), dev(sw, "bf16"), 0, True,
                                w_scale_group=0)
    ref = oracle.epilogue(oracle.gemm(codes, wq), sa, sw, "bf16", "bf16")
    assert np.array_equal(bits(host(out)), bits(ref))


def _layer_inputs(M, K, N, R, dt, seed):
    rng = np.random.default_rng(seed)
    x = workloads.f32_to_storage(rng.standard_normal((M, K)).astype(np.float32), dt)
    wq = rng.integers(-8, 8, size=(N, K)).astype(np.int8)
    sw = workloads.f32_to_storage(rng.uniform(0.005, 0.02, size=(K // 64, N)), dt)
    sm = workloads.f32_to_storage(rng.uniform(0.5, 2.0, size=K), dt)
    down = workloads.f32_to_storage((rng.standard_normal((K, R)) / np.sqrt(K)).astype(np.float32), dt)
    up = workloads.f32_to_storage(rng.normal(0, 0.1, size=(N, R)).astype(np.float32), dt)
    bias = workloads.f32_to_storage(rng.normal(0, 0.1, size=N).astype(np.float32), dt)
    return x, wq, sw, sm, down, up, bias


def _compare_layer(out, ref, lowrank, dt, x=None, down=None, up=None, L=None):
    go = host(out)
    if lowrank:
        _lowrank_close(go, ref, dt, x, down, up, L, with_l_error=True)
    else:
        assert np.array_equal(bits(go), bits(ref))


@pytest.mark.parametrize("unsigned", [False, True])
@pytest.mark.parametrize("group", [0, 64])
@pytest.mark.parametrize("lowrank", [False, True])
def test_linear_svdquant_reduced(unsigned, group, lowrank):
    need_gpu()
    dt = "bf16"
    M, K, N, R = 160, 2048, 320, 32
    x, wq, sw, sm, down, up, bias = _layer_inputs(M, K, N, R, dt, seed=73)
    if unsigned:
        x = workloads.f32_to_storage(np.maximum(workloads.storage_to_f32(x, dt), -0.17), dt)
    out = w4.w4a4_linear_svdquant(dev(x, dt), dev(oracle.pack(wq)), dev(sw, dt), 64, bias=dev(bias, dt),
                                  smooth=dev(sm, dt), proj_down=dev(down, dt) if lowrank else None,
                                  proj_up=dev(up, dt) if lowrank else None, act_unsigned=unsigned,
                                  act_group=group)
    ref = oracle.linear_svdquant(x, oracle.pack(wq), sw, dt, dt, 64, sm, bias, down if lowrank else None,
                                 up if lowrank else None, act_unsigned=unsigned, act_group=group)
    _compare_layer(out, ref["out"], lowrank, dt, x, down, up, ref["L"])
    if lowrank:
        # against the oracle's epilogue on the GPU's own codes, scales and L
        c, s = w4.w4a4_quantize_svdquant(dev(x, dt), dev(sm, dt), unsigned, group)
        Lg = host(w4.w4a4_lowrank_down(dev(x, dt), dev(down, dt)))
        gc, gs = host(c), host(s)
        if group:
            own = oracle.epilogue_ag(oracle.gemm(gc, wq, 64), gs, sw, dt, dt, 64, bias=bias, bias_dtype=dt, L=Lg,
                                     proj_up=up, up_dtype=dt)
        else:
            own = oracle.epilogue(oracle.gemm(gc, wq, 64), gs, sw, dt, dt, bias=bias, bias_dtype=dt, group=64,
                                  L=Lg, proj_up=up, up_dtype=dt)
        _lowrank_close(host(out), own, dt, x, down, up, Lg, with_l_error=False)


def test_linear_svdquant_full_size_lowrank_shape():
    # the low-rank workload's shape (M=4096, K=16384, N=6144, rank 32, bf16,
    # smoothing, per-64-group weight scales) with group activation scales and
    # the unsigned grid; codes and scales of every row, sampled outputs
    need_gpu()
    w = workloads.WORKLOADS["lowrank"]
    inp = workloads.generate(w)
    dt = w.dtype
    x = workloads.f32_to_storage(np.maximum(workloads.storage_to_f32(inp["x"], dt), -0.17), dt)
    xd = dev(x, dt)
    d = dict(w_packed=dev(inp["w_packed"]), w_scale=dev(inp["s_w"], w.sw_dtype), smooth=dev(inp["smooth"], dt),
             down=dev(inp["proj_down"], dt), up=dev(inp["proj_up"], dt))
    out = host(w4.w4a4_linear_svdquant(xd, d["w_packed"], d["w_scale"], 64, smooth=d["smooth"],
                                       proj_down=d["down"], proj_up=d["up"], act_unsigned=True, act_group=64))
    c, s = w4.w4a4_quantize_svdquant(xd, d["smooth"], True, 64)
    rc, rs = _oracle_quant(x, dt, inp["smooth"], True, 64)
    assert np.array_equal(host(c), rc) and scales_equal(host(s).reshape(-1), rs.reshape(-1))
    rng = np.random.default_rng(74)
    rows = np.unique(np.concatenate([[0, w.M - 1], rng.choice(w.M, 62, replace=False)]))
    cols = np.unique(np.concatenate([[0, w.N - 1], rng.choice(w.N, 254, replace=False)]))
    ref = oracle.linear_svdquant(x, inp["w_packed"], inp["s_w"], dt, w.sw_dtype, 64, inp["smooth"], None,
                                 inp["proj_down"], inp["proj_up"], act_unsigned=True, act_group=64,
                                 rows=rows, cols=cols)
    _lowrank_close(out[np.ix_(rows, cols)], ref["out"], dt, x[rows], inp["proj_down"], inp["proj_up"][cols],
                   ref["L"], with_l_error=True)


def test_grouped_and_fused_projections():
    # split Q/K/V sharing smoothing and proj_down: the grouped call, separate
    # calls and the N-fused layer give the same bits; all match the oracle
    need_gpu()
    dt = "bf16"
    M, K, R = 130, 1024, 16
    rng = np.random.default_rng(75)
    x = workloads.f32_to_storage(rng.standard_normal((M, K)).astype(np.float32), dt)
    sm = workloads.f32_to_storage(rng.uniform(0.5, 2.0, size=K), dt)
    down = workloads.f32_to_storage((rng.standard_normal((K, R)) / 32).astype(np.float32), dt)
    projs, hosts = [], []
    for i, N in enumerate((256, 256, 96)):
        wq = rng.integers(-8, 8, size=(N, K)).astype(np.int8)
        sw = workloads.f32_to_storage(rng.uniform(0.005, 0.02, size=(K // 64, N)), dt)
        up = workloads.f32_to_storage(rng.normal(0, 0.1, size=(N, R)).astype(np.float32), dt)
        bias = workloads.f32_to_storage(rng.normal(0, 0.1, size=N).astype(np.float32), dt) if i != 1 else None
        projs.append(dict(w_packed=dev(oracle.pack(wq)), w_scale=dev(sw, dt), proj_up=dev(up, dt),
                          bias=dev(bias, dt) if bias is not None else None))
        hosts.append((wq, sw, up, bias))
    xd, smd, downd = dev(x, dt), dev(sm, dt), dev(down, dt)
    grouped = w4.w4a4_linear_svdquant_grouped(xd, projs, smooth=smd, proj_down=downd, act_group=64)
    fused, feats = w4.fuse_linear_weights(projs)
    fout = w4.w4a4_linear_svdquant(xd, fused["w_packed"], fused["w_scale"], 64, bias=fused["bias"], smooth=smd,
                                   proj_down=downd, proj_up=fused["proj_up"], act_group=64)
    fsplit = torch.split(fout, feats, dim=-1)
    for i, p in enumerate(projs):
        single = w4.w4a4_linear_svdquant(xd, p["w_packed"], p["w_scale"], 64, bias=p["bias"], smooth=smd,
                                         proj_down=downd, proj_up=p["proj_up"], act_group=64)
        assert torch.equal(grouped[i].view(torch.int16), single.view(torch.int16))
        assert torch.equal(fsplit[i].contiguous().view(torch.int16), single.view(torch.int16))
        wq, sw, up, bias = hosts[i]
        ref = oracle.linear_svdquant(x, oracle.pack(wq), sw, dt, dt, 64, sm, bias, down, up, act_group=64)
        _lowrank_close(host(single), ref["out"], dt, x, down, up, ref["L"], with_l_error=True)


def test_svdquant_rejects_bad_arguments():
    need_gpu()
    x = torch.zeros((8, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):
        w4.w4a4_quantize_svdquant(x, act_group=32)
    with pytest.raises(NotImplementedError):
        w4.w4a4_quantize_svdquant(x.float())
    with pytest.raises(NotImplementedError):
        w4.w4a4_quantize_svdquant(x.t().contiguous().t())
    with pytest.raises(ValueError):
        w4.w4a4_quantize_svdquant(torch.zeros((8, 96), dtype=torch.bfloat16, device="cuda"), act_group=64)
