"""Helpers shared by the GPU parity tests: host<->device transfer of the
storage formats and the comparison rules of the parity protocol."""
import numpy as np
import pytest
import torch

TORCH_DT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import bit_quantized_linear_rotate_amd as b
    if not b.w4a4_device_supported():
        pytest.skip("device is not gfx950")


def dev(a, dt=None):
    """numpy storage -> device tensor (bf16 from uint16 patterns)."""
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    if dt == "bf16":
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(a).cuda()


def host(t, dt=None):
    """device tensor -> numpy storage (bf16 to uint16 patterns)."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def bits(a):
    a = np.ascontiguousarray(a)
    return a.view(np.uint32) if a.dtype == np.float32 else a.view(np.uint16)


def same_values(a, b, dt):
    """Equal storage, counting every NaN as equal to every NaN and +0 == -0."""
    import oracle
    va, vb = oracle.decode(dt, a), oracle.decode(dt, b)
    both_nan = np.isnan(va) & np.isnan(vb)
    return (va == vb) | both_nan


def ulp_distance(a, b, dt):
    """Distance in units in the last place between two arrays of T (finite)."""
    if dt == "f32":
        ia = np.ascontiguousarray(a, np.float32).view(np.int32).astype(np.int64)
        ib = np.ascontiguousarray(b, np.float32).view(np.int32).astype(np.int64)
        top = 0x80000000
    else:
        ia = np.ascontiguousarray(a).view(np.int16).astype(np.int64)
        ib = np.ascontiguousarray(b).view(np.int16).astype(np.int64)
        top = 0x8000
    # map sign-magnitude to a monotone integer line
    ia = np.where(ia < 0, -(ia + top) , ia)
    ib = np.where(ib < 0, -(ib + top), ib)
    return np.abs(ia - ib)


def _ulp(v, dt):
    """Spacing of T at each value (the gap to the next value away from zero)."""
    v = np.abs(np.asarray(v, dtype=np.float64))
    if dt == "f16":
        return np.spacing(v.astype(np.float16)).astype(np.float64)
    if dt == "bf16":
        e = np.floor(np.log2(np.where(v > 0, v, 1.0)))
        e = np.maximum(e, -126.0)
        return np.exp2(e - 7.0)
    return np.spacing(v.astype(np.float32)).astype(np.float64)


def rotated_close(yg, yo, x_in, R, g, dt):
    """Rotated 16-bit values against the oracle's.  The oracle rounds the exact
    group sum once; the GPU sums the exact products in fp32 on MFMA and rounds
    that.  Each value must be within one ulp of T of the oracle's, or within
    one ulp plus the fp32 summation bound g * 2^-24 * sum_i |x_i R_ij| (the
    only room a near-cancelling sum needs).  NaN where the oracle has NaN,
    equal infinities.  Returns (fraction of values not bit-equal, number
    beyond one ulp)."""
    import oracle
    vg, vo = oracle.decode(dt, yg), oracle.decode(dt, yo)
    assert np.array_equal(np.isnan(vg), np.isnan(vo)), "NaN positions differ"
    ok = ~np.isnan(vo)
    d = ulp_distance(np.where(ok, yg, 0).astype(yg.dtype), np.where(ok, yo, 0).astype(yo.dtype), dt)
    xv = np.abs(oracle.decode(dt, x_in))
    M, K = xv.shape
    with np.errstate(invalid="ignore", over="ignore"):
        S = (xv.reshape(M, K // g, g) @ np.abs(np.asarray(R, np.float64))).reshape(M, K)
        bound = np.maximum(_ulp(vo, dt), _ulp(vg, dt)) + g * 2.0 ** -24 * S
        err = np.abs(vg - vo)
    fin = ok & np.isfinite(vo) & np.isfinite(vg) & np.isfinite(S)
    beyond = fin & (d > 1)
    assert (err[beyond] <= bound[beyond]).all(), \
        f"rotated values beyond the fp32 summation bound: {int((err[beyond] > bound[beyond]).sum())}"
    # infinities: equal, or the largest finite value next to the oracle's
    inf = ok & ~fin
    assert (d[inf & np.isfinite(S)] <= 1).all()
    return float((d[ok] > 0).mean()) if ok.any() else 0.0, int(beyond.sum())
