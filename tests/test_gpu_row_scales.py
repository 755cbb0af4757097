"""Every row-absmax significand through the rotate-quant kernels that take
their row scales from the significand table.

The prefill row kernel (and, for INT4 codes, the g = 256 and column-major
kernels, one thread per row) takes a row's scale s = max(a / qmax, 2^-126),
its reciprocal, the bracketing multipliers and the outcomes of exact ties from
a table indexed by the significand of the 16-bit absmax a, shifted by a's
exponent; rows the table does not cover (zero, a < 2^-119, Inf, NaN) use
divisions.  The per-row
absmax scale and the round-half-even codes follow "[Feat][Ascend] Consolidate
INT8, RotateQuant, RoPE and ConvRot W4A4 backends", section "W4A4 correctness
and performance scope" (qmax = 7) and "[Feat][Ascend] Add fused RotateQuant
backend" (INT8 codes, qmax = 127).

With R = I the rotated values are the inputs themselves (a sum of exact
products with zeros), so every planted value reaches the quantizer exactly:
  * row m's absmax takes fraction pattern m mod 2^F (every significand of the
    format), with an exponent drawn from the whole range, including both
    sides of the table's lower bound 2^-119 (bf16) and fp16 subnormals;
  * each row holds every exact tie (k + 1/2) a / qmax that the format can
    represent, with both signs, plus values drawn below a.
The oracle's quantizer on the same inputs must give the same codes and
scales, bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from tests.gpu_util import bits, dev, host, need_gpu

pytestmark = pytest.mark.gpu

import bit_quantized_linear_rotate_amd as w4  # noqa: E402

FB = {"bf16": 7, "f16": 10}


def representable(v, dt):
    with np.errstate(over="ignore"):
        s = workloads.f32_to_storage(np.array([v], dtype=np.float32), dt)
        back = workloads.storage_to_f32(s, dt)[0]
    return np.float32(v) == np.float64(v) and back == np.float32(v)


def rows_every_significand(dt, M, K, qmax, seed):
    rng = np.random.default_rng(seed)
    F = FB[dt]
    x = np.zeros((M, K), dtype=np.float64)
    for m in range(M):
        f = m % (1 << F)
        if dt == "bf16":
            # exponents over the whole range, with the table's boundary
            # (2^-119 covered, 2^-120 not) and the clamp region
            choices = [-126, -121, -120, -119, -118, -60, -8, 0, 3, 20, 64, 65, 100, 126, 127]
        else:
            # fp16: normal exponents -14..15; -15..-24 make subnormals
            choices = [-24, -20, -15, -14, -13, -4, 0, 2, 7, 14, 15]
        if dt == "bf16":
            E = choices[(m >> F) % len(choices)] if m >= (1 << F) else int(rng.integers(-100, 100))
        else:
            E = choices[int(rng.integers(len(choices)))]
        a = (1.0 + f / (1 << F)) * 2.0 ** E
        if dt == "f16" and E < -14:
            # subnormal fp16: keep the pattern's top bits only
            a = np.floor(a * 2.0 ** 24) * 2.0 ** -24
            if a == 0.0:
                a = 2.0 ** -24
        if not representable(a, dt):
            a = workloads.storage_to_f32(workloads.f32_to_storage(np.array([a], np.float32), dt), dt)[0]
        row = rng.uniform(-1, 1, size=K) * a * 0.9
        row = workloads.storage_to_f32(workloads.f32_to_storage(row.astype(np.float32), dt), dt).astype(np.float64)
        vals = [a if m % 2 else -a]
        for k in range(min(qmax, 7) if qmax == 7 else 7):
            t = (k + 0.5) * a / qmax
            if representable(t, dt):
                vals += [t, -t]
        if qmax == 127:
            for k in (0, 1, 62, 63, 125, 126):
                t = (k + 0.5) * a / qmax
                if representable(t, dt):
                    vals += [t, -t]
        pos = rng.choice(K, size=len(vals), replace=False)
        row[pos] = vals
        x[m] = row
    return workloads.f32_to_storage(x.astype(np.float32), dt)


@pytest.mark.parametrize("dt", ["bf16", "f16"])
@pytest.mark.parametrize("qmax", [7, 127])
def test_row_kernel_every_significand(dt, qmax):
    need_gpu()
    M, K, g = 2048 if dt == "bf16" else 3072, 1152, 64
    x = rows_every_significand(dt, M, K, qmax, seed=17 + qmax)
    xd = dev(x, dt)
    rot = torch.eye(g, dtype=torch.float32, device="cuda")
    if qmax == 7:
        assert w4.w4a4_rotate_quant_plan(xd, rot, g) == "row"
        c, s = w4.w4a4_rotate_quant_rowwise(xd, rot, g)
    else:
        assert w4.w8a8_rotate_quant_plan(xd, rot, g) == "row"
        c, s = w4.w8a8_rotate_quant_rowwise(xd, rot, g)
    c, s = host(c), host(s)
    oc, os_ = oracle.quantize(x, dt, qmax=qmax)
    bad = np.flatnonzero((c != oc).any(axis=1) | (bits(s) != bits(os_)))
    assert bad.size == 0, f"{bad.size} rows differ, first row {bad[0]}: scale {s[bad[0]]!r} vs {os_[bad[0]]!r}"
    ties = int((np.abs(workloads.storage_to_f32(x, dt).astype(np.float64) * qmax /
                       np.abs(workloads.storage_to_f32(x, dt)).max(axis=1, keepdims=True)) % 1 == 0.5).sum())
    print(f"{dt} qmax={qmax}: {M} rows, {1 << FB[dt]} significands, {ties} tie elements, codes and scales bit-exact")


@pytest.mark.parametrize("dt", ["bf16", "f16"])
@pytest.mark.parametrize("qmax", [7, 127])
def test_g256_kernel_every_significand(dt, qmax):
    # contiguous rows, g = 256: the low-rank layer's kernel, whose INT4 codes
    # take the same table through one thread per row
    need_gpu()
    M, K, g = 2048, 2048, 256
    x = rows_every_significand(dt, M, K, qmax, seed=29 + qmax)
    xd = dev(x, dt)
    rot = torch.eye(g, dtype=torch.float32, device="cuda")
    if qmax == 7:
        assert w4.w4a4_rotate_quant_plan(xd, rot, g) == "g256"
        c, s = w4.w4a4_rotate_quant_rowwise(xd, rot, g)
    else:
        assert w4.w8a8_rotate_quant_plan(xd, rot, g) == "g256"
        c, s = w4.w8a8_rotate_quant_rowwise(xd, rot, g)
    c, s = host(c), host(s)
    oc, os_ = oracle.quantize(x, dt, qmax=qmax)
    bad = np.flatnonzero((c != oc).any(axis=1) | (bits(s) != bits(os_)))
    assert bad.size == 0, f"{bad.size} rows differ, first row {bad[0]}: scale {s[bad[0]]!r} vs {os_[bad[0]]!r}"


@pytest.mark.parametrize("dt", ["bf16", "f16"])
def test_colmajor_kernel_every_significand(dt):
    # a transposed view, g = 256: the wide-K kernel, whose second pass takes
    # every code from the row's table entry (one thread per row)
    need_gpu()
    M, K, g = 2048, 2048, 256
    x = rows_every_significand(dt, M, K, 7, seed=31)
    xt = np.ascontiguousarray(x.T)
    xd = dev(xt, dt).t()
    rot = torch.eye(g, dtype=torch.float32, device="cuda")
    assert w4.w4a4_rotate_quant_plan(xd, rot, g) == "colmajor"
    c, s = w4.w4a4_rotate_quant_rowwise(xd, rot, g)
    c, s = host(c), host(s)
    oc, os_ = oracle.quantize(x, dt)
    bad = np.flatnonzero((c != oc).any(axis=1) | (bits(s) != bits(os_)))
    assert bad.size == 0, f"{bad.size} rows differ, first row {bad[0]}: scale {s[bad[0]]!r} vs {os_[bad[0]]!r}"
