"""CPU oracle for the W4A4 rotate/quantize linear -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  It wraps ``w4a4_oracle.c`` (plain C,
fp64 where the method leaves precision open, OpenMP over rows) with numpy
marshalling; each function below follows one step of the method, and the
citations and readings are in the C source next to each step.

Parity status: every step is pinned by the ``not gpu`` tests (brute force in
exact rationals, closed forms of the normalized Hadamard, exhaustive nibble
tables, library conversions, invariants).  Agreement with the pages' own eager
code is unpinned: the pages print no worked example and the captured samples
they replay are not available.

Storage conventions (same as ``workloads``): f32 -> np.float32, f16 ->
np.float16, bf16 -> np.uint16 bit patterns.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "w4a4_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

DT = {"f32": 0, "f16": 1, "bf16": 2}
_NP = {"f32": np.float32, "f16": np.float16, "bf16": np.uint16}

_lib = None


def build() -> str:
    """Compile the oracle with gcc (no fused multiply-add, no fast math)."""
    tmp = _LIB + ".tmp"
    subprocess.check_call([
        "gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
        "-fno-finite-math-only", "-std=c11", "-fPIC", "-shared", "-o", tmp, _SRC, "-lm",
    ])
    os.replace(tmp, _LIB)
    return _LIB


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        _lib = ctypes.CDLL(_LIB)
        i64, vp, i32 = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
        L = _lib
        L.orc_round_to.argtypes = [i32, vp, i64, vp, vp]
        L.orc_decode.argtypes = [i32, vp, i64, vp]
        L.orc_smooth.argtypes = [i32, vp, i64, i64, vp, vp]
        L.orc_rotate.argtypes = [i32, vp, i64, i64, vp, i32, vp]
        L.orc_quantize.argtypes = [i32, vp, i64, i64, vp, vp]
        L.orc_quantize_q.argtypes = [i32, vp, i64, i64, i32, vp, vp]
        L.orc_unpack.argtypes = [vp, i64, i64, vp]
        L.orc_pack.argtypes = [vp, i64, i64, vp]
        L.orc_gemm.argtypes = [vp, i64, i64, vp, i64, i32, vp]
        L.orc_lowrank_down.argtypes = [i32, vp, i64, i64, vp, i32, vp]
        L.orc_epilogue.argtypes = [vp, i64, i64, i64, i32, vp, vp, i32, vp, i32, vp, vp, i32,
                                   i32, vp, i32]
        L.orc_shift.argtypes = [i32, vp, i64, i64, ctypes.c_double, vp]
        L.orc_quantize_ex.argtypes = [i32, vp, i64, i64, i32, i32, vp, vp]
        L.orc_epilogue_ag.argtypes = [vp, i64, i64, i64, vp, vp, i32, i32, vp, i32, vp, vp, i32, i32, vp, i32]
        L.orc_num_threads.argtypes = []
        for f in ("orc_round_to", "orc_decode", "orc_smooth", "orc_rotate", "orc_quantize", "orc_quantize_q",
                  "orc_unpack", "orc_pack", "orc_gemm", "orc_lowrank_down", "orc_epilogue",
                  "orc_shift", "orc_quantize_ex", "orc_epilogue_ag", "orc_num_threads"):
            getattr(L, f).restype = ctypes.c_int
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype=None):
    if a is None:
        return None
    return np.ascontiguousarray(a, dtype=dtype)


def _t(a, dtype):
    """Contiguous storage array for a T-typed operand.  16-bit patterns are
    reinterpreted, never converted; bf16 must arrive as bit patterns."""
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    if dtype == "f16" and a.dtype in (np.uint16, np.int16):
        a = a.view(np.float16)
    if dtype == "bf16":
        if a.dtype == np.int16:
            a = a.view(np.uint16)
        if a.dtype != np.uint16:
            raise TypeError("bf16 operands are passed as uint16 bit patterns")
    return np.ascontiguousarray(a, dtype=_NP[dtype])


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"oracle {what} rejected its arguments (rc={rc})")


def num_threads() -> int:
    return lib().orc_num_threads()


def round_to(dtype: str, v) -> tuple:
    """Round fp64 values to ``dtype`` (nearest-even, overflow to Inf).
    Returns (values as fp64, storage array)."""
    v = _c(np.asarray(v, dtype=np.float64))
    vals = np.empty_like(v)
    bits = np.empty(v.shape, dtype=_NP[dtype])
    lib().orc_round_to(DT[dtype], _p(v), v.size, _p(vals), _p(bits))
    return vals, bits


def decode(dtype: str, bits) -> np.ndarray:
    bits = _t(bits, dtype)
    out = np.empty(bits.shape, dtype=np.float64)
    lib().orc_decode(DT[dtype], _p(bits), bits.size, _p(out))
    return out


def smooth(x, factors, dtype: str) -> np.ndarray:
    x = _t(x, dtype)
    f = _t(factors, dtype)
    M, K = x.shape
    out = np.empty_like(x)
    _check(lib().orc_smooth(DT[dtype], _p(x), M, K, _p(f), _p(out)), "smooth")
    return out


def rotate(x, R, g: int, dtype: str) -> np.ndarray:
    x = _t(x, dtype)
    R = _c(R, np.float64)
    assert R.shape == (g, g)
    M, K = x.shape
    y = np.empty_like(x)
    _check(lib().orc_rotate(DT[dtype], _p(x), M, K, _p(R), g, _p(y)), "rotate")
    return y


def quantize(y, dtype: str, qmax: int = 7) -> tuple:
    """Per-row absmax quantizer -> (codes int8 (M,K), scales fp32 (M,)):
    INT4 codes for qmax = 7, the INT8 mode for qmax = 127."""
    y = _t(y, dtype)
    M, K = y.shape
    codes = np.empty((M, K), dtype=np.int8)
    scales = np.empty((M,), dtype=np.float32)
    _check(lib().orc_quantize_q(DT[dtype], _p(y), M, K, int(qmax), _p(codes), _p(scales)), "quantize")
    return codes, scales


# the post-GELU shift of the SVDQuant page's act_unsigned layers
GELU_UNSIGNED_SHIFT = 0.171875


def shift(x, dtype: str, c: float = GELU_UNSIGNED_SHIFT) -> np.ndarray:
    """T(fp32(x) + c): the act_unsigned main-path activation (reading R18)."""
    x = _t(x, dtype)
    M, K = x.shape
    out = np.empty_like(x)
    _check(lib().orc_shift(DT[dtype], _p(x), M, K, float(c), _p(out)), "shift")
    return out


def quantize_groups(y, dtype: str, unsigned: bool = False, group: int = 0) -> tuple:
    """The INT4 quantizer per block of ``group`` entries of a row (0: the whole
    row), signed [-7, 7] or on the unsigned grid [0, 15] (readings R18/R19).
    Returns (codes int8 (M, K), scales fp32 (M, K/group) or (M,))."""
    y = _t(y, dtype)
    M, K = y.shape
    codes = np.empty((M, K), dtype=np.int8)
    scales = np.empty((M, K // group) if group else (M,), dtype=np.float32)
    _check(lib().orc_quantize_ex(DT[dtype], _p(y), M, K, int(bool(unsigned)), int(group), _p(codes),
                                 _p(scales)), "quantize_groups")
    return codes, scales


def unpack(w_packed, K: int) -> np.ndarray:
    wp = _c(w_packed, np.uint8)
    N = wp.shape[0]
    assert wp.shape == (N, K // 2)
    w = np.empty((N, K), dtype=np.int8)
    _check(lib().orc_unpack(_p(wp), N, K, _p(w)), "unpack")
    return w


def pack(w) -> np.ndarray:
    w = _c(w, np.int8)
    N, K = w.shape
    wp = np.empty((N, K // 2), dtype=np.uint8)
    _check(lib().orc_pack(_p(w), N, K, _p(wp)), "pack")
    return wp


def gemm(codes, w, group: int = 0) -> np.ndarray:
    """Exact integer product -> int64 (M, N), or (M, K/group, N) per K-group."""
    c = _c(codes, np.int8)
    w = _c(w, np.int8)
    M, K = c.shape
    N = w.shape[0]
    assert w.shape == (N, K)
    G = K // group if group else 1
    acc = np.empty((M, G, N) if group else (M, N), dtype=np.int64)
    _check(lib().orc_gemm(_p(c), M, K, _p(w), N, group, _p(acc)), "gemm")
    return acc


def lowrank_down(x, down, dtype: str) -> np.ndarray:
    x = _t(x, dtype)
    down = _t(down, dtype)
    M, K = x.shape
    R = down.shape[1]
    L = np.empty((M, R), dtype=np.float32)
    _check(lib().orc_lowrank_down(DT[dtype], _p(x), M, K, _p(down), R, _p(L)), "lowrank_down")
    return L


def epilogue(acc, s_a, s_w, sw_dtype: str, out_dtype: str, bias=None, bias_dtype=None,
             group: int = 0, L=None, proj_up=None, up_dtype=None) -> np.ndarray:
    acc = _c(acc, np.int64)
    s_a = _c(s_a, np.float32)
    s_w = _t(s_w, sw_dtype)
    M = acc.shape[0]
    N = acc.shape[-1]
    G = acc.shape[1] if group else 1
    bias = _t(bias, bias_dtype) if bias is not None else None
    L = _c(L, np.float32) if L is not None else None
    up = _t(proj_up, up_dtype) if proj_up is not None else None
    R = 0 if L is None else L.shape[1]
    out = np.empty((M, N), dtype=_NP[out_dtype])
    rc = lib().orc_epilogue(_p(acc), M, N, G, group, _p(s_a), _p(s_w), DT[sw_dtype], _p(bias),
                            DT[bias_dtype] if bias_dtype else 0, _p(L), _p(up),
                            DT[up_dtype] if up_dtype else 0, R, _p(out), DT[out_dtype])
    _check(rc, "epilogue")
    return out


def epilogue_ag(acc, s_a, s_w, sw_dtype: str, out_dtype: str, sw_group: int = 0, bias=None,
                bias_dtype=None, L=None, proj_up=None, up_dtype=None) -> np.ndarray:
    """Epilogue with per-group activation scales s_a (M, G) on per-group sums
    acc (M, G, N); s_w (N,) or (G, N) (reading R19)."""
    acc = _c(acc, np.int64)
    s_a = _c(s_a, np.float32)
    s_w = _t(s_w, sw_dtype)
    M, G, N = acc.shape
    assert s_a.shape == (M, G)
    bias = _t(bias, bias_dtype) if bias is not None else None
    L = _c(L, np.float32) if L is not None else None
    up = _t(proj_up, up_dtype) if proj_up is not None else None
    R = 0 if L is None else L.shape[1]
    out = np.empty((M, N), dtype=_NP[out_dtype])
    _check(lib().orc_epilogue_ag(_p(acc), M, N, G, _p(s_a), _p(s_w), DT[sw_dtype], int(sw_group), _p(bias),
                                 DT[bias_dtype] if bias_dtype else 0, _p(L), _p(up),
                                 DT[up_dtype] if up_dtype else 0, R, _p(out), DT[out_dtype]), "epilogue_ag")
    return out


def linear_svdquant(x, w_packed, s_w, dtype: str, sw_dtype: str, sw_group: int = 64, smooth_factors=None,
                    bias=None, proj_down=None, proj_up=None, act_unsigned: bool = False,
                    act_group: int = 64, rows=None, cols=None) -> dict:
    """The SVDQuant W4A4 layer of the svdquant page (``_w4a4_forward``):
    main path x_main = shift(x) when act_unsigned, smoothed, quantized per
    ``act_group`` (no rotation); the low-rank branch on the raw x; the exact
    integer product; the epilogue with per-group activation scales (R19), or
    the per-row epilogue (R9/R10) when act_group = 0.  Optional subsets of
    rows and output columns."""
    x = _t(x, dtype)
    if rows is not None:
        x = x[rows]
    K = x.shape[1]
    wq = unpack(w_packed, K)
    if cols is not None:
        wq = wq[cols]
        s_w = np.asarray(s_w)[..., cols]
        bias = np.asarray(bias)[cols] if bias is not None else None
        proj_up = np.asarray(proj_up)[cols] if proj_up is not None else None
    xm = shift(x, dtype) if act_unsigned else x
    xs = smooth(xm, smooth_factors, dtype) if smooth_factors is not None else xm
    codes, scales = quantize_groups(xs, dtype, act_unsigned, act_group)
    L = lowrank_down(x, proj_down, dtype) if proj_down is not None else None
    bd = dtype if bias is not None else None
    ud = dtype if proj_up is not None else None
    if act_group:
        acc = gemm(codes, wq, act_group)
        out = epilogue_ag(acc, scales, s_w, sw_dtype, dtype, sw_group, bias=bias, bias_dtype=bd, L=L,
                          proj_up=proj_up, up_dtype=ud)
    else:
        acc = gemm(codes, wq, sw_group)
        out = epilogue(acc, scales, s_w, sw_dtype, dtype, bias=bias, bias_dtype=bd, group=sw_group, L=L,
                       proj_up=proj_up, up_dtype=ud)
    return {"codes": codes, "scales": scales, "L": L, "out": out}


def rotate_quant(x, R, g, dtype, smooth_factors=None, qmax: int = 7):
    """Steps a1..a4: (optional smoothing), rotation, per-row quantization.
    ``R=None`` skips the rotation.  Returns (y, codes, scales)."""
    xs = smooth(x, smooth_factors, dtype) if smooth_factors is not None else _t(x, dtype)
    y = rotate(xs, R, g, dtype) if R is not None else xs
    codes, scales = quantize(y, dtype, qmax)
    return y, codes, scales


def linear_int8(x, R, g, w, s_w, dtype: str, sw_dtype: str, bias=None, rows=None, cols=None) -> dict:
    """The dynamic INT8 ConvRot linear ("[Feat][Ascend] Add fused RotateQuant
    backend", "What this PR does": RotateQuant feeding the INT8 linear):
    rotation, per-token INT8 codes (qmax = 127), the exact integer product
    with INT8 weights w (N, K), then the same epilogue as the W4A4 layer
    (per-token scale, per-channel weight scale, bias), on (optionally) a subset
    of rows and columns."""
    if rows is not None:
        x = _t(x, dtype)[rows]
    if cols is not None:
        w = np.asarray(w)[cols]
        s_w = np.asarray(s_w)[cols]
        if bias is not None:
            bias = np.asarray(bias)[cols]
    y, codes, scales = rotate_quant(x, R, g, dtype, qmax=127)
    acc = gemm(codes, w)
    out = epilogue(acc, scales, s_w, sw_dtype, dtype, bias=bias,
                   bias_dtype=dtype if bias is not None else None)
    return {"y": y, "codes": codes, "scales": scales, "acc": acc, "out": out}


def linear(inputs: dict, dtype: str, g: int, sw_dtype: str, sw_group: int = 0,
           rows=None, cols=None) -> dict:
    """The whole forward pass on (optionally) a subset of rows and columns.
    ``inputs`` is a dict as produced by ``workloads.generate``.  Returns the
    intermediate results and the output for the selected rows/columns."""
    x = inputs["x"] if rows is None else inputs["x"][rows]
    K = x.shape[1]
    wp = inputs["w_packed"] if cols is None else inputs["w_packed"][cols]
    s_w = inputs["s_w"]
    if cols is not None:
        s_w = s_w[..., cols]
    bias = inputs.get("bias")
    if bias is not None and cols is not None:
        bias = bias[cols]
    up = inputs.get("proj_up")
    if up is not None and cols is not None:
        up = up[cols]
    y, codes, scales = rotate_quant(x, inputs["rot"], g, dtype, inputs.get("smooth"))
    w = unpack(wp, K)
    acc = gemm(codes, w, sw_group)
    L = lowrank_down(x, inputs["proj_down"], dtype) if inputs.get("proj_down") is not None else None
    out = epilogue(acc, scales, s_w, sw_dtype, dtype, bias=bias,
                   bias_dtype=dtype if bias is not None else None, group=sw_group, L=L,
                   proj_up=up if L is not None else None, up_dtype=dtype if L is not None else None)
    return {"y": y, "codes": codes, "scales": scales, "acc": acc, "L": L, "out": out}
