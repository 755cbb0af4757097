"""Thin ctypes binding over libw4a4.so (C ABI in include/w4a4.h).

Argument marshalling only: every step of the layer runs in the HIP kernels
behind the C ABI.  torch supplies device memory and the current HIP stream.
There is no CPU fallback: if the library is missing or the device is not
gfx950, the calls raise.
"""
from __future__ import annotations

import ctypes
import os
import warnings
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libw4a4.so")

OK, INVALID, UNSUPPORTED, HIP_ERROR = 0, -1, -2, -3
F32, F16, BF16 = 0, 1, 2
_DT = {torch.float32: F32, torch.float16: F16, torch.bfloat16: BF16}
_TORCH = {F32: torch.float32, F16: torch.float16, BF16: torch.bfloat16}

_lib: Optional[ctypes.CDLL] = None

_i64, _i32, _vp, _sz = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t
_SIGNATURES = {
    "w4a4_rotate_quant_rowwise": ([_vp, ctypes.c_int, _i64, _i64, _i64, _i64, _vp, _i32, _vp, _vp,
                                   _vp, _vp, _vp], ctypes.c_int),
    "w4a4_lowrank_down": ([_vp, ctypes.c_int, _i64, _i64, _i64, _i64, _vp, _i32, _vp, _vp],
                          ctypes.c_int),
    "w4a4_gemm_from_codes": ([_vp, _vp, _i64, _i64, _vp, _i64, _vp, ctypes.c_int, _i32, _vp,
                              ctypes.c_int, _vp, _vp, ctypes.c_int, _i32, _vp, ctypes.c_int, _vp,
                              _i64, _vp, _sz, _vp], ctypes.c_int),
    "w4a4_gemm_workspace_size": ([_i64, _i64, _i64, _i64], _sz),
    "w4a4_linear": ([_vp, ctypes.c_int, _i64, _i64, _i64, _i64, _vp, _i32, _vp, _vp, _i64, _vp,
                     ctypes.c_int, _i32, _vp, _vp, _vp, _i32, _vp, ctypes.c_int, _vp, _sz, _vp],
                    ctypes.c_int),
    "w4a4_linear_workspace_size": ([_i64, _i64, _i64, _i32], _sz),
    "w4a4_int32_guard": ([_i64, ctypes.POINTER(_i64)], ctypes.c_int),
    "w4a4_last_error": ([], ctypes.c_char_p),
    "w4a4_device_supported": ([], ctypes.c_int),
}


class W4A4Error(RuntimeError):
    pass


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is not built; run `python -c 'import __graft_entry__ as g; g.build()'` "
                "(no CPU fallback exists)")
        L = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in _SIGNATURES.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = res
        _lib = L
    return _lib


def _check(rc: int, what: str):
    if rc == OK:
        return
    msg = lib().w4a4_last_error().decode(errors="replace")
    if rc == INVALID:
        raise ValueError(f"{what}: {msg}")
    if rc == UNSUPPORTED:
        raise NotImplementedError(f"{what}: {msg}")
    raise W4A4Error(f"{what}: {msg}")


# (plain ints for pointer arguments: ctypes converts them through argtypes,
# and building c_void_p objects per call costs host time that small layers
# notice)
def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(device) -> int:
    """The current HIP stream of `device` as an integer handle."""
    if _raw_stream is not None:
        idx = device.index if device.index is not None else torch.cuda.current_device()
        return _raw_stream(idx)
    return torch.cuda.current_stream(device).cuda_stream


def _dt(t: torch.Tensor) -> int:
    try:
        return _DT[t.dtype]
    except KeyError:
        raise NotImplementedError(f"dtype {t.dtype} is not fp32/fp16/bf16") from None


def _as_2d(x: torch.Tensor) -> torch.Tensor:
    if x.dim() == 2:
        return x
    K = x.shape[-1]
    try:
        return x.view(-1, K)
    except RuntimeError:
        warnings.warn("activation view cannot be flattened to (M, K) without a copy; copying")
        return x.reshape(-1, K)


def _rot_arg(rot: Optional[torch.Tensor], g: int):
    if rot is None:
        return None, 0
    if rot.dtype != torch.float32 or rot.shape != (g, g) or not rot.is_contiguous():
        raise ValueError("rot must be a contiguous (g, g) float32 tensor")
    return rot, g


def w4a4_int32_guard(K: int):
    """(needs_chunking, k_chunk) for a K-long INT32 accumulation."""
    c = _i64(0)
    need = lib().w4a4_int32_guard(K, ctypes.byref(c))
    return bool(need), int(c.value)


def w4a4_linear_workspace_size(M: int, K: int, N: int, rank: int = 0) -> int:
    return int(lib().w4a4_linear_workspace_size(M, K, N, rank))


def w4a4_gemm_workspace_size(M: int, N: int, K: int, k_chunk: int = 0) -> int:
    return int(lib().w4a4_gemm_workspace_size(M, N, K, k_chunk))


def w4a4_device_supported() -> bool:
    return lib().w4a4_device_supported() == OK


def w4a4_rotate_quant_rowwise(x: torch.Tensor, rot: Optional[torch.Tensor], g: int,
                              smooth: Optional[torch.Tensor] = None,
                              return_rotated: bool = False):
    """Rotate + quantize rows of x (..., K).  Returns (codes int8 (M, K),
    scales fp32 (M,)) and, if requested, the rotated values (M, K) in x.dtype."""
    x2 = _as_2d(x)
    M, K = x2.shape
    rot, g = _rot_arg(rot, g)
    dev = x2.device
    codes = torch.empty((M, K), dtype=torch.int8, device=dev)
    scales = torch.empty((M,), dtype=torch.float32, device=dev)
    rotated = torch.empty((M, K), dtype=x2.dtype, device=dev) if return_rotated else None
    if smooth is not None and (smooth.dtype != x2.dtype or not smooth.is_contiguous()):
        raise ValueError("smooth must be contiguous and in x.dtype")
    rc = lib().w4a4_rotate_quant_rowwise(
        _ptr(x2), _dt(x2), M, K, x2.stride(0), x2.stride(1), _ptr(rot), g, _ptr(smooth),
        _ptr(codes), _ptr(scales), _ptr(rotated), _stream(dev))
    _check(rc, "w4a4_rotate_quant_rowwise")
    return (codes, scales, rotated) if return_rotated else (codes, scales)


def w4a4_lowrank_down(x: torch.Tensor, proj_down: torch.Tensor) -> torch.Tensor:
    x2 = _as_2d(x)
    M, K = x2.shape
    R = proj_down.shape[1]
    lora = torch.empty((M, R), dtype=torch.float32, device=x2.device)
    rc = lib().w4a4_lowrank_down(_ptr(x2), _dt(x2), M, K, x2.stride(0), x2.stride(1),
                                 _ptr(proj_down.contiguous()), R, _ptr(lora), _stream(x2.device))
    _check(rc, "w4a4_lowrank_down")
    return lora


def w4a4_gemm_from_codes(codes: torch.Tensor, scales: torch.Tensor, w_packed: torch.Tensor,
                         w_scale: torch.Tensor, w_scale_group: int = 0,
                         bias: Optional[torch.Tensor] = None,
                         lora_act: Optional[torch.Tensor] = None,
                         proj_up: Optional[torch.Tensor] = None,
                         out_dtype: torch.dtype = torch.bfloat16,
                         return_acc: bool = False, k_chunk: int = 0):
    """INT4-code GEMM with the fused epilogue.  Returns out (M, N) and, if
    requested, the exact int32 sums (M, N)."""
    M, K = codes.shape
    N = w_packed.shape[0]
    dev = codes.device
    out = torch.empty((M, N), dtype=out_dtype, device=dev)
    acc = torch.empty((M, N), dtype=torch.int32, device=dev) if return_acc else None
    wsz = w4a4_gemm_workspace_size(M, N, K, k_chunk)
    ws = torch.empty((max(wsz, 1),), dtype=torch.uint8, device=dev) if wsz else None
    rank = 0 if lora_act is None else lora_act.shape[1]
    rc = lib().w4a4_gemm_from_codes(
        _ptr(codes), _ptr(scales), M, K, _ptr(w_packed), N, _ptr(w_scale), _dt(w_scale),
        w_scale_group, _ptr(bias), _dt(bias) if bias is not None else 0, _ptr(lora_act),
        _ptr(proj_up), _dt(proj_up) if proj_up is not None else 0, rank, _ptr(out),
        _DT[out_dtype], _ptr(acc), k_chunk, _ptr(ws), wsz, _stream(dev))
    _check(rc, "w4a4_gemm_from_codes")
    return (out, acc) if return_acc else out


def w4a4_linear(x: torch.Tensor, rot: Optional[torch.Tensor], g: int, w_packed: torch.Tensor,
                w_scale: torch.Tensor, w_scale_group: int = 0,
                bias: Optional[torch.Tensor] = None, smooth: Optional[torch.Tensor] = None,
                proj_down: Optional[torch.Tensor] = None, proj_up: Optional[torch.Tensor] = None,
                out_dtype: Optional[torch.dtype] = None,
                workspace: Optional[torch.Tensor] = None,
                out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """The whole W4A4 linear: y = layer(x) of shape (..., N)."""
    lead = x.shape[:-1]
    x2 = _as_2d(x)
    M, K = x2.shape
    N = w_packed.shape[0]
    rot, g = _rot_arg(rot, g)
    dev = x2.device
    out_dtype = out_dtype or x2.dtype
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=dev)
    rank = 0 if proj_down is None else proj_down.shape[1]
    need = w4a4_linear_workspace_size(M, K, N, rank)
    if workspace is None:
        workspace = torch.empty((max(need, 1),), dtype=torch.uint8, device=dev)
    rc = lib().w4a4_linear(
        _ptr(x2), _dt(x2), M, K, x2.stride(0), x2.stride(1), _ptr(rot), g, _ptr(smooth),
        _ptr(w_packed), N, _ptr(w_scale), _dt(w_scale), w_scale_group, _ptr(bias),
        _ptr(proj_down), _ptr(proj_up), rank, _ptr(out), _DT[out.dtype], _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(dev))
    _check(rc, "w4a4_linear")
    return out.view(*lead, N)
