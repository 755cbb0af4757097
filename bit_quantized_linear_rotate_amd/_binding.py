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
    "w8a8_rotate_quant_rowwise": ([_vp, ctypes.c_int, _i64, _i64, _i64, _i64, _vp, _i32, _vp, _vp,
                                   _vp, _vp, _vp], ctypes.c_int),
    "w8a8_gemm_from_codes": ([_vp, _vp, _i64, _i64, _vp, _i64, _vp, ctypes.c_int, _vp, ctypes.c_int,
                              _vp, ctypes.c_int, _vp, _sz, _vp], ctypes.c_int),
    "w8a8_gemm_workspace_size": ([_i64, _i64, _i64], _sz),
    "w8a8_linear": ([_vp, ctypes.c_int, _i64, _i64, _i64, _i64, _vp, _i32, _vp, _vp, _i64, _vp,
                     ctypes.c_int, _vp, _vp, ctypes.c_int, _vp, _sz, _vp], ctypes.c_int),
    "w8a8_linear_workspace_size": ([_i64, _i64, _i64], _sz),
    "w8a8_rotate_quant_plan": ([_vp, ctypes.c_int, _i64, _i64, _i64, _i64, _vp, _i32, _vp, _vp, _vp,
                                ctypes.POINTER(ctypes.c_int)], ctypes.c_int),
    "w8a8_gemm_plan": ([_vp, _i64, _i64, _vp, _i64, _vp, ctypes.POINTER(ctypes.c_int)], ctypes.c_int),
    "w4a4_rotate_quant_hadamard": ([_vp, ctypes.c_int, _i64, _i64, _i64, _i64, _i32, _vp, _vp, _vp,
                                    _i32, _vp, _vp, _vp, _vp], ctypes.c_int),
    "w4a4_rotate_quant_hadamard_plan": ([_vp, ctypes.c_int, _i64, _i64, _i64, _i64, _i32, _vp, _i32,
                                         _vp, _vp, ctypes.POINTER(ctypes.c_int)], ctypes.c_int),
    "w4a4_linear_hadamard": ([_vp, ctypes.c_int, _i64, _i64, _i64, _i64, _i32, _vp, _vp, _vp, _vp,
                              _i64, _vp, ctypes.c_int, _i32, _vp, _vp, _vp, _i32, _vp, ctypes.c_int,
                              _vp, _sz, _vp], ctypes.c_int),
    "w8a8_linear_hadamard": ([_vp, ctypes.c_int, _i64, _i64, _i64, _i64, _i32, _vp, _vp, _vp, _vp,
                              _i64, _vp, ctypes.c_int, _vp, _vp, ctypes.c_int, _vp, _sz, _vp],
                             ctypes.c_int),
    "w4a4_svdquant_workspace_size": ([_i64, _i64, _i64, _i32, _i32, _i32], _sz),
    "w4a4_quantize_svdquant": ([_vp, ctypes.c_int, _i64, _i64, _i64, _i64, _vp, _i32, _i32, _vp, _vp, _vp],
                               ctypes.c_int),
    "w4a4_gemm_svdquant": ([_vp, _vp, _i32, _i32, _i64, _i64, _vp, _i64, _vp, ctypes.c_int, _i32, _vp,
                            ctypes.c_int, _vp, _vp, ctypes.c_int, _i32, _vp, ctypes.c_int, _vp, _sz, _vp],
                           ctypes.c_int),
    "w4a4_linear_svdquant": ([_vp, ctypes.c_int, _i64, _i64, _i64, _i64, _vp, _i32, _i32, _vp, _i64, _vp,
                              ctypes.c_int, _i32, _vp, _vp, _vp, _i32, _vp, ctypes.c_int, _vp, _sz, _vp],
                             ctypes.c_int),
    "w4a4_linear_svdquant_grouped": ([_vp, ctypes.c_int, _i64, _i64, _i64, _i64, _vp, _i32, _i32, _vp, _i32,
                                      _i32, _vp, _vp, _vp, ctypes.c_int, _i32, _vp, _vp, _vp, ctypes.c_int,
                                      _vp, _sz, _vp], ctypes.c_int),
    "w4a4_codes_to_bf6": ([_vp, _i64, _i64, _vp, _vp], ctypes.c_int),
    "w4a4_pack_weights_bf6": ([_vp, _i64, _i64, _vp, _vp], ctypes.c_int),
    "w4a4_gemm_bf6": ([_vp, _vp, _i64, _i64, _vp, _i64, _vp, ctypes.c_int, _vp, ctypes.c_int, _vp, ctypes.c_int,
                       _vp], ctypes.c_int),
    "w4a4_linear_bf6_workspace_size": ([_i64, _i64], _sz),
    "w4a4_linear_bf6": ([_vp, ctypes.c_int, _i64, _i64, _i64, _i64, _vp, _i32, _vp, _vp, _i64, _vp, ctypes.c_int,
                         _vp, _vp, ctypes.c_int, _vp, _sz, _vp], ctypes.c_int),
    "w4a4_linear_noalloc": ([_vp, ctypes.c_int, _i64, _i64, _i64, _i64, _vp, _i32, _vp, _vp, _i64,
                             _vp, ctypes.c_int, _i32, _vp, _vp, _vp, _i32, _vp, ctypes.c_int, _vp],
                            ctypes.c_int),
    "w4a4_int32_guard": ([_i64, ctypes.POINTER(_i64)], ctypes.c_int),
    "w4a4_rotate_quant_plan": ([_vp, ctypes.c_int, _i64, _i64, _i64, _i64, _vp, _i32, _vp, _vp, _vp,
                                ctypes.POINTER(ctypes.c_int)], ctypes.c_int),
    "w4a4_gemm_plan": ([_vp, _i64, _i64, _vp, _i64, _i32, ctypes.c_int, _vp, _i64, _vp,
                        ctypes.POINTER(ctypes.c_int)], ctypes.c_int),
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


def _need(t, name: str, shape=None, dtypes=None, contiguous: bool = True):
    """Layout check of one tensor argument (shape, dtype, contiguity).  The
    device is checked afterwards, for every argument at once, so that a layout
    error is reported before any device access."""
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch.Tensor, got {type(t).__name__}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if dtypes is not None and t.dtype not in dtypes:
        names = "/".join(str(d).replace("torch.", "") for d in dtypes)
        raise ValueError(f"{name} has dtype {t.dtype}, expected {names}")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _same_device(ref: torch.Tensor, **tensors):
    """Every tensor on the CUDA (HIP) device of `ref`."""
    if ref.device.type != "cuda":
        raise ValueError(f"tensors must be on a CUDA (HIP) device, got {ref.device}")
    for name, t in tensors.items():
        if t is not None and t.device != ref.device:
            raise ValueError(f"{name} is on {t.device}, expected {ref.device}")


_FLOAT = (torch.float32, torch.float16, torch.bfloat16)


def _rot_arg(rot: Optional[torch.Tensor], g: int):
    if rot is None:
        return None, 0
    _need(rot, "rot", (g, g), (torch.float32,))
    return rot, g


def _wscale_shape(w_scale_group: int, K: int, N: int):
    if w_scale_group == 0:
        return (N,)
    if w_scale_group == 64:
        return (K // 64, N)
    raise ValueError(f"w_scale_group must be 0 or 64, got {w_scale_group}")


def w4a4_int32_guard(K: int):
    """(needs_chunking, k_chunk) for a K-long INT32 accumulation."""
    c = _i64(0)
    need = lib().w4a4_int32_guard(K, ctypes.byref(c))
    return bool(need), int(c.value)


def w4a4_linear_workspace_size(M: int, K: int, N: int, rank: int = 0) -> int:
    return int(lib().w4a4_linear_workspace_size(M, K, N, rank))


def w4a4_gemm_workspace_size(M: int, N: int, K: int, k_chunk: int = 0) -> int:
    return int(lib().w4a4_gemm_workspace_size(M, N, K, k_chunk))


# kernel names of the plan queries (include/w4a4.h)
RQ_KERNELS = {0: "generic", 1: "mfma_lds", 2: "reg", 3: "wave", 4: "colmajor", 5: "g256", 6: "row"}
GEMM_KERNELS = {0: "tile128", 1: "tile128_splitk", 2: "ring3", 3: "skinny", 4: "pingpong"}
_ALIGNED = 1 << 12   # stands for a buffer the binding allocates (torch aligns to >= 256 bytes)


def w4a4_rotate_quant_plan(x: torch.Tensor, rot: Optional[torch.Tensor], g: int,
                           smooth: Optional[torch.Tensor] = None,
                           return_rotated: bool = False) -> str:
    """Name of the rotate-quant kernel w4a4_rotate_quant_rowwise would launch
    for these arguments (host-only; nothing runs)."""
    x2 = _as_2d(x)
    M, K = x2.shape
    rot, g = _rot_arg(rot, g)
    k = ctypes.c_int(-1)
    rc = lib().w4a4_rotate_quant_plan(_ptr(x2), _dt(x2), M, K, x2.stride(0), x2.stride(1),
                                      _ptr(rot), g, _ptr(smooth), _ALIGNED,
                                      _ALIGNED if return_rotated else None, ctypes.byref(k))
    _check(rc, "w4a4_rotate_quant_plan")
    return RQ_KERNELS.get(k.value, "none")


def w4a4_gemm_plan(M: int, K: int, N: int, w_scale_group: int = 0, lowrank: bool = False,
                   return_acc: bool = False, k_chunk: int = 0) -> str:
    """Name of the GEMM kernel w4a4_gemm_from_codes (or w4a4_linear) would
    launch for operands the binding allocates (host-only; nothing runs)."""
    k = ctypes.c_int(-1)
    rc = lib().w4a4_gemm_plan(_ALIGNED, M, K, _ALIGNED, N, w_scale_group, int(lowrank),
                              _ALIGNED if return_acc else None, k_chunk, _ALIGNED, ctypes.byref(k))
    _check(rc, "w4a4_gemm_plan")
    return GEMM_KERNELS.get(k.value, "none")


def w4a4_device_supported() -> bool:
    return lib().w4a4_device_supported() == OK


def w4a4_rotate_quant_rowwise(x: torch.Tensor, rot: Optional[torch.Tensor], g: int,
                              smooth: Optional[torch.Tensor] = None,
                              return_rotated: bool = False):
    """Rotate + quantize rows of x (..., K).  Returns (codes int8 (M, K),
    scales fp32 (M,)) and, if requested, the rotated values (M, K) in x.dtype."""
    x2 = _as_2d(_need(x, "x", contiguous=False))
    M, K = x2.shape
    _dt(x2)
    rot, g = _rot_arg(rot, g)
    if smooth is not None:
        _need(smooth, "smooth", (K,), (x2.dtype,))
    _same_device(x2, rot=rot, smooth=smooth)
    dev = x2.device
    codes = torch.empty((M, K), dtype=torch.int8, device=dev)
    scales = torch.empty((M,), dtype=torch.float32, device=dev)
    rotated = torch.empty((M, K), dtype=x2.dtype, device=dev) if return_rotated else None
    rc = lib().w4a4_rotate_quant_rowwise(
        _ptr(x2), _dt(x2), M, K, x2.stride(0), x2.stride(1), _ptr(rot), g, _ptr(smooth),
        _ptr(codes), _ptr(scales), _ptr(rotated), _stream(dev))
    _check(rc, "w4a4_rotate_quant_rowwise")
    return (codes, scales, rotated) if return_rotated else (codes, scales)


def w4a4_lowrank_down(x: torch.Tensor, proj_down: torch.Tensor) -> torch.Tensor:
    x2 = _as_2d(_need(x, "x", contiguous=False))
    M, K = x2.shape
    _dt(x2)
    _need(proj_down, "proj_down", dtypes=(x2.dtype,))
    if proj_down.dim() != 2 or proj_down.shape[0] != K:
        raise ValueError(f"proj_down has shape {tuple(proj_down.shape)}, expected ({K}, rank)")
    R = proj_down.shape[1]
    _same_device(x2, proj_down=proj_down)
    lora = torch.empty((M, R), dtype=torch.float32, device=x2.device)
    rc = lib().w4a4_lowrank_down(_ptr(x2), _dt(x2), M, K, x2.stride(0), x2.stride(1),
                                 _ptr(proj_down), R, _ptr(lora), _stream(x2.device))
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
    _need(codes, "codes", dtypes=(torch.int8,))
    if codes.dim() != 2:
        raise ValueError(f"codes must be (M, K), got shape {tuple(codes.shape)}")
    M, K = codes.shape
    _need(w_packed, "w_packed", dtypes=(torch.uint8,))
    if w_packed.dim() != 2 or w_packed.shape[1] * 2 != K:
        raise ValueError(f"w_packed has shape {tuple(w_packed.shape)}, expected (N, {K // 2})")
    N = w_packed.shape[0]
    _need(scales, "scales", (M,), (torch.float32,))
    _need(w_scale, "w_scale", _wscale_shape(w_scale_group, K, N), _FLOAT)
    if bias is not None:
        _need(bias, "bias", (N,), _FLOAT)
    if (lora_act is None) != (proj_up is None):
        raise ValueError("lora_act and proj_up go together")
    if lora_act is not None:
        _need(lora_act, "lora_act", dtypes=(torch.float32,))
        if lora_act.dim() != 2 or lora_act.shape[0] != M:
            raise ValueError(f"lora_act has shape {tuple(lora_act.shape)}, expected ({M}, rank)")
        _need(proj_up, "proj_up", (N, lora_act.shape[1]), _FLOAT)
    if out_dtype not in _FLOAT:
        raise ValueError(f"out_dtype {out_dtype} is not float32/float16/bfloat16")
    _same_device(codes, scales=scales, w_packed=w_packed, w_scale=w_scale, bias=bias,
                 lora_act=lora_act, proj_up=proj_up)
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


def _linear_checks(x, rot, g, w_packed, w_scale, w_scale_group, bias, smooth, proj_down, proj_up,
                   out_dtype, out):
    """Validation shared by w4a4_linear and w4a4_linear_noalloc; returns
    (lead shape, x as (M, K), rot, g, N, rank, out dtype)."""
    lead = _need(x, "x", contiguous=False).shape[:-1]
    x2 = _as_2d(x)
    M, K = x2.shape
    _dt(x2)
    rot, g = _rot_arg(rot, g)
    _need(w_packed, "w_packed", dtypes=(torch.uint8,))
    if w_packed.dim() != 2 or w_packed.shape[1] * 2 != K:
        raise ValueError(f"w_packed has shape {tuple(w_packed.shape)}, expected (N, {K // 2})")
    N = w_packed.shape[0]
    _need(w_scale, "w_scale", _wscale_shape(w_scale_group, K, N), _FLOAT)
    # the layer reads bias, smooth and the low-rank factors in x's dtype
    if bias is not None:
        _need(bias, "bias", (N,), (x2.dtype,))
    if smooth is not None:
        _need(smooth, "smooth", (K,), (x2.dtype,))
    if (proj_down is None) != (proj_up is None):
        raise ValueError("proj_down and proj_up go together")
    rank = 0
    if proj_down is not None:
        _need(proj_down, "proj_down", dtypes=(x2.dtype,))
        if proj_down.dim() != 2 or proj_down.shape[0] != K:
            raise ValueError(f"proj_down has shape {tuple(proj_down.shape)}, expected ({K}, rank)")
        rank = proj_down.shape[1]
        _need(proj_up, "proj_up", (N, rank), (x2.dtype,))
    out_dtype = out_dtype or (out.dtype if out is not None else x2.dtype)
    if out_dtype not in _FLOAT:
        raise ValueError(f"out_dtype {out_dtype} is not float32/float16/bfloat16")
    if out is not None:
        _need(out, "out", (M, N), (out_dtype,))
    return lead, x2, rot, g, N, rank, out_dtype


def w4a4_linear(x: torch.Tensor, rot: Optional[torch.Tensor], g: int, w_packed: torch.Tensor,
                w_scale: torch.Tensor, w_scale_group: int = 0,
                bias: Optional[torch.Tensor] = None, smooth: Optional[torch.Tensor] = None,
                proj_down: Optional[torch.Tensor] = None, proj_up: Optional[torch.Tensor] = None,
                out_dtype: Optional[torch.dtype] = None,
                workspace: Optional[torch.Tensor] = None,
                out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """The whole W4A4 linear: y = layer(x) of shape (..., N)."""
    lead, x2, rot, g, N, rank, out_dtype = _linear_checks(
        x, rot, g, w_packed, w_scale, w_scale_group, bias, smooth, proj_down, proj_up, out_dtype, out)
    M, K = x2.shape
    need = w4a4_linear_workspace_size(M, K, N, rank)
    if workspace is not None:
        _need(workspace, "workspace", dtypes=(torch.uint8,))
        if workspace.numel() < need:
            raise ValueError(f"workspace holds {workspace.numel()} bytes, need {need}")
    _same_device(x2, rot=rot, w_packed=w_packed, w_scale=w_scale, bias=bias, smooth=smooth,
                 proj_down=proj_down, proj_up=proj_up, out=out, workspace=workspace)
    dev = x2.device
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=dev)
    if workspace is None:
        workspace = torch.empty((max(need, 1),), dtype=torch.uint8, device=dev)
    rc = lib().w4a4_linear(
        _ptr(x2), _dt(x2), M, K, x2.stride(0), x2.stride(1), _ptr(rot), g, _ptr(smooth),
        _ptr(w_packed), N, _ptr(w_scale), _dt(w_scale), w_scale_group, _ptr(bias),
        _ptr(proj_down), _ptr(proj_up), rank, _ptr(out), _DT[out.dtype], _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(dev))
    _check(rc, "w4a4_linear")
    return out.view(*lead, N)


# size of the library's per-GPU scratch (W4A4_NOALLOC_SCRATCH_BYTES)
NOALLOC_SCRATCH_BYTES = 128 << 20


def w4a4_linear_noalloc(x: torch.Tensor, rot: Optional[torch.Tensor], g: int,
                        w_packed: torch.Tensor, w_scale: torch.Tensor, out: torch.Tensor,
                        w_scale_group: int = 0, bias: Optional[torch.Tensor] = None,
                        smooth: Optional[torch.Tensor] = None,
                        proj_down: Optional[torch.Tensor] = None,
                        proj_up: Optional[torch.Tensor] = None) -> torch.Tensor:
    """w4a4_linear without a workspace and without any allocation: the
    library's per-GPU scratch holds the intermediates (calls that overlap on
    one GPU race).  `out` (M, N) is required; layers needing more than
    NOALLOC_SCRATCH_BYTES of scratch are refused (ValueError)."""
    if not isinstance(out, torch.Tensor):
        raise ValueError("out must be a torch.Tensor (the no-allocation call allocates nothing)")
    lead, x2, rot, g, N, rank, out_dtype = _linear_checks(
        x, rot, g, w_packed, w_scale, w_scale_group, bias, smooth, proj_down, proj_up, None, out)
    M, K = x2.shape
    _same_device(x2, rot=rot, w_packed=w_packed, w_scale=w_scale, bias=bias, smooth=smooth,
                 proj_down=proj_down, proj_up=proj_up, out=out)
    rc = lib().w4a4_linear_noalloc(
        _ptr(x2), _dt(x2), M, K, x2.stride(0), x2.stride(1), _ptr(rot), g, _ptr(smooth),
        _ptr(w_packed), N, _ptr(w_scale), _dt(w_scale), w_scale_group, _ptr(bias),
        _ptr(proj_down), _ptr(proj_up), rank, _ptr(out), _DT[out.dtype], _stream(x2.device))
    _check(rc, "w4a4_linear_noalloc")
    return out.view(*lead, N)


# ---- INT8 mode (qmax = 127) and the dynamic INT8 linear --------------------

def w8a8_rotate_quant_rowwise(x: torch.Tensor, rot: Optional[torch.Tensor], g: int,
                              smooth: Optional[torch.Tensor] = None,
                              return_rotated: bool = False):
    """Rotate + per-row INT8 quantization (codes in [-127, 127]).  Returns
    (codes int8 (M, K), scales fp32 (M,)) and, if requested, the rotated
    values (M, K) in x.dtype."""
    x2 = _as_2d(_need(x, "x", contiguous=False))
    M, K = x2.shape
    _dt(x2)
    rot, g = _rot_arg(rot, g)
    if smooth is not None:
        _need(smooth, "smooth", (K,), (x2.dtype,))
    _same_device(x2, rot=rot, smooth=smooth)
    dev = x2.device
    codes = torch.empty((M, K), dtype=torch.int8, device=dev)
    scales = torch.empty((M,), dtype=torch.float32, device=dev)
    rotated = torch.empty((M, K), dtype=x2.dtype, device=dev) if return_rotated else None
    rc = lib().w8a8_rotate_quant_rowwise(
        _ptr(x2), _dt(x2), M, K, x2.stride(0), x2.stride(1), _ptr(rot), g, _ptr(smooth),
        _ptr(codes), _ptr(scales), _ptr(rotated), _stream(dev))
    _check(rc, "w8a8_rotate_quant_rowwise")
    return (codes, scales, rotated) if return_rotated else (codes, scales)


def w8a8_rotate_quant_plan(x: torch.Tensor, rot: Optional[torch.Tensor], g: int,
                           smooth: Optional[torch.Tensor] = None,
                           return_rotated: bool = False) -> str:
    """Name of the kernel w8a8_rotate_quant_rowwise would launch (host-only)."""
    x2 = _as_2d(x)
    M, K = x2.shape
    rot, g = _rot_arg(rot, g)
    k = ctypes.c_int(-1)
    rc = lib().w8a8_rotate_quant_plan(_ptr(x2), _dt(x2), M, K, x2.stride(0), x2.stride(1),
                                      _ptr(rot), g, _ptr(smooth), _ALIGNED,
                                      _ALIGNED if return_rotated else None, ctypes.byref(k))
    _check(rc, "w8a8_rotate_quant_plan")
    return RQ_KERNELS.get(k.value, "none")


def w8a8_gemm_workspace_size(M: int, N: int, K: int) -> int:
    return int(lib().w8a8_gemm_workspace_size(M, N, K))


def w8a8_gemm_plan(M: int, K: int, N: int) -> str:
    """Name of the GEMM kernel w8a8_gemm_from_codes (or w8a8_linear) would
    launch for operands the binding allocates (host-only; nothing runs)."""
    k = ctypes.c_int(-1)
    rc = lib().w8a8_gemm_plan(_ALIGNED, M, K, _ALIGNED, N, _ALIGNED, ctypes.byref(k))
    _check(rc, "w8a8_gemm_plan")
    return GEMM_KERNELS.get(k.value, "none")


def w8a8_linear_workspace_size(M: int, K: int, N: int) -> int:
    return int(lib().w8a8_linear_workspace_size(M, K, N))


def w8a8_gemm_from_codes(codes: torch.Tensor, scales: torch.Tensor, w: torch.Tensor,
                         w_scale: torch.Tensor, bias: Optional[torch.Tensor] = None,
                         out_dtype: torch.dtype = torch.bfloat16) -> torch.Tensor:
    """INT8-code x INT8-weight GEMM (w: (N, K) int8) with the E-B epilogue."""
    _need(codes, "codes", dtypes=(torch.int8,))
    if codes.dim() != 2:
        raise ValueError(f"codes must be (M, K), got shape {tuple(codes.shape)}")
    M, K = codes.shape
    _need(w, "w", dtypes=(torch.int8,))
    if w.dim() != 2 or w.shape[1] != K:
        raise ValueError(f"w has shape {tuple(w.shape)}, expected (N, {K})")
    N = w.shape[0]
    _need(scales, "scales", (M,), (torch.float32,))
    _need(w_scale, "w_scale", (N,), _FLOAT)
    if bias is not None:
        _need(bias, "bias", (N,), _FLOAT)
    if out_dtype not in _FLOAT:
        raise ValueError(f"out_dtype {out_dtype} is not float32/float16/bfloat16")
    _same_device(codes, scales=scales, w=w, w_scale=w_scale, bias=bias)
    dev = codes.device
    out = torch.empty((M, N), dtype=out_dtype, device=dev)
    wsz = w8a8_gemm_workspace_size(M, N, K)
    ws = torch.empty((max(wsz, 1),), dtype=torch.uint8, device=dev) if wsz else None
    rc = lib().w8a8_gemm_from_codes(
        _ptr(codes), _ptr(scales), M, K, _ptr(w), N, _ptr(w_scale), _dt(w_scale), _ptr(bias),
        _dt(bias) if bias is not None else 0, _ptr(out), _DT[out_dtype], _ptr(ws), wsz, _stream(dev))
    _check(rc, "w8a8_gemm_from_codes")
    return out


def w8a8_linear(x: torch.Tensor, rot: Optional[torch.Tensor], g: int, w: torch.Tensor,
                w_scale: torch.Tensor, bias: Optional[torch.Tensor] = None,
                smooth: Optional[torch.Tensor] = None, out_dtype: Optional[torch.dtype] = None,
                workspace: Optional[torch.Tensor] = None,
                out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """The dynamic INT8 ConvRot linear: y = layer(x) of shape (..., N)."""
    lead = _need(x, "x", contiguous=False).shape[:-1]
    x2 = _as_2d(x)
    M, K = x2.shape
    _dt(x2)
    rot, g = _rot_arg(rot, g)
    _need(w, "w", dtypes=(torch.int8,))
    if w.dim() != 2 or w.shape[1] != K:
        raise ValueError(f"w has shape {tuple(w.shape)}, expected (N, {K})")
    N = w.shape[0]
    _need(w_scale, "w_scale", (N,), _FLOAT)
    if bias is not None:
        _need(bias, "bias", (N,), (x2.dtype,))
    if smooth is not None:
        _need(smooth, "smooth", (K,), (x2.dtype,))
    out_dtype = out_dtype or (out.dtype if out is not None else x2.dtype)
    if out_dtype not in _FLOAT:
        raise ValueError(f"out_dtype {out_dtype} is not float32/float16/bfloat16")
    if out is not None:
        _need(out, "out", (M, N), (out_dtype,))
    need = w8a8_linear_workspace_size(M, K, N)
    if workspace is not None:
        _need(workspace, "workspace", dtypes=(torch.uint8,))
        if workspace.numel() < need:
            raise ValueError(f"workspace holds {workspace.numel()} bytes, need {need}")
    _same_device(x2, rot=rot, w=w, w_scale=w_scale, bias=bias, smooth=smooth, out=out,
                 workspace=workspace)
    dev = x2.device
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=dev)
    if workspace is None:
        workspace = torch.empty((max(need, 1),), dtype=torch.uint8, device=dev)
    rc = lib().w8a8_linear(
        _ptr(x2), _dt(x2), M, K, x2.stride(0), x2.stride(1), _ptr(rot), g, _ptr(smooth), _ptr(w), N,
        _ptr(w_scale), _dt(w_scale), _ptr(bias), _ptr(out), _DT[out.dtype], _ptr(workspace),
        workspace.numel(), _stream(dev))
    _check(rc, "w8a8_linear")
    return out.view(*lead, N)


# ---- structured (Hadamard) rotation: the fast Walsh-Hadamard kernel --------

class Hadamard:
    """The rotation R = diag(sign_in) . H_g . diag(sign_out) / sqrt(g), given by
    its structure (H_g the Sylvester Hadamard matrix); sign_in / sign_out are
    int8 (g,) device tensors of +-1 or None (all +1).  The *_hadamard calls
    take it in place of a dense (g, g) rot."""

    def __init__(self, g: int, sign_in: Optional[torch.Tensor] = None,
                 sign_out: Optional[torch.Tensor] = None):
        if g not in (16, 32, 64, 128, 256):
            raise ValueError(f"g must be a power of two in [16, 256], got {g}")
        for name, s in (("sign_in", sign_in), ("sign_out", sign_out)):
            if s is not None:
                _need(s, name, (g,), (torch.int8,))
        self.g, self.sign_in, self.sign_out = g, sign_in, sign_out

    def dense(self) -> torch.Tensor:
        """The same R written out, fp32 (g, g) on the signs' device (CPU if
        none): what the dense calls take."""
        h = torch.ones((1, 1), dtype=torch.float64)
        while h.shape[0] < self.g:
            h = torch.cat([torch.cat([h, h], 1), torch.cat([h, -h], 1)], 0)
        dev = next((s.device for s in (self.sign_in, self.sign_out) if s is not None), torch.device("cpu"))
        h = h.to(dev)
        if self.sign_in is not None:
            h = h * torch.where(self.sign_in < 0, -1.0, 1.0).to(torch.float64)[:, None]
        if self.sign_out is not None:
            h = h * torch.where(self.sign_out < 0, -1.0, 1.0).to(torch.float64)[None, :]
        return (h / float(self.g) ** 0.5).to(torch.float32)


def _hadamard_arg(h) -> "Hadamard":
    if not isinstance(h, Hadamard):
        raise ValueError(f"expected a Hadamard rotation, got {type(h).__name__}")
    return h


def w4a4_rotate_quant_hadamard(x: torch.Tensor, h: Hadamard, qmax: int = 7,
                               smooth: Optional[torch.Tensor] = None,
                               return_rotated: bool = False):
    """Rotate + per-row quantization with a Hadamard rotation (fast
    Walsh-Hadamard transform), INT4 codes (qmax 7) or the INT8 mode (127).
    Returns (codes int8 (M, K), scales fp32 (M,)) and, if requested, the
    rotated values (M, K) in x.dtype."""
    h = _hadamard_arg(h)
    x2 = _as_2d(_need(x, "x", contiguous=False))
    M, K = x2.shape
    _dt(x2)
    if smooth is not None:
        _need(smooth, "smooth", (K,), (x2.dtype,))
    _same_device(x2, sign_in=h.sign_in, sign_out=h.sign_out, smooth=smooth)
    dev = x2.device
    codes = torch.empty((M, K), dtype=torch.int8, device=dev)
    scales = torch.empty((M,), dtype=torch.float32, device=dev)
    rotated = torch.empty((M, K), dtype=x2.dtype, device=dev) if return_rotated else None
    rc = lib().w4a4_rotate_quant_hadamard(
        _ptr(x2), _dt(x2), M, K, x2.stride(0), x2.stride(1), h.g, _ptr(h.sign_in), _ptr(h.sign_out),
        _ptr(smooth), qmax, _ptr(codes), _ptr(scales), _ptr(rotated), _stream(dev))
    _check(rc, "w4a4_rotate_quant_hadamard")
    return (codes, scales, rotated) if return_rotated else (codes, scales)


def w4a4_rotate_quant_hadamard_plan(x: torch.Tensor, g: int, qmax: int = 7,
                                    smooth: Optional[torch.Tensor] = None,
                                    return_rotated: bool = False) -> str:
    """"hadamard" (fast Walsh-Hadamard kernel) or "row" (the one-wave-per-row
    kernel with R built from the signs, g = 64 on many contiguous rows) for
    the kernel w4a4_rotate_quant_hadamard takes; raises W4A4Error
    (unsupported) when none does.  Host-only."""
    x2 = _as_2d(x)
    M, K = x2.shape
    k = ctypes.c_int(-1)
    rc = lib().w4a4_rotate_quant_hadamard_plan(
        _ptr(x2), _dt(x2), M, K, x2.stride(0), x2.stride(1), g, _ptr(smooth), qmax, _ALIGNED,
        _ALIGNED if return_rotated else None, ctypes.byref(k))
    _check(rc, "w4a4_rotate_quant_hadamard_plan")
    return {6: "row", 7: "hadamard"}.get(k.value, "none")


def w4a4_linear_hadamard(x: torch.Tensor, h: Hadamard, w_packed: torch.Tensor,
                         w_scale: torch.Tensor, w_scale_group: int = 0,
                         bias: Optional[torch.Tensor] = None, smooth: Optional[torch.Tensor] = None,
                         proj_down: Optional[torch.Tensor] = None,
                         proj_up: Optional[torch.Tensor] = None,
                         out_dtype: Optional[torch.dtype] = None,
                         workspace: Optional[torch.Tensor] = None,
                         out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """w4a4_linear with a Hadamard rotation (fast Walsh-Hadamard transform)."""
    h = _hadamard_arg(h)
    lead, x2, _, _, N, rank, out_dtype = _linear_checks(
        x, None, h.g, w_packed, w_scale, w_scale_group, bias, smooth, proj_down, proj_up, out_dtype, out)
    M, K = x2.shape
    need = w4a4_linear_workspace_size(M, K, N, rank)
    if workspace is not None:
        _need(workspace, "workspace", dtypes=(torch.uint8,))
        if workspace.numel() < need:
            raise ValueError(f"workspace holds {workspace.numel()} bytes, need {need}")
    _same_device(x2, sign_in=h.sign_in, sign_out=h.sign_out, w_packed=w_packed, w_scale=w_scale,
                 bias=bias, smooth=smooth, proj_down=proj_down, proj_up=proj_up, out=out,
                 workspace=workspace)
    dev = x2.device
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=dev)
    if workspace is None:
        workspace = torch.empty((max(need, 1),), dtype=torch.uint8, device=dev)
    rc = lib().w4a4_linear_hadamard(
        _ptr(x2), _dt(x2), M, K, x2.stride(0), x2.stride(1), h.g, _ptr(h.sign_in), _ptr(h.sign_out),
        _ptr(smooth), _ptr(w_packed), N, _ptr(w_scale), _dt(w_scale), w_scale_group, _ptr(bias),
        _ptr(proj_down), _ptr(proj_up), rank, _ptr(out), _DT[out.dtype], _ptr(workspace),
        workspace.numel(), _stream(dev))
    _check(rc, "w4a4_linear_hadamard")
    return out.view(*lead, N)


def w8a8_linear_hadamard(x: torch.Tensor, h: Hadamard, w: torch.Tensor, w_scale: torch.Tensor,
                         bias: Optional[torch.Tensor] = None, smooth: Optional[torch.Tensor] = None,
                         out_dtype: Optional[torch.dtype] = None,
                         workspace: Optional[torch.Tensor] = None,
                         out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """The dynamic INT8 linear with a Hadamard rotation."""
    h = _hadamard_arg(h)
    lead = _need(x, "x", contiguous=False).shape[:-1]
    x2 = _as_2d(x)
    M, K = x2.shape
    _dt(x2)
    _need(w, "w", dtypes=(torch.int8,))
    if w.dim() != 2 or w.shape[1] != K:
        raise ValueError(f"w has shape {tuple(w.shape)}, expected (N, {K})")
    N = w.shape[0]
    _need(w_scale, "w_scale", (N,), _FLOAT)
    if bias is not None:
        _need(bias, "bias", (N,), (x2.dtype,))
    if smooth is not None:
        _need(smooth, "smooth", (K,), (x2.dtype,))
    out_dtype = out_dtype or (out.dtype if out is not None else x2.dtype)
    if out_dtype not in _FLOAT:
        raise ValueError(f"out_dtype {out_dtype} is not float32/float16/bfloat16")
    if out is not None:
        _need(out, "out", (M, N), (out_dtype,))
    need = w8a8_linear_workspace_size(M, K, N)
    if workspace is not None:
        _need(workspace, "workspace", dtypes=(torch.uint8,))
        if workspace.numel() < need:
            raise ValueError(f"workspace holds {workspace.numel()} bytes, need {need}")
    _same_device(x2, sign_in=h.sign_in, sign_out=h.sign_out, w=w, w_scale=w_scale, bias=bias,
                 smooth=smooth, out=out, workspace=workspace)
    dev = x2.device
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=dev)
    if workspace is None:
        workspace = torch.empty((max(need, 1),), dtype=torch.uint8, device=dev)
    rc = lib().w8a8_linear_hadamard(
        _ptr(x2), _dt(x2), M, K, x2.stride(0), x2.stride(1), h.g, _ptr(h.sign_in), _ptr(h.sign_out),
        _ptr(smooth), _ptr(w), N, _ptr(w_scale), _dt(w_scale), _ptr(bias), _ptr(out), _DT[out.dtype],
        _ptr(workspace), workspace.numel(), _stream(dev))
    _check(rc, "w8a8_linear_hadamard")
    return out.view(*lead, N)


# ---- the SVDQuant variant ------------------------------------------------------

def w4a4_svdquant_workspace_size(M: int, K: int, N: int, rank: int = 0, act_group: int = 64,
                                 act_unsigned: bool = False) -> int:
    return int(lib().w4a4_svdquant_workspace_size(M, K, N, rank, act_group, int(bool(act_unsigned))))


def _svd_act(x, smooth, act_group):
    x2 = _as_2d(_need(x, "x", contiguous=False))
    M, K = x2.shape
    _dt(x2)
    if act_group not in (0, 64):
        raise ValueError(f"act_group must be 0 or 64, got {act_group}")
    if smooth is not None:
        _need(smooth, "smooth", (K,), (x2.dtype,))
    return x2, M, K


def w4a4_quantize_svdquant(x: torch.Tensor, smooth: Optional[torch.Tensor] = None,
                           act_unsigned: bool = False, act_group: int = 64):
    """SVDQuant activation quantizer: (codes int8 (M, K), scales fp32 (M, K/64)
    or (M,)); act_unsigned shifts by 0.171875 onto the unsigned grid [0, 15]."""
    x2, M, K = _svd_act(x, smooth, act_group)
    _same_device(x2, smooth=smooth)
    dev = x2.device
    codes = torch.empty((M, K), dtype=torch.int8, device=dev)
    scales = torch.empty((M, K // 64) if act_group else (M,), dtype=torch.float32, device=dev)
    rc = lib().w4a4_quantize_svdquant(_ptr(x2), _dt(x2), M, K, x2.stride(0), x2.stride(1), _ptr(smooth),
                                      int(bool(act_unsigned)), act_group, _ptr(codes), _ptr(scales), _stream(dev))
    _check(rc, "w4a4_quantize_svdquant")
    return codes, scales


def w4a4_gemm_svdquant(codes: torch.Tensor, scales: torch.Tensor, w_packed: torch.Tensor,
                       w_scale: torch.Tensor, act_group: int = 64, act_unsigned: bool = False,
                       w_scale_group: int = 64, bias: Optional[torch.Tensor] = None,
                       lora_act: Optional[torch.Tensor] = None, proj_up: Optional[torch.Tensor] = None,
                       out_dtype: torch.dtype = torch.bfloat16) -> torch.Tensor:
    """The SVDQuant GEMM and epilogue on quantized activations."""
    _need(codes, "codes", dtypes=(torch.int8,))
    if codes.dim() != 2:
        raise ValueError(f"codes must be (M, K), got shape {tuple(codes.shape)}")
    M, K = codes.shape
    if act_group not in (0, 64):
        raise ValueError(f"act_group must be 0 or 64, got {act_group}")
    _need(scales, "scales", (M, K // 64) if act_group else (M,), (torch.float32,))
    _need(w_packed, "w_packed", dtypes=(torch.uint8,))
    if w_packed.dim() != 2 or w_packed.shape[1] * 2 != K:
        raise ValueError(f"w_packed has shape {tuple(w_packed.shape)}, expected (N, {K // 2})")
    N = w_packed.shape[0]
    _need(w_scale, "w_scale", _wscale_shape(w_scale_group, K, N), _FLOAT)
    if bias is not None:
        _need(bias, "bias", (N,), _FLOAT)
    rank = 0
    if (lora_act is None) != (proj_up is None):
        raise ValueError("lora_act and proj_up go together")
    if lora_act is not None:
        _need(lora_act, "lora_act", dtypes=(torch.float32,))
        rank = lora_act.shape[1]
        _need(proj_up, "proj_up", (N, rank), _FLOAT)
    if out_dtype not in _FLOAT:
        raise ValueError(f"out_dtype {out_dtype} is not float32/float16/bfloat16")
    _same_device(codes, scales=scales, w_packed=w_packed, w_scale=w_scale, bias=bias, lora_act=lora_act,
                 proj_up=proj_up)
    dev = codes.device
    out = torch.empty((M, N), dtype=out_dtype, device=dev)
    need = w4a4_svdquant_workspace_size(M, K, N, 0, act_group, act_unsigned) - \
        w4a4_svdquant_workspace_size(M, K, 0, 0, act_group, act_unsigned) if w_scale_group == 0 else 0
    ws = torch.empty((need,), dtype=torch.uint8, device=dev) if need > 0 else None
    rc = lib().w4a4_gemm_svdquant(
        _ptr(codes), _ptr(scales), act_group, int(bool(act_unsigned)), M, K, _ptr(w_packed), N, _ptr(w_scale),
        _dt(w_scale), w_scale_group, _ptr(bias), _dt(bias) if bias is not None else 0, _ptr(lora_act),
        _ptr(proj_up), _dt(proj_up) if proj_up is not None else 0, rank, _ptr(out), _DT[out_dtype], _ptr(ws),
        need, _stream(dev))
    _check(rc, "w4a4_gemm_svdquant")
    return out


def w4a4_linear_svdquant_grouped(x: torch.Tensor, projections, smooth: Optional[torch.Tensor] = None,
                                 proj_down: Optional[torch.Tensor] = None, act_unsigned: bool = False,
                                 act_group: int = 64, w_scale_group: int = 64,
                                 out_dtype: Optional[torch.dtype] = None,
                                 workspace: Optional[torch.Tensor] = None):
    """Split projections of one activation sharing smoothing and proj_down
    (e.g. Q/K/V): quantized and projected down once, then one GEMM each.
    ``projections``: sequence of dicts with w_packed, w_scale and optional bias
    and proj_up.  Returns one (..., N_i) output per projection."""
    lead = _need(x, "x", contiguous=False).shape[:-1]
    x2, M, K = _svd_act(x, smooth, act_group)
    out_dtype = out_dtype or x2.dtype
    if out_dtype not in _FLOAT:
        raise ValueError(f"out_dtype {out_dtype} is not float32/float16/bfloat16")
    projections = list(projections)
    if not projections:
        return ()
    rank = 0
    if proj_down is not None:
        _need(proj_down, "proj_down", dtypes=(x2.dtype,))
        if proj_down.dim() != 2 or proj_down.shape[0] != K:
            raise ValueError(f"proj_down has shape {tuple(proj_down.shape)}, expected ({K}, R)")
        rank = proj_down.shape[1]
    ws_dtype = None
    Ns, outs = [], []
    for i, p in enumerate(projections):
        wp, sw = p["w_packed"], p["w_scale"]
        _need(wp, f"w_packed[{i}]", dtypes=(torch.uint8,))
        if wp.dim() != 2 or wp.shape[1] * 2 != K:
            raise ValueError(f"w_packed[{i}] has shape {tuple(wp.shape)}, expected (N, {K // 2})")
        N = wp.shape[0]
        _need(sw, f"w_scale[{i}]", _wscale_shape(w_scale_group, K, N), _FLOAT)
        if ws_dtype is None:
            ws_dtype = sw.dtype
        elif sw.dtype != ws_dtype:
            raise ValueError("every projection's w_scale must have the same dtype")
        if p.get("bias") is not None:
            _need(p["bias"], f"bias[{i}]", (N,), (x2.dtype,))
        up = p.get("proj_up")
        if (up is None) != (proj_down is None):
            raise ValueError(f"projection {i}: proj_down and proj_up go together")
        if up is not None:
            _need(up, f"proj_up[{i}]", (N, rank), (x2.dtype,))
        _same_device(x2, w_packed=wp, w_scale=sw, bias=p.get("bias"), proj_up=up)
        Ns.append(N)
        outs.append(torch.empty((M, N), dtype=out_dtype, device=x2.device))
    _same_device(x2, smooth=smooth, proj_down=proj_down, workspace=workspace)
    need = w4a4_svdquant_workspace_size(M, K, max(Ns), rank, act_group, act_unsigned)
    if workspace is not None:
        _need(workspace, "workspace", dtypes=(torch.uint8,))
        if workspace.numel() < need:
            raise ValueError(f"workspace holds {workspace.numel()} bytes, need {need}")
    else:
        workspace = torch.empty((max(need, 1),), dtype=torch.uint8, device=x2.device)
    n = len(projections)
    P = ctypes.c_void_p * n
    wps = P(*[p["w_packed"].data_ptr() for p in projections])
    sws = P(*[p["w_scale"].data_ptr() for p in projections])
    bs = P(*[(p["bias"].data_ptr() if p.get("bias") is not None else None) for p in projections])
    ups = P(*[(p["proj_up"].data_ptr() if p.get("proj_up") is not None else None) for p in projections])
    os_ = P(*[o.data_ptr() for o in outs])
    Narr = (ctypes.c_int64 * n)(*Ns)
    rc = lib().w4a4_linear_svdquant_grouped(
        _ptr(x2), _dt(x2), M, K, x2.stride(0), x2.stride(1), _ptr(smooth), int(bool(act_unsigned)), act_group,
        _ptr(proj_down), rank, n, wps, Narr, sws, _DT[ws_dtype], w_scale_group, bs, ups, os_, _DT[out_dtype],
        _ptr(workspace), workspace.numel(), _stream(x2.device))
    _check(rc, "w4a4_linear_svdquant_grouped")
    return tuple(o.view(*lead, N) for o, N in zip(outs, Ns))


def w4a4_linear_svdquant(x: torch.Tensor, w_packed: torch.Tensor, w_scale: torch.Tensor,
                         w_scale_group: int = 64, bias: Optional[torch.Tensor] = None,
                         smooth: Optional[torch.Tensor] = None, proj_down: Optional[torch.Tensor] = None,
                         proj_up: Optional[torch.Tensor] = None, act_unsigned: bool = False,
                         act_group: int = 64, out_dtype: Optional[torch.dtype] = None,
                         workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """The SVDQuant W4A4 layer (one projection)."""
    return w4a4_linear_svdquant_grouped(
        x, [dict(w_packed=w_packed, w_scale=w_scale, bias=bias, proj_up=proj_up)], smooth=smooth,
        proj_down=proj_down, act_unsigned=act_unsigned, act_group=act_group, w_scale_group=w_scale_group,
        out_dtype=out_dtype, workspace=workspace)[0]


def fuse_linear_weights(projections, w_scale_group: int = 64):
    """Runtime N-fusion of split projections that share their activation
    side: concatenates w_packed (N_i, K/2), w_scale (along N), bias (zeros
    where a projection has none) and proj_up along N, so that the projections
    run as one wider layer.  Returns (fused dict, out_features); split the
    fused output with ``torch.split(out, out_features, dim=-1)``.  Weight
    preparation, done once; nothing of the layer's arithmetic happens here."""
    projections = list(projections)
    if not projections:
        raise ValueError("expected at least one projection")
    feats = tuple(int(p["w_packed"].shape[0]) for p in projections)
    wp = torch.cat([p["w_packed"] for p in projections], dim=0).contiguous()
    sw = torch.cat([p["w_scale"] for p in projections], dim=1 if w_scale_group else 0).contiguous()
    fused = dict(w_packed=wp, w_scale=sw, bias=None, proj_up=None)
    if any(p.get("bias") is not None for p in projections):
        ref = next(p["bias"] for p in projections if p.get("bias") is not None)
        fused["bias"] = torch.cat([p["bias"] if p.get("bias") is not None else
                                   torch.zeros(n, dtype=ref.dtype, device=ref.device)
                                   for p, n in zip(projections, feats)]).contiguous()
    ups = [p.get("proj_up") for p in projections]
    if any(u is not None for u in ups):
        if any(u is None for u in ups):
            raise ValueError("either every projection has proj_up or none")
        fused["proj_up"] = torch.cat(ups, dim=0).contiguous()
    return fused, feats


# ---- FP6 (bf6 e3m2) GEMM path ---------------------------------------------------

def w4a4_codes_to_bf6(codes: torch.Tensor) -> torch.Tensor:
    """int8 codes (M, K) in [-8, 8] -> bf6 blocks (M, K) uint8."""
    _need(codes, "codes", dtypes=(torch.int8,))
    if codes.dim() != 2:
        raise ValueError(f"codes must be (M, K), got shape {tuple(codes.shape)}")
    M, K = codes.shape
    out = torch.empty((M, K), dtype=torch.uint8, device=codes.device)
    _same_device(codes)
    rc = lib().w4a4_codes_to_bf6(_ptr(codes), M, K, _ptr(out), _stream(codes.device))
    _check(rc, "w4a4_codes_to_bf6")
    return out


def w4a4_pack_weights_bf6(w_packed: torch.Tensor) -> torch.Tensor:
    """Packed INT4 weights (N, K/2) -> bf6 blocks (N, K) uint8 (once per layer)."""
    _need(w_packed, "w_packed", dtypes=(torch.uint8,))
    if w_packed.dim() != 2:
        raise ValueError(f"w_packed must be (N, K/2), got shape {tuple(w_packed.shape)}")
    N, K = w_packed.shape[0], 2 * w_packed.shape[1]
    out = torch.empty((N, K), dtype=torch.uint8, device=w_packed.device)
    _same_device(w_packed)
    rc = lib().w4a4_pack_weights_bf6(_ptr(w_packed), N, K, _ptr(out), _stream(w_packed.device))
    _check(rc, "w4a4_pack_weights_bf6")
    return out


def w4a4_gemm_bf6(codes6: torch.Tensor, scales: torch.Tensor, w6: torch.Tensor, w_scale: torch.Tensor,
                  bias: Optional[torch.Tensor] = None, out_dtype: torch.dtype = torch.bfloat16) -> torch.Tensor:
    """The W4A4 GEMM + epilogue (per-channel weight scales) on the FP6 matrix
    cores, from bf6 codes (M, K) and bf6 weights (N, K)."""
    _need(codes6, "codes6", dtypes=(torch.uint8,))
    _need(w6, "w6", dtypes=(torch.uint8,))
    if codes6.dim() != 2 or w6.dim() != 2 or w6.shape[1] != codes6.shape[1]:
        raise ValueError(f"codes6 {tuple(codes6.shape)} and w6 {tuple(w6.shape)} must be (M, K) and (N, K)")
    M, K = codes6.shape
    N = w6.shape[0]
    _need(scales, "scales", (M,), (torch.float32,))
    _need(w_scale, "w_scale", (N,), _FLOAT)
    if bias is not None:
        _need(bias, "bias", (N,), _FLOAT)
    if out_dtype not in _FLOAT:
        raise ValueError(f"out_dtype {out_dtype} is not float32/float16/bfloat16")
    _same_device(codes6, scales=scales, w6=w6, w_scale=w_scale, bias=bias)
    out = torch.empty((M, N), dtype=out_dtype, device=codes6.device)
    rc = lib().w4a4_gemm_bf6(_ptr(codes6), _ptr(scales), M, K, _ptr(w6), N, _ptr(w_scale), _dt(w_scale),
                             _ptr(bias), _dt(bias) if bias is not None else 0, _ptr(out), _DT[out_dtype],
                             _stream(codes6.device))
    _check(rc, "w4a4_gemm_bf6")
    return out


def w4a4_linear_bf6_workspace_size(M: int, K: int) -> int:
    return int(lib().w4a4_linear_bf6_workspace_size(M, K))


def w4a4_linear_bf6(x: torch.Tensor, rot: Optional[torch.Tensor], g: int, w6: torch.Tensor,
                    w_scale: torch.Tensor, bias: Optional[torch.Tensor] = None,
                    smooth: Optional[torch.Tensor] = None, out_dtype: Optional[torch.dtype] = None,
                    workspace: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """The W4A4 linear (per-channel weight scales) with the GEMM on the FP6
    matrix cores; w6 from w4a4_pack_weights_bf6."""
    lead = _need(x, "x", contiguous=False).shape[:-1]
    x2 = _as_2d(x)
    M, K = x2.shape
    _dt(x2)
    rot, g = _rot_arg(rot, g)
    _need(w6, "w6", dtypes=(torch.uint8,))
    if w6.dim() != 2 or w6.shape[1] != K:
        raise ValueError(f"w6 has shape {tuple(w6.shape)}, expected (N, {K})")
    N = w6.shape[0]
    _need(w_scale, "w_scale", (N,), _FLOAT)
    if bias is not None:
        _need(bias, "bias", (N,), (x2.dtype,))
    if smooth is not None:
        _need(smooth, "smooth", (K,), (x2.dtype,))
    out_dtype = out_dtype or (out.dtype if out is not None else x2.dtype)
    if out_dtype not in _FLOAT:
        raise ValueError(f"out_dtype {out_dtype} is not float32/float16/bfloat16")
    if out is not None:
        _need(out, "out", (M, N), (out_dtype,))
    need = w4a4_linear_bf6_workspace_size(M, K)
    if workspace is not None:
        _need(workspace, "workspace", dtypes=(torch.uint8,))
        if workspace.numel() < need:
            raise ValueError(f"workspace holds {workspace.numel()} bytes, need {need}")
    _same_device(x2, rot=rot, w6=w6, w_scale=w_scale, bias=bias, smooth=smooth, out=out, workspace=workspace)
    dev = x2.device
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=dev)
    if workspace is None:
        workspace = torch.empty((max(need, 1),), dtype=torch.uint8, device=dev)
    rc = lib().w4a4_linear_bf6(
        _ptr(x2), _dt(x2), M, K, x2.stride(0), x2.stride(1), _ptr(rot), g, _ptr(smooth), _ptr(w6), N,
        _ptr(w_scale), _dt(w_scale), _ptr(bias), _ptr(out), _DT[out.dtype], _ptr(workspace), workspace.numel(),
        _stream(dev))
    _check(rc, "w4a4_linear_bf6")
    return out.view(*lead, N)
