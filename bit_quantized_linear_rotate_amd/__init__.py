"""MI355X (gfx950) W4A4 rotate/quantize linear layer.

The hot path is hand-written HIP behind a C ABI (include/w4a4.h, built into
libw4a4.so next to this file); this package is the thin Python binding.
"""
from ._binding import (  # noqa: F401
    W4A4Error,
    lib,
    w4a4_device_supported,
    w4a4_gemm_plan,
    w4a4_gemm_from_codes,
    w4a4_gemm_workspace_size,
    w4a4_int32_guard,
    w4a4_linear,
    w4a4_linear_noalloc,
    NOALLOC_SCRATCH_BYTES,
    w4a4_linear_workspace_size,
    w4a4_lowrank_down,
    w4a4_rotate_quant_plan,
    w4a4_rotate_quant_rowwise,
    w8a8_gemm_from_codes,
    w8a8_gemm_workspace_size,
    w8a8_linear,
    w8a8_linear_workspace_size,
    w8a8_rotate_quant_plan,
    w8a8_gemm_plan,
    Hadamard,
    w4a4_rotate_quant_hadamard,
    w4a4_rotate_quant_hadamard_plan,
    w4a4_linear_hadamard,
    w8a8_linear_hadamard,
    w4a4_svdquant_workspace_size,
    w4a4_quantize_svdquant,
    w4a4_gemm_svdquant,
    w4a4_linear_svdquant,
    w4a4_linear_svdquant_grouped,
    fuse_linear_weights,
    w8a8_rotate_quant_rowwise,
)
