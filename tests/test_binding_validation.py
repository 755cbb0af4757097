"""The binding rejects bad layouts before any device access (bindings that
reject bad layouts: "HIP port of #191: W6A8 decode in the W4A8 kernels",
section "Description").

These run on the CPU: every argument's shape, dtype and contiguity is checked
first, then the device, so a wrong layout raises ValueError whether or not a
GPU is present, and well-formed CPU tensors are refused as not being on a HIP
device.  No kernel is launched by any of these calls."""
import os

import pytest
import torch

from bit_quantized_linear_rotate_amd import _binding as b

pytestmark = pytest.mark.skipif(not os.path.exists(b.LIB_PATH), reason="libw4a4.so not built")

M, K, N, G, R = 8, 128, 16, 64, 4
BF = torch.bfloat16


def layer_args(**over):
    a = dict(x=torch.zeros(M, K, dtype=BF), rot=torch.zeros(G, G), g=G,
             w_packed=torch.zeros(N, K // 2, dtype=torch.uint8), w_scale=torch.zeros(N, dtype=BF),
             w_scale_group=0, bias=None, smooth=None, proj_down=None, proj_up=None,
             out_dtype=None, workspace=None, out=None)
    a.update(over)
    return a


def gemm_args(**over):
    a = dict(codes=torch.zeros(M, K, dtype=torch.int8), scales=torch.zeros(M),
             w_packed=torch.zeros(N, K // 2, dtype=torch.uint8), w_scale=torch.zeros(N, dtype=BF),
             w_scale_group=0, bias=None, lora_act=None, proj_up=None, out_dtype=BF)
    a.update(over)
    return a


def raises(fn, kwargs, match):
    with pytest.raises(ValueError, match=match):
        fn(**kwargs)


# ---- w4a4_linear ----------------------------------------------------------
LINEAR_BAD = {
    "w_packed_shape": (dict(w_packed=torch.zeros(N, K, dtype=torch.uint8)), "w_packed"),
    "w_packed_dtype": (dict(w_packed=torch.zeros(N, K // 2, dtype=torch.int8)), "w_packed"),
    "w_packed_strided": (dict(w_packed=torch.zeros(N, K, dtype=torch.uint8)[:, ::2]), "w_packed"),
    "w_scale_shape": (dict(w_scale=torch.zeros(N + 1, dtype=BF)), "w_scale"),
    "w_scale_group_shape": (dict(w_scale_group=64, w_scale=torch.zeros(N, dtype=BF)), "w_scale"),
    "w_scale_group_value": (dict(w_scale_group=32), "w_scale_group"),
    "w_scale_dtype": (dict(w_scale=torch.zeros(N, dtype=torch.int32)), "w_scale"),
    "bias_shape": (dict(bias=torch.zeros(N - 1, dtype=BF)), "bias"),
    "bias_dtype": (dict(bias=torch.zeros(N, dtype=torch.float32)), "bias"),
    "smooth_shape": (dict(smooth=torch.zeros(K // 2, dtype=BF)), "smooth"),
    "smooth_dtype": (dict(smooth=torch.zeros(K, dtype=torch.float16)), "smooth"),
    "proj_down_rows": (dict(proj_down=torch.zeros(K + 2, R, dtype=BF),
                            proj_up=torch.zeros(N, R, dtype=BF)), "proj_down"),
    "proj_down_dtype": (dict(proj_down=torch.zeros(K, R), proj_up=torch.zeros(N, R, dtype=BF)),
                        "proj_down"),
    "proj_up_shape": (dict(proj_down=torch.zeros(K, R, dtype=BF),
                           proj_up=torch.zeros(N, R + 1, dtype=BF)), "proj_up"),
    "proj_up_alone": (dict(proj_up=torch.zeros(N, R, dtype=BF)), "together"),
    "rot_shape": (dict(rot=torch.zeros(G, G // 2)), "rot"),
    "rot_dtype": (dict(rot=torch.zeros(G, G, dtype=torch.float64)), "rot"),
    "out_shape": (dict(out=torch.zeros(M, N + 1, dtype=BF)), "out"),
    "out_dtype_mismatch": (dict(out=torch.zeros(M, N, dtype=BF), out_dtype=torch.float32), "out"),
    "out_strided": (dict(out=torch.zeros(N, M, dtype=BF).t()), "out"),
    "out_dtype_int": (dict(out_dtype=torch.int32), "out_dtype"),
    "workspace_small": (dict(workspace=torch.zeros(16, dtype=torch.uint8)), "workspace"),
    "workspace_dtype": (dict(workspace=torch.zeros(1 << 16, dtype=torch.int32)), "workspace"),
    "x_not_tensor": (dict(x=[[0.0] * K] * M), "x"),
}


@pytest.mark.parametrize("case", list(LINEAR_BAD))
def test_linear_rejects_bad_layout(case):
    over, match = LINEAR_BAD[case]
    raises(b.w4a4_linear, layer_args(**over), match)


def test_linear_rejects_host_tensors():
    raises(b.w4a4_linear, layer_args(), "CUDA")


def test_linear_rejects_unsupported_dtype():
    with pytest.raises(NotImplementedError):
        b.w4a4_linear(**layer_args(x=torch.zeros(M, K, dtype=torch.float64)))


# ---- w4a4_gemm_from_codes -------------------------------------------------
GEMM_BAD = {
    "codes_dtype": (dict(codes=torch.zeros(M, K, dtype=torch.uint8)), "codes"),
    "codes_strided": (dict(codes=torch.zeros(K, M, dtype=torch.int8).t()), "codes"),
    "codes_rank": (dict(codes=torch.zeros(M * K, dtype=torch.int8)), "codes"),
    "scales_shape": (dict(scales=torch.zeros(M + 1)), "scales"),
    "scales_dtype": (dict(scales=torch.zeros(M, dtype=BF)), "scales"),
    "w_packed_shape": (dict(w_packed=torch.zeros(N, K // 2 + 1, dtype=torch.uint8)), "w_packed"),
    "w_scale_shape": (dict(w_scale=torch.zeros(N, 2, dtype=BF)), "w_scale"),
    "w_scale_group_shape": (dict(w_scale_group=64, w_scale=torch.zeros(K // 64 + 1, N, dtype=BF)),
                            "w_scale"),
    "bias_shape": (dict(bias=torch.zeros(2 * N, dtype=BF)), "bias"),
    "lora_rows": (dict(lora_act=torch.zeros(M + 1, R), proj_up=torch.zeros(N, R, dtype=BF)),
                  "lora_act"),
    "lora_dtype": (dict(lora_act=torch.zeros(M, R, dtype=BF), proj_up=torch.zeros(N, R, dtype=BF)),
                   "lora_act"),
    "proj_up_rank": (dict(lora_act=torch.zeros(M, R), proj_up=torch.zeros(N, R - 1, dtype=BF)),
                     "proj_up"),
    "lora_alone": (dict(lora_act=torch.zeros(M, R)), "together"),
    "out_dtype": (dict(out_dtype=torch.int8), "out_dtype"),
}


@pytest.mark.parametrize("case", list(GEMM_BAD))
def test_gemm_rejects_bad_layout(case):
    over, match = GEMM_BAD[case]
    raises(b.w4a4_gemm_from_codes, gemm_args(**over), match)


def test_gemm_rejects_host_tensors():
    raises(b.w4a4_gemm_from_codes, gemm_args(), "CUDA")


# ---- w4a4_rotate_quant_rowwise and w4a4_lowrank_down ----------------------
def test_rotate_quant_rejections():
    x = torch.zeros(M, K, dtype=BF)
    raises(b.w4a4_rotate_quant_rowwise, dict(x=x, rot=torch.zeros(G, G + 1), g=G), "rot")
    raises(b.w4a4_rotate_quant_rowwise, dict(x=x, rot=None, g=0, smooth=torch.zeros(K)), "smooth")
    raises(b.w4a4_rotate_quant_rowwise, dict(x=x, rot=None, g=0,
                                             smooth=torch.zeros(K - 2, dtype=BF)), "smooth")
    raises(b.w4a4_rotate_quant_rowwise, dict(x=x, rot=torch.zeros(G, G), g=G), "CUDA")


def test_lowrank_down_rejections():
    x = torch.zeros(M, K, dtype=BF)
    raises(b.w4a4_lowrank_down, dict(x=x, proj_down=torch.zeros(R, K, dtype=BF)), "proj_down")
    raises(b.w4a4_lowrank_down, dict(x=x, proj_down=torch.zeros(K, R)), "proj_down")
    raises(b.w4a4_lowrank_down, dict(x=x, proj_down=torch.zeros(K, 2 * R, dtype=BF)[:, ::2]),
           "contiguous")
    raises(b.w4a4_lowrank_down, dict(x=x, proj_down=torch.zeros(K, R, dtype=BF)), "CUDA")
