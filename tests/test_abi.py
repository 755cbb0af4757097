"""CPU tests of the C ABI: the library loads, exports every function that
include/w4a4.h declares, and rejects bad arguments on the host before any
device access (no GPU needed: validation precedes the device check)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "w4a4.h")


@pytest.fixture(scope="module")
def L():
    from bit_quantized_linear_rotate_amd import _binding
    if not os.path.exists(_binding.LIB_PATH):
        pytest.skip("libw4a4.so not built")
    return _binding.lib()


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(w4a4_[a-z_0-9]+)\s*\(", src, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_boundary():
    names = declared_functions()
    for want in ["w4a4_rotate_quant_rowwise", "w4a4_linear", "w4a4_gemm_from_codes",
                 "w4a4_lowrank_down", "w4a4_int32_guard", "w4a4_last_error"]:
        assert want in names


def test_every_declared_symbol_is_exported(L):
    for name in declared_functions():
        assert hasattr(L, name), name


def test_library_has_gfx950_code_object():
    from bit_quantized_linear_rotate_amd import _binding
    blob = open(_binding.LIB_PATH, "rb").read()
    assert b"gfx950" in blob


FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: validation fails first


def rq(L, x=FAKE, dt=2, M=4, K=64, sm=64, sk=1, rot=FAKE, g=16, codes=FAKE, scales=FAKE):
    return L.w4a4_rotate_quant_rowwise(x, dt, M, K, sm, sk, rot, g, None, codes, scales, None, None)


def test_rotate_quant_rejections(L):
    from bit_quantized_linear_rotate_amd._binding import INVALID, OK, UNSUPPORTED
    assert rq(L, K=63, sm=63) == INVALID                       # odd width
    assert b"odd" in L.w4a4_last_error()
    assert rq(L, K=48, sm=48, g=32) == INVALID                 # K % g
    assert rq(L, M=-1) == INVALID
    assert rq(L, sm=-1) == INVALID
    assert rq(L, x=None) == INVALID
    assert rq(L, codes=None) == INVALID
    assert rq(L, dt=7) == UNSUPPORTED
    assert rq(L, g=24, K=48, sm=48) == UNSUPPORTED             # not a power of two
    assert rq(L, g=512, K=1024, sm=1024) == UNSUPPORTED
    assert rq(L, M=0) == OK                                    # empty: nothing launched


def gemm(L, M=4, K=64, N=8, sw_group=0, k_chunk=0, lora=None, up=None, rank=0, ws=None, wsb=0,
         codes=FAKE, sw_dt=2, out=FAKE):
    return L.w4a4_gemm_from_codes(codes, FAKE, M, K, FAKE, N, FAKE, sw_dt, sw_group, None, 0, lora,
                                  up, 2, rank, out, 2, None, k_chunk, ws, wsb, None)


def test_gemm_rejections(L):
    from bit_quantized_linear_rotate_amd._binding import INVALID, OK, UNSUPPORTED
    assert gemm(L, K=63) == INVALID
    assert gemm(L, sw_group=32) == INVALID
    assert gemm(L, sw_group=64, K=96) == INVALID
    assert gemm(L, k_chunk=100) == INVALID
    assert gemm(L, k_chunk=64, sw_group=64, K=128) == INVALID
    assert gemm(L, lora=FAKE) == INVALID                       # lora without proj_up
    assert gemm(L, lora=FAKE, up=FAKE, rank=65) == INVALID
    assert gemm(L, codes=None) == INVALID
    assert gemm(L, out=None) == INVALID
    assert gemm(L, sw_dt=9) == UNSUPPORTED
    assert gemm(L, k_chunk=64) == INVALID                      # workspace missing
    assert gemm(L, M=0) == OK


def test_guard_and_workspace_sizes(L):
    from bit_quantized_linear_rotate_amd import _binding as b
    assert b.w4a4_int32_guard(3840) == (False, 0)
    assert b.w4a4_int32_guard(16384) == (False, 0)
    need, chunk = b.w4a4_int32_guard(3_000_000)
    assert need and chunk % 64 == 0 and chunk * 16 * 7 * 8 <= 2 ** 31 - 1
    assert b.w4a4_gemm_workspace_size(10, 20, 256, 64) >= 10 * 20 * 8
    assert b.w4a4_gemm_workspace_size(10, 20, 256, 0) == 0
    assert b.w4a4_linear_workspace_size(8192, 3840, 3840, 0) >= 8192 * 3840 + 8192 * 4
    assert b.w4a4_linear_workspace_size(0, 3840, 3840, 0) == 0


def test_linear_rejections(L):
    from bit_quantized_linear_rotate_amd._binding import INVALID
    rc = L.w4a4_linear(FAKE, 2, 4, 64, 64, 1, FAKE, 16, None, FAKE, 8, FAKE, 2, 0, None, FAKE,
                       None, 32, FAKE, 2, FAKE, 1 << 20, None)
    assert rc == INVALID                                      # proj_down without proj_up
    rc = L.w4a4_linear(FAKE, 2, 4, 64, 64, 1, FAKE, 16, None, FAKE, 8, FAKE, 2, 0, None, None,
                       None, 0, FAKE, 2, FAKE, 16, None)
    assert rc == INVALID                                      # workspace too small


def test_plan_queries_name_the_config_kernels(L):
    # host-only: which kernels the five workloads' calls take (nothing runs)
    import torch
    from bit_quantized_linear_rotate_amd import _binding as b
    bf, h = torch.bfloat16, torch.float16
    assert b.w4a4_rotate_quant_plan(torch.zeros(8192, 3840, dtype=bf), torch.zeros(64, 64), 64) == "row"
    assert b.w4a4_rotate_quant_plan(torch.zeros(1600, 3840, dtype=bf), torch.zeros(64, 64), 64) == "wave"
    xt = torch.zeros(10240, 8192, dtype=h).t()
    assert b.w4a4_rotate_quant_plan(xt, torch.zeros(256, 256), 256) == "colmajor"
    assert b.w4a4_rotate_quant_plan(torch.zeros(4096, 16384, dtype=bf), torch.zeros(256, 256), 256,
                                    smooth=torch.zeros(16384, dtype=bf)) == "g256"
    assert b.w4a4_rotate_quant_plan(torch.zeros(32, 3840, dtype=bf), torch.zeros(64, 64), 64) == "reg"
    assert b.w4a4_rotate_quant_plan(torch.zeros(32, 256), torch.zeros(16, 16), 16) == "generic"
    assert b.w4a4_gemm_plan(8192, 3840, 3840) == "pingpong"
    assert b.w4a4_gemm_plan(8192, 10240, 3840) == "pingpong"
    assert b.w4a4_gemm_plan(300, 1024, 260) == "ring3"    # N % 16 != 0
    assert b.w4a4_gemm_plan(32, 3840, 3840) == "skinny"
    assert b.w4a4_gemm_plan(4096, 16384, 6144, 64, lowrank=True) == "tile128"
    assert b.w4a4_gemm_plan(300, 1024, 200, k_chunk=128) == "tile128_splitk"
    assert b.w4a4_gemm_plan(300, 1024, 256, return_acc=True) == "tile128"
    assert b.w4a4_gemm_plan(0, 1024, 256) == "none"
    with pytest.raises(ValueError):
        b.w4a4_rotate_quant_plan(torch.zeros(4, 63, dtype=bf), None, 0)
