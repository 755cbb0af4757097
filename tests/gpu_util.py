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
