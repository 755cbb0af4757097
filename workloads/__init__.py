"""Seeded synthetic inputs for the W4A4 rotate/quantize linear.

This module only draws random numbers and lays them out in the storage formats
the layer consumes.  It holds none of the method's arithmetic (no rotation, no
quantization, no GEMM, no epilogue), so that both the CPU oracle and the HIP
path can be fed from it without sharing any computation.

Storage formats (numpy arrays on the host):
  * "f32" activations/scales: ``np.float32``
  * "f16": ``np.float16``
  * "bf16": ``np.uint16`` holding the bfloat16 bit pattern (numpy has no bf16);
    values are drawn in fp32 and rounded to nearest-even by torch's CPU cast.
  * packed weights: ``np.uint8`` (N, K/2), two 4-bit two's-complement nibbles
    per byte, the even k in the low nibble.  Nibbles are drawn from the 15
    patterns that encode -7..7 (the pattern for -8 is never drawn).

The five workloads follow the shapes the pages measure: the Z-Image activation
shapes [32|8192, 3840|10240] timed for the fused RotateQuant operator, and the
Krea-like wide-K layer with SVDQuant-style extras (smoothing, per-64-group
weight scales, rank-32 correction).  Real captured activations and checkpoints
are not available; these seeded draws stand in for them.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

DTYPES = ("f32", "f16", "bf16")


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    M: int
    K: int
    N: int
    g: int
    dtype: str                 # activation dtype = output dtype
    dist: str                  # "normal" | "student_t4"
    outlier_frac: float = 0.0  # fraction of channels scaled by outlier_scale
    outlier_scale: float = 20.0
    zero_row_frac: float = 0.0
    transposed: bool = False   # x passed as a (K, M) buffer viewed as (M, K)
    sw_dtype: str = "f32"
    sw_group: int = 0          # 0: per output channel; 64: (K/64, N)
    bias: bool = False
    smooth: bool = False
    rank: int = 0
    seed: int = 1000

    def scaled(self, M: Optional[int] = None, N: Optional[int] = None,
               K: Optional[int] = None, seed: Optional[int] = None) -> "Workload":
        """Same recipe at another size (used by parity tests)."""
        return dataclasses.replace(
            self,
            M=self.M if M is None else M,
            N=self.N if N is None else N,
            K=self.K if K is None else K,
            seed=self.seed if seed is None else seed,
            name=self.name if (M, N, K) == (None, None, None) else self.name + "-scaled",
        )


WORKLOADS = {
    "tiny": Workload("tiny", M=32, K=256, N=256, g=16, dtype="f32", dist="normal",
                     sw_dtype="f32", bias=True, seed=1000),
    "decode": Workload("decode", M=32, K=3840, N=3840, g=64, dtype="bf16", dist="normal",
                       outlier_frac=0.01, sw_dtype="bf16", bias=True, seed=1001),
    "prefill": Workload("prefill", M=8192, K=3840, N=3840, g=64, dtype="bf16",
                        dist="student_t4", sw_dtype="bf16", bias=False, seed=1002),
    "widek": Workload("widek", M=8192, K=10240, N=3840, g=256, dtype="f16", dist="normal",
                      zero_row_frac=0.01, transposed=True, sw_dtype="f16", bias=True,
                      seed=1003),
    "lowrank": Workload("lowrank", M=4096, K=16384, N=6144, g=256, dtype="bf16",
                        dist="normal", outlier_frac=0.01, sw_dtype="bf16", sw_group=64,
                        smooth=True, rank=32, seed=1004),
}


def f32_to_storage(a: np.ndarray, dtype: str) -> np.ndarray:
    """Round fp32 draws to the storage dtype (nearest-even) and return storage."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    if dtype == "f32":
        return a
    if dtype == "f16":
        return a.astype(np.float16)
    if dtype == "bf16":
        import torch
        t = torch.from_numpy(a).to(torch.bfloat16)
        return t.view(torch.int16).numpy().view(np.uint16).copy()
    raise ValueError(dtype)


def storage_to_f32(a: np.ndarray, dtype: str) -> np.ndarray:
    """Widen storage to fp32 values (exact for all three formats)."""
    if dtype == "f32":
        return np.asarray(a, dtype=np.float32)
    if dtype == "f16":
        return np.asarray(a, dtype=np.float16).astype(np.float32)
    if dtype == "bf16":
        return (np.asarray(a, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)
    raise ValueError(dtype)


def hadamard(g: int) -> np.ndarray:
    """Normalized Sylvester-Hadamard matrix H_g / sqrt(g) in fp64 (g a power of 2)."""
    if g < 1 or g & (g - 1):
        raise ValueError("g must be a power of two")
    h = np.ones((1, 1))
    while h.shape[0] < g:
        h = np.block([[h, h], [h, -h]])
    return h / np.sqrt(g)


def asymmetric_rotation(g: int, seed: int) -> np.ndarray:
    """D @ H @ P / sqrt(g): random signs and a random column permutation of the
    normalized Hadamard.  Orthonormal, generally not symmetric, and every entry
    is +-2^-k (exact in fp16/bf16 for g in {16, 64, 256})."""
    rng = np.random.default_rng(seed)
    h = hadamard(g)
    d = rng.choice([-1.0, 1.0], size=g)
    perm = rng.permutation(g)
    return (d[:, None] * h)[:, perm]


_NIBBLES = np.array([0, 1, 2, 3, 4, 5, 6, 7, 9, 10, 11, 12, 13, 14, 15], dtype=np.uint8)


def random_packed_weights(rng: np.random.Generator, N: int, K: int) -> np.ndarray:
    lo = rng.choice(_NIBBLES, size=(N, K // 2))
    hi = rng.choice(_NIBBLES, size=(N, K // 2))
    return (lo | (hi << 4)).astype(np.uint8)


def generate(w: Workload) -> dict:
    """Draw every input of workload ``w`` in a fixed order from one seeded
    generator.  Returns a dict of host numpy arrays in storage formats:

    x          (M, K) storage in w.dtype, C-contiguous.  When w.transposed,
               ``x_buffer`` (K, M) holds the same values and x == x_buffer.T.
    rot        (g, g) fp64 normalized Hadamard.
    w_packed   (N, K/2) uint8.
    s_w        (N,) or (K/64, N) storage in w.sw_dtype, values U(0.005, 0.02).
    bias       (N,) storage in w.dtype or None, values N(0, 0.1^2).
    smooth     (K,) storage in w.dtype or None, values U(0.5, 2).
    proj_down  (K, R) storage in w.dtype or None, values N(0, 1) / sqrt(K).
    proj_up    (N, R) storage in w.dtype or None, values N(0, 0.1^2).
    """
    rng = np.random.default_rng(w.seed)
    M, K, N = w.M, w.K, w.N
    if w.dist == "normal":
        x = rng.standard_normal((M, K), dtype=np.float32)
    elif w.dist == "student_t4":
        x = rng.standard_t(4, size=(M, K)).astype(np.float32)
    else:
        raise ValueError(w.dist)
    if w.outlier_frac > 0 and K > 0:
        n_out = max(1, int(round(w.outlier_frac * K)))
        cols = rng.choice(K, size=n_out, replace=False)
        x[:, cols] *= np.float32(w.outlier_scale)
    if w.zero_row_frac > 0 and M > 0:
        n_zero = max(1, int(round(w.zero_row_frac * M)))
        rows = rng.choice(M, size=n_zero, replace=False)
        x[rows, :] = 0.0
    out = {}
    xs = f32_to_storage(x, w.dtype)
    if w.transposed:
        out["x_buffer"] = np.ascontiguousarray(xs.T)
        out["x"] = np.ascontiguousarray(xs)
    else:
        out["x"] = xs
    out["rot"] = hadamard(w.g)
    out["w_packed"] = random_packed_weights(rng, N, K)
    if w.sw_group:
        sw = rng.uniform(0.005, 0.02, size=(K // w.sw_group, N)).astype(np.float32)
    else:
        sw = rng.uniform(0.005, 0.02, size=(N,)).astype(np.float32)
    out["s_w"] = f32_to_storage(sw, w.sw_dtype)
    out["bias"] = (f32_to_storage(rng.normal(0.0, 0.1, size=(N,)).astype(np.float32), w.dtype)
                   if w.bias else None)
    out["smooth"] = (f32_to_storage(rng.uniform(0.5, 2.0, size=(K,)).astype(np.float32), w.dtype)
                     if w.smooth else None)
    if w.rank:
        out["proj_down"] = f32_to_storage(
            (rng.standard_normal((K, w.rank)) / np.sqrt(K)).astype(np.float32), w.dtype)
        out["proj_up"] = f32_to_storage(
            rng.normal(0.0, 0.1, size=(N, w.rank)).astype(np.float32), w.dtype)
    else:
        out["proj_down"] = None
        out["proj_up"] = None
    return out
