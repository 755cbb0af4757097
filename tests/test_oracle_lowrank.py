"""Pins for the oracle's low-rank down projection L = x . proj_down on the raw
activation (source page comfy_kitchen/tensor/svdquant_w4a4.py: proj_down is
(K, R) in the module docstring; the _w4a4_forward docstring has the low-rank
branch read the raw, unshifted activation, i.e. before smoothing and rotation).

Each test would fail on a plausible mistake in the oracle:
  * brute force in exact rationals: a dropped term, a wrong index, a sum that
    is rounded more than once;
  * one-hot projections with K != R and an asymmetric pattern: proj_down
    indexed as (R, K) instead of (K, R), or the result transposed;
  * the whole layer with smoothing on: the branch reading the smoothed (or
    rotated) activation instead of the raw one.
"""
from fractions import Fraction

import numpy as np
import pytest

import workloads
from tests.exact import round_exact_f32


def _bf16_grid(rng, shape, lo_exp=-3, hi_exp=3):
    """bf16 values with a narrow exponent range, so that every product of two
    of them and every sum of up to 64 products is exact in float64."""
    mant = rng.integers(128, 256, size=shape)
    exp = rng.integers(lo_exp, hi_exp + 1, size=shape)
    sign = rng.choice([-1.0, 1.0], size=shape)
    vals = sign * mant.astype(np.float64) * np.exp2(exp - 7)
    vals[rng.random(shape) < 0.1] = 0.0
    return workloads.f32_to_storage(vals.astype(np.float32), "bf16")


@pytest.mark.parametrize("M,K,R", [(1, 2, 1), (3, 16, 4), (4, 64, 3), (2, 40, 2)])
def test_brute_force_exact_rationals(orc, M, K, R):
    rng = np.random.default_rng(M * 100 + K + R)
    x = _bf16_grid(rng, (M, K))
    down = _bf16_grid(rng, (K, R))
    L = orc.lowrank_down(x, down, "bf16")
    xv = workloads.storage_to_f32(x, "bf16")
    dv = workloads.storage_to_f32(down, "bf16")
    for m in range(M):
        for r in range(R):
            exact = sum((Fraction(float(xv[m, k])) * Fraction(float(dv[k, r])) for k in range(K)),
                        Fraction(0))
            assert float(L[m, r]) == round_exact_f32(exact), (m, r)


@pytest.mark.parametrize("dt", ["f32", "f16", "bf16"])
def test_one_hot_projection_selects_columns(orc, dt):
    # proj_down[k, r] = 1 exactly when k == sel[r]: L[:, r] = x[:, sel[r]].
    # K != R and sel is not a permutation of range(R), so reading proj_down as
    # (R, K) or transposing the result cannot give the same numbers.
    M, K, R = 5, 48, 7
    rng = np.random.default_rng(3)
    x = workloads.f32_to_storage(rng.standard_normal((M, K)).astype(np.float32), dt)
    sel = np.array([40, 3, 17, 3, 0, 47, 29])
    d = np.zeros((K, R), dtype=np.float32)
    d[sel, np.arange(R)] = 1.0
    L = orc.lowrank_down(x, workloads.f32_to_storage(d, dt), dt)
    xv = workloads.storage_to_f32(x, dt)
    assert np.array_equal(L, xv[:, sel])
    # a scaled one-hot: the weight multiplies (powers of two stay exact)
    d2 = d * np.float32(-0.25)
    L2 = orc.lowrank_down(x, workloads.f32_to_storage(d2, dt), dt)
    assert np.array_equal(L2, xv[:, sel] * np.float32(-0.25))


def test_two_terms_round_once(orc):
    # 1 + 2^-24 + 2^-30 lies just above the midpoint of 1 and 1 + 2^-23, so
    # one rounding of the exact sum gives 1 + 2^-23, while fp32 partial sums
    # (1 + 2^-24 ties to 1 first) or a dropped last term give 1.
    x = np.array([[1.0, 2.0 ** -24, 2.0 ** -30]], dtype=np.float32)
    d = np.ones((3, 1), dtype=np.float32)
    L = orc.lowrank_down(x, d, "f32")
    assert L[0, 0] == np.float32(1.0 + 2.0 ** -23)
    # fp32 partial sums would give fl(fl(1 + 2^-24) + 2^-30) = fl(1 + 2^-30) = 1
    assert np.float32(np.float32(np.float32(1.0) + np.float32(2.0 ** -24)) + np.float32(2.0 ** -30)) == 1.0


def test_layer_branch_reads_the_raw_activation(orc):
    # The whole layer with smoothing on: the L it returns equals x . proj_down
    # on the raw x (numpy in float64, exact for these inputs, then one fp32
    # rounding), and differs from the same product on the smoothed x.
    M, K, N, R, g = 4, 64, 8, 3, 16
    rng = np.random.default_rng(12)
    x = _bf16_grid(rng, (M, K))
    down = _bf16_grid(rng, (K, R))
    sm = workloads.f32_to_storage(np.full(K, 2.0, dtype=np.float32), "bf16")
    inp = {"x": x, "rot": workloads.hadamard(g),
           "w_packed": workloads.random_packed_weights(rng, N, K),
           "s_w": workloads.f32_to_storage(np.full(N, 0.01, np.float32), "bf16"),
           "bias": None, "smooth": sm, "proj_down": down,
           "proj_up": workloads.f32_to_storage(rng.normal(0, 0.1, size=(N, R)).astype(np.float32),
                                               "bf16")}
    r = orc.linear(inp, "bf16", g, "bf16")
    xv = workloads.storage_to_f32(x, "bf16").astype(np.float64)
    dv = workloads.storage_to_f32(down, "bf16").astype(np.float64)
    raw = (xv @ dv).astype(np.float32)
    assert np.array_equal(r["L"], raw)
    smoothed = ((xv / 2.0) @ dv).astype(np.float32)
    assert not np.array_equal(r["L"], smoothed)
    # and the output carries that term: removing it changes the result
    no_lr = dict(inp, proj_down=None, proj_up=None)
    r0 = orc.linear(no_lr, "bf16", g, "bf16")
    assert not np.array_equal(r0["out"], r["out"])
