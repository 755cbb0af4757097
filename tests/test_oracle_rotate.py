"""Pins for the oracle's block rotation: Hadamard closed forms, orientation
under an asymmetric rotation, and exact-rational brute force."""
from fractions import Fraction

import numpy as np
import pytest

import workloads
from tests.exact import round_exact, round_exact_f32

DTS = ["f32", "f16", "bf16"]


def to_storage(vals, dt):
    return workloads.f32_to_storage(np.asarray(vals, dtype=np.float32), dt)


@pytest.mark.parametrize("g", [16, 64, 256])
def test_generated_hadamard_is_orthonormal_exactly(g):
    H = workloads.hadamard(g)
    assert np.array_equal(H @ H.T, np.eye(g))  # entries are +-2^-k: exact in fp64
    A = workloads.asymmetric_rotation(g, seed=g)
    assert np.array_equal(A @ A.T, np.eye(g))
    assert not np.array_equal(A, A.T)


@pytest.mark.parametrize("dt", DTS)
@pytest.mark.parametrize("g", [16, 64, 256])
def test_one_hot_gives_row_of_R(orc, dt, g):
    # x = e_i in one group -> y = row i of R (reading: y_j = sum_i x_i R[i][j]).
    R = workloads.asymmetric_rotation(g, seed=7)
    K = 2 * g
    x = np.zeros((g, K), dtype=np.float32)
    for i in range(g):
        x[i, g + i] = 1.0  # second group
    y = orc.decode(dt, orc.rotate(to_storage(x, dt), R, g, dt))
    assert np.array_equal(y[:, :g], np.zeros((g, g)))
    assert np.array_equal(y[:, g:], R)  # +-2^-k exactly representable in every dtype


@pytest.mark.parametrize("dt", DTS)
@pytest.mark.parametrize("g", [16, 64, 256])
def test_all_ones_group_gives_sqrt_g_e0(orc, dt, g):
    R = workloads.hadamard(g)
    x = np.ones((3, g), dtype=np.float32)
    y = orc.decode(dt, orc.rotate(to_storage(x, dt), R, g, dt))
    want = np.zeros(g)
    want[0] = np.sqrt(g)
    assert np.array_equal(y, np.tile(want, (3, 1)))


@pytest.mark.parametrize("dt", DTS)
def test_identity_rotation_is_identity(orc, dt):
    rng = np.random.default_rng(11)
    x = to_storage(rng.standard_normal((5, 64)), dt)
    y = orc.rotate(x, np.eye(16), 16, dt)
    assert np.array_equal(orc.decode(dt, y), orc.decode(dt, x))


@pytest.mark.parametrize("dt", ["f16", "bf16", "f32"])
@pytest.mark.parametrize("g", [16, 64])
def test_rotation_matches_exact_rational(orc, dt, g):
    # exact sum of exact products, one nearest-even rounding to T
    rng = np.random.default_rng(12 + g)
    R = workloads.asymmetric_rotation(g, seed=3)
    x = to_storage(rng.standard_normal((3, 2 * g)) * 3, dt)
    xv = orc.decode(dt, x)
    Rq = [[Fraction(float(v)) for v in row] for row in R]  # +-2^-k, exact in T
    y = orc.decode(dt, orc.rotate(x, R, g, dt))
    for m in range(x.shape[0]):
        for b in range(2):
            xs = [Fraction(float(v)) for v in xv[m, b * g:(b + 1) * g]]
            for j in range(g):
                s = sum(xs[i] * Rq[i][j] for i in range(g))
                want = round_exact_f32(s) if dt == "f32" else round_exact(s, dt)
                assert y[m, b * g + j] == want


@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_rotation_rounds_R_to_T_first(orc, dt):
    # A rotation entry that is not representable in T must be rounded to T
    # before use: 1/3 in T times 3 differs from exact 1.
    g = 16
    R = np.eye(g)
    R[0, 0] = 1.0 / 3.0
    x = to_storage(np.full((1, g), 3.0), dt)
    y = orc.decode(dt, orc.rotate(x, R, g, dt))
    r_t = orc.round_to(dt, [1.0 / 3.0])[0][0]
    want = round_exact(Fraction(3) * Fraction(r_t), dt)
    assert y[0, 0] == want


@pytest.mark.parametrize("g", [16, 64, 256])
def test_round_trip_and_norm(orc, g):
    rng = np.random.default_rng(13)
    R = workloads.hadamard(g)
    x = rng.standard_normal((4, 2 * g)).astype(np.float32)
    y = orc.decode("f32", orc.rotate(x, R, g, "f32"))
    back = orc.decode("f32", orc.rotate(y.astype(np.float32), R.T.copy(), g, "f32"))
    assert np.allclose(back, x, rtol=0, atol=1e-5)
    for b in range(2):
        assert np.allclose(np.linalg.norm(y[:, b * g:(b + 1) * g], axis=1),
                           np.linalg.norm(x[:, b * g:(b + 1) * g], axis=1), rtol=1e-6)


def test_smoothing_divides_in_fp32_then_rounds(orc):
    # reading: x' = T(fp32(x) / fp32(s)); checked against numpy fp32 division
    rng = np.random.default_rng(14)
    for dt in DTS:
        x = to_storage(rng.standard_normal((3, 32)) * 4, dt)
        s = to_storage(rng.uniform(0.5, 2.0, size=32), dt)
        got = orc.decode(dt, orc.smooth(x, s, dt))
        q = (orc.decode(dt, x).astype(np.float32) / orc.decode(dt, s).astype(np.float32))
        want = orc.decode(dt, workloads.f32_to_storage(q, dt))
        assert np.array_equal(got, want)
