"""End-to-end pins for the oracle on the tiny fp32 workload (M=32, K=256,
N=256, g=16): the output against an fp64 evaluation of the dequantized
product with a rounding-analysis bound, and a hand-checkable worked case."""
from fractions import Fraction

import numpy as np

import oracle
import workloads


def test_tiny_workload_rounding_bound():
    w = workloads.WORKLOADS["tiny"]
    inp = workloads.generate(w)
    r = oracle.linear(inp, w.dtype, w.g, w.sw_dtype)
    codes, s = r["codes"], r["scales"].astype(np.float64)
    wq = oracle.unpack(inp["w_packed"], w.K).astype(np.float64)
    sw = inp["s_w"].astype(np.float64)
    b = inp["bias"].astype(np.float64)
    main = (codes.astype(np.float64) @ wq.T) * s[:, None] * sw[None, :]
    y64 = main + b[None, :]
    u = 2.0 ** -24
    bound = 4 * u * (np.abs(main) + np.abs(b)[None, :]) + 1e-45
    assert (np.abs(r["out"].astype(np.float64) - y64) <= bound).all()
    # and it approximates the float linear on rotated activations: the stored
    # weight codes live in the rotated basis, x W^T = (x R)(W R)^T
    x = inp["x"].astype(np.float64)
    R = np.kron(np.eye(w.K // w.g), inp["rot"])
    ref = (x @ R) @ (wq * sw[:, None]).T + b[None, :]
    rel = np.linalg.norm(r["out"] - ref) / np.linalg.norm(ref)
    assert rel < 0.2


def test_worked_example_all_ones_group():
    # x = 16 ones, g = 16, normalized Hadamard: y = (4, 0, ..., 0); absmax 4,
    # s = fp32(4/7); codes (7, 0, ..., 0).  One weight row with code 3 at k=0
    # gives acc = 21; out = fp32(fp32(21 * s) * s_w) + bias.
    K, g = 16, 16
    x = np.ones((1, K), dtype=np.float32)
    wcodes = np.zeros((1, K), dtype=np.int8)
    wcodes[0, 0] = 3
    wcodes[0, 5] = -8          # multiplies a zero code
    inp = {"x": x, "rot": workloads.hadamard(g), "w_packed": oracle.pack(wcodes),
           "s_w": np.array([0.0625], dtype=np.float32), "bias": np.array([0.5], np.float32),
           "smooth": None, "proj_down": None, "proj_up": None}
    r = oracle.linear(inp, "f32", g, "f32")
    assert list(r["y"][0]) == [4.0] + [0.0] * 15
    s = np.float32(4.0) / np.float32(7.0)
    assert r["scales"][0] == s
    assert Fraction(float(s)) != Fraction(4, 7)           # s is the rounded quotient
    assert list(r["codes"][0]) == [7] + [0] * 15
    assert r["acc"][0, 0] == 21
    want = np.float32(np.float32(np.float32(21.0) * s) * np.float32(0.0625)) + np.float32(0.5)
    assert r["out"][0, 0] == want
