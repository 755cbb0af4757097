"""Regression guard: the oracle still reproduces the fixture that
tests/golden/make_golden.py wrote from it (not an independent pin)."""
import hashlib
import json
import os

import oracle
import workloads


def test_oracle_reproduces_regression_fixture():
    path = os.path.join(os.path.dirname(__file__), "golden", "oracle_regression.json")
    with open(path) as f:
        rec = json.load(f)
    w = workloads.WORKLOADS["tiny"]
    r = oracle.linear(workloads.generate(w), w.dtype, w.g, w.sw_dtype)
    h = lambda a: hashlib.sha256(a.tobytes()).hexdigest()  # noqa: E731
    assert h(r["y"]) == rec["y_sha256"]
    assert h(r["codes"]) == rec["codes_sha256"]
    assert [format(int(v), "08x") for v in r["scales"].view("uint32")] == rec["scales_hex"]
    assert h(r["acc"]) == rec["acc_sha256"]
    assert h(r["out"]) == rec["out_sha256"]
