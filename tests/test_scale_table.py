"""Host check of the row kernel's per-significand scale table.

The prefill row kernel reads a row's scale s = max(a / qmax, 2^-126), 1/s,
the two multipliers that bracket every quotient and the outcomes of exact ties
from a table indexed by the significand of its 16-bit absmax a, shifted by a's
exponent (bit_quantized_linear_rotate_amd/csrc/scale_table.hpp).  This test
compiles tests/scale_table_check.cpp with g++ and runs it: for every 16-bit
pattern of bf16 and fp16 that the table covers, and for qmax 7 and 127, the
shifted table values must equal, bit for bit, the IEEE divisions the kernel
performs for rows the table does not cover (the per-row absmax scale of "[Feat]
[Ascend] Consolidate INT8, RotateQuant, RoPE and ConvRot W4A4 backends",
section "W4A4 correctness and performance scope").
"""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "..", "bit_quantized_linear_rotate_amd", "csrc")


def test_scale_table_matches_divisions(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    exe = str(tmp_path / "scale_table_check")
    subprocess.check_call([gxx, "-std=c++17", "-O2", "-ffp-contract=off", "-I", CSRC,
                           os.path.join(HERE, "scale_table_check.cpp"), "-o", exe])
    out = subprocess.run([exe], capture_output=True, text=True)
    print(out.stdout)
    assert out.returncode == 0, out.stdout + out.stderr
    counts = [int(l.split(":")[1].split()[0]) for l in out.stdout.splitlines() if "covered" in l]
    # bf16: every pattern with a biased exponent in 8..254; fp16: every
    # nonzero finite pattern (subnormals normalised)
    assert counts == [247 * 128, 247 * 128, 31 * 1024 - 1, 31 * 1024 - 1]
