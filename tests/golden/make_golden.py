"""Write oracle_regression.json from the oracle alone (seeded tiny workload).

Run from the repository root:  python tests/golden/make_golden.py
"""
import hashlib
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import workloads  # noqa: E402


def digest(a):
    return hashlib.sha256(a.tobytes()).hexdigest()


def main():
    w = workloads.WORKLOADS["tiny"]
    r = oracle.linear(workloads.generate(w), w.dtype, w.g, w.sw_dtype)
    rec = {
        "workload": "tiny: M=32 K=256 N=256 g=16 fp32, seed %d" % w.seed,
        "y_sha256": digest(r["y"]),
        "codes_sha256": digest(r["codes"]),
        "scales_hex": [format(int(v), "08x") for v in r["scales"].view("uint32")],
        "acc_sha256": digest(r["acc"]),
        "out_sha256": digest(r["out"]),
        "out_row0_hex": [format(int(v), "08x") for v in r["out"][0].view("uint32")[:16]],
    }
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "oracle_regression.json")
    with open(path, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    print("wrote", path)


if __name__ == "__main__":
    main()
