"""Build the HIP library libw4a4.so in-tree for gfx950 (hipcc, no torch)."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libw4a4.so")
PROBE_LIB = os.path.join(HERE, "libw4a4_probe.so")
SOURCES = ["api.hip", "rotate_quant.hip", "rq_row.hip", "rq_hadamard.hip", "rq_svdquant.hip", "gemm.hip",
           "lowrank.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # IEEE arithmetic: no contraction of the epilogue's multiplies and adds,
    # denormals kept, correctly rounded fp32 division.
    "-ffp-contract=off", "-fno-fast-math", "-fno-gpu-flush-denormals-to-zero",
    # never let the compiler form packed fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result",
]
# per-source extra flags: the GEMM kernels' MFMA results live in ordinary
# VGPRs (the group-scale loop converts every result with VALU instructions,
# which cannot read accumulation registers)
SOURCE_FLAGS = {"gemm.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
                "rq_row.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
                "rq_hadamard.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def build(verbose: bool = False, jobs: int = 4) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    objs = []
    procs = []
    for src in SOURCES:
        obj = os.path.join(CSRC, "_build", src.replace(".hip", ".o"))
        os.makedirs(os.path.dirname(obj), exist_ok=True)
        cmd = [hipcc, *HIPCC_FLAGS, *SOURCE_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stderr=subprocess.PIPE, text=True)))
        objs.append(obj)
    failed = []
    for src, p in procs:
        _, err = p.communicate()
        err = "\n".join(l for l in err.splitlines() if "packed-fp32-ops" not in l)
        if p.returncode != 0:
            failed.append((src, err))
        elif err.strip() and verbose:
            print(err, file=sys.stderr)
    if failed:
        raise RuntimeError("\n".join(f"--- {s}\n{e}" for s, e in failed))
    tmp = LIB + ".tmp"
    subprocess.check_call([hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, LIB)
    # the streaming-bandwidth probe the benchmark measures the HBM ceiling with
    # (a library of its own: not part of the layer)
    ptmp = PROBE_LIB + ".tmp"
    subprocess.check_call([hipcc, *HIPCC_FLAGS, "-shared", "-o", ptmp, os.path.join(CSRC, "stream_probe.hip")])
    os.replace(ptmp, PROBE_LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
