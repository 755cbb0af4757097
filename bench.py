#!/usr/bin/env python3
"""Benchmark of the W4A4 rotate/quantize linear on one MI355X.

One step = the whole hot path on one batch: fused rotate+quantize of the
activation rows, then the INT8-MFMA W4A4 GEMM with its fused epilogue (plus the
low-rank down projection when the workload has one), i.e. one w4a4_linear call.

Prints ONE JSON line.  `value` is whole-job throughput in TOPS (2*M*N*K per
step / step time) with all inputs resident in HBM.  Four independent input /
weight / output sets are cycled so that consecutive steps do not find their
operands in the 256 MB last-level cache.  Each kernel is also timed alone with
HIP events on the stream it runs on, giving the roofline fractions.

The line also carries the other four workloads (wide-K transposed-view fp16,
decode-like M=32, tiny fp32, large-K with smoothing, per-64-group scales and a
rank-32 term), each as a step and per kernel.

Usage: python bench.py [--gpus 1] [--steps 50] [--warmup 10] [--workload prefill]
                       [--no-cpu] [--no-extra] [--copy-calibration]

`roofline.traffic` is the HBM traffic of one launch of the kernel as measured
by rocprofv3 FETCH_SIZE / WRITE_SIZE counters (scaled by a plain device copy
of known size, see profiles/), taken from the committed summary only while
the kernel's source file still has the hash recorded there; otherwise null.
--copy-calibration adds one untimed 256 MiB device copy before the timed
region, which is the calibration dispatch for those counter runs.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
INT8_PEAK_TOPS = 5000.0        # MI355X dense INT8 MFMA, published
GEMM_KERNEL = "w4a4_gemm_ring3_kernel (INT8 MFMA GEMM + fused scale/bias/cast epilogue)"
TRAFFIC_FILES = {  # kernel source -> committed counter summary
    "gemm": ("bit_quantized_linear_rotate_amd/csrc/gemm.hip", "profiles/gemm_prefill_m8192_k3840_n3840_traffic.json"),
    "rotate_quant": ("bit_quantized_linear_rotate_amd/csrc/rotate_quant.hip",
                     "profiles/rotate_quant_prefill_m8192_k3840_g64_traffic.json"),
}


def _traffic(which, workload):
    """HBM bytes per launch from the committed counter summary, or None when
    the summary is missing, is for another workload, or predates the current
    kernel source."""
    import hashlib
    src, summ = TRAFFIC_FILES[which]
    try:
        with open(os.path.join(ROOT, summ)) as f:
            rec = json.load(f)
        with open(os.path.join(ROOT, src), "rb") as f:
            digest = hashlib.sha256(f.read()).hexdigest()
    except (OSError, ValueError):
        return None
    if rec.get("source_sha256") != digest or rec.get("workload") != workload:
        return None
    return rec.get("traffic_bytes_per_launch")


METRIC = "W4A4 linear TOPS + rotate-quant GB/s (% roofline) at M=8192,K=3840/10240"


def _dev_inputs(w, inp, torch, np):
    def d(a, dt=None):
        if a is None:
            return None
        a = np.ascontiguousarray(a)
        if dt == "bf16":
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(a).cuda()
    x = d(inp["x_buffer"], w.dtype).t() if w.transposed else d(inp["x"], w.dtype)
    return dict(x=x, rot=torch.from_numpy(inp["rot"].astype(np.float32)).cuda(),
                w_packed=d(inp["w_packed"]), w_scale=d(inp["s_w"], w.sw_dtype),
                bias=d(inp["bias"], w.dtype), smooth=d(inp["smooth"], w.dtype),
                proj_down=d(inp["proj_down"], w.dtype), proj_up=d(inp["proj_up"], w.dtype))


def _variant(d, i, torch):
    """A distinct copy of the operands (same values, other addresses) so that
    cycling through sets defeats the last-level cache without new draws."""
    if i == 0:
        return d
    out = {}
    for k, v in d.items():
        if v is None or k == "rot":
            out[k] = v
        elif k == "x" and not v.is_contiguous():
            out[k] = v.t().contiguous().t()     # keep the transposed view
        else:
            out[k] = v.clone()
    return out


def _time_loop(fn, n, torch):
    """Average ms per call over n calls, HIP events on the current stream."""
    st = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(st)
    for i in range(n):
        fn(i)
    e1.record(st)
    e1.synchronize()
    return e0.elapsed_time(e1) / n


def measure(name, steps, warmup, torch, np, w4, workloads):
    w = workloads.WORKLOADS[name]
    inp = workloads.generate(w)
    base = _dev_inputs(w, inp, torch, np)
    sets = [_variant(base, i, torch) for i in range(4)]
    M, K, N, g = w.M, w.K, w.N, w.g
    rank = w.rank
    outs = [torch.empty((M, N), dtype=base["x"].dtype, device="cuda") for _ in sets]
    wss = [torch.empty((w4.w4a4_linear_workspace_size(M, K, N, rank),), dtype=torch.uint8,
                       device="cuda") for _ in sets]

    def step(i):
        s = sets[i % 4]
        w4.w4a4_linear(s["x"], s["rot"], g, s["w_packed"], s["w_scale"], w_scale_group=w.sw_group,
                       bias=s["bias"], smooth=s["smooth"], proj_down=s["proj_down"],
                       proj_up=s["proj_up"], workspace=wss[i % 4], out=outs[i % 4])

    for i in range(warmup):
        step(i)
    ms_step = _time_loop(step, steps, torch)

    # rotate+quantize alone (the kernel w4a4_linear launches first)
    qbufs = [(torch.empty((M, K), dtype=torch.int8, device="cuda"),
              torch.empty((M,), dtype=torch.float32, device="cuda")) for _ in sets]
    lib = w4.lib()
    import ctypes

    def rq(i):
        s = sets[i % 4]
        c, sc = qbufs[i % 4]
        x = s["x"]
        lib.w4a4_rotate_quant_rowwise(
            ctypes.c_void_p(x.data_ptr()), {torch.bfloat16: 2, torch.float16: 1, torch.float32: 0}[x.dtype],
            M, K, x.stride(0), x.stride(1), ctypes.c_void_p(s["rot"].data_ptr()), g,
            ctypes.c_void_p(s["smooth"].data_ptr()) if s["smooth"] is not None else None,
            ctypes.c_void_p(c.data_ptr()), ctypes.c_void_p(sc.data_ptr()), None,
            ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))

    for i in range(warmup):
        rq(i)
    ms_rq = _time_loop(rq, steps, torch)
    rq_bytes = M * K * base["x"].element_size() + M * K + 4 * M + 4 * g * g
    if w.smooth:
        rq_bytes += K * base["x"].element_size()

    # GEMM + epilogue alone, on the codes just produced
    def gemm(i):
        s = sets[i % 4]
        c, sc = qbufs[i % 4]
        w4.w4a4_gemm_from_codes(c, sc, s["w_packed"], s["w_scale"], w_scale_group=w.sw_group,
                                bias=s["bias"], out_dtype=outs[i % 4].dtype)
    if rank:
        gemm_note = "low-rank term excluded from the GEMM-alone timing"
    else:
        gemm_note = None
    for i in range(warmup):
        gemm(i)
    ms_gemm = _time_loop(gemm, steps, torch)
    ops = 2.0 * M * N * K
    # bytes the GEMM must move: codes, packed weights, scales, bias, output
    gemm_bytes = (M * K + N * K // 2 + 4 * M + base["w_scale"].numel() * base["w_scale"].element_size()
                  + (N * base["bias"].element_size() if base["bias"] is not None else 0)
                  + M * N * outs[0].element_size())
    res = {
        "workload": f"{name}: M={M} K={K} N={N} g={g} {w.dtype}"
                    + (" transposed-view input" if w.transposed else "")
                    + (f" smooth+rank{rank}" if rank else "")
                    + (" per-64-group scales" if w.sw_group else ""),
        "ms_per_step": ms_step,
        "tops": ops / (ms_step * 1e-3) / 1e12,
        "rotate_quant": {"ms": ms_rq, "GB_s": rq_bytes / (ms_rq * 1e-3) / 1e9,
                         "frac_hbm": rq_bytes / (ms_rq * 1e-3) / 1e9 / HBM_PEAK_GBS,
                         "algorithmic_bytes": rq_bytes},
        "gemm": {"ms": ms_gemm, "TOPS": ops / (ms_gemm * 1e-3) / 1e12,
                 "frac_int8": ops / (ms_gemm * 1e-3) / 1e12 / INT8_PEAK_TOPS, "ops": ops,
                 "GB_s": gemm_bytes / (ms_gemm * 1e-3) / 1e9, "algorithmic_bytes": gemm_bytes},
    }
    if gemm_note:
        res["gemm"]["note"] = gemm_note
    if rank:
        # low-rank down projection alone (the first kernel of a low-rank step)
        lbufs = [torch.empty((M, rank), dtype=torch.float32, device="cuda") for _ in sets]

        def lrd(i):
            s = sets[i % 4]
            x = s["x"]
            lib.w4a4_lowrank_down(
                ctypes.c_void_p(x.data_ptr()), {torch.bfloat16: 2, torch.float16: 1, torch.float32: 0}[x.dtype],
                M, K, x.stride(0), x.stride(1), ctypes.c_void_p(s["proj_down"].data_ptr()), rank,
                ctypes.c_void_p(lbufs[i % 4].data_ptr()), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))

        for i in range(warmup):
            lrd(i)
        ms_lrd = _time_loop(lrd, steps, torch)
        lrd_bytes = M * K * base["x"].element_size() + K * rank * base["proj_down"].element_size() + 4 * M * rank
        res["lowrank_down"] = {"ms": ms_lrd, "GB_s": lrd_bytes / (ms_lrd * 1e-3) / 1e9,
                               "frac_hbm": lrd_bytes / (ms_lrd * 1e-3) / 1e9 / HBM_PEAK_GBS,
                               "algorithmic_bytes": lrd_bytes}
    return w, inp, res


def cpu_baseline(w, inp, np, target_s=15.0):
    """The oracle as it stands, on a bounded sample of rows of the same
    workload (every column, the whole layer per row)."""
    import oracle

    def run(n):
        t0 = time.perf_counter()
        oracle.linear(inp, w.dtype, w.g, w.sw_dtype, w.sw_group, rows=np.arange(n))
        return time.perf_counter() - t0

    # Two short runs split the oracle's cost into a fixed part (the weight
    # side, done once per call) and a per-row part, which sizes the sample.
    t8, t64 = run(8), run(64)
    per_row = max((t64 - t8) / 56.0, 1e-6)
    fixed = max(t8 - 8 * per_row, 0.0)
    n = int(min(w.M, max(64, (target_s - fixed) / per_row)))
    # when the whole workload takes well under the target, repeat it
    reps = max(1, int(math.ceil(target_s / (fixed + per_row * n))))
    dt = sum(run(n) for _ in range(reps))
    ops = 2.0 * n * w.N * w.K * reps
    what = (f"all {w.M} rows" if n == w.M else f"first {n} of {w.M} rows") + \
        f" of the {w.name} workload, all {w.N} columns (rotation, quantization, exact GEMM, epilogue)"
    return {"value": ops / dt / 1e12, "unit": "TOPS", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": f"{what}, {reps} call(s): {dt:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="prefill")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-extra", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the layer's data-parallel split (rows of the "
              f"activation across GPUs, weights replicated) needs no exchange, so N={args.gpus} "
              f"is not run here", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import bit_quantized_linear_rotate_amd as w4
    import workloads

    torch.cuda.init()
    if args.copy_calibration:
        # one plain 256 MiB device copy (FETCH_SIZE / WRITE_SIZE calibration)
        src = torch.empty(256 << 20, dtype=torch.uint8, device="cuda").random_(0, 255)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    w, inp, main_res = measure(args.workload, args.steps, args.warmup, torch, np, w4, workloads)
    extras = {}
    if not args.no_extra and args.workload == "prefill":
        for name in ("widek", "decode", "tiny", "lowrank"):
            _, _, extras[name] = measure(name, max(10, args.steps // 2), args.warmup, torch, np, w4,
                                         workloads)
    g = main_res["gemm"]
    line = {
        "metric": METRIC,
        "value": round(main_res["tops"], 2),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(main_res["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {"workload": main_res["workload"], "M": w.M, "K": w.K, "N": w.N, "g": w.g,
                   "activation_dtype": w.dtype},
        "rotate_quant": {k: (round(v, 4) if isinstance(v, float) else v)
                         for k, v in main_res["rotate_quant"].items()},
        "gemm": {k: (round(v, 4) if isinstance(v, float) else v) for k, v in g.items()},
        "roofline": {"bound": "mfma", "achieved": round(g["TOPS"], 2), "peak": INT8_PEAK_TOPS,
                     "unit": "TOPS", "frac": round(g["frac_int8"], 4),
                     "traffic": _traffic("gemm", args.workload), "kernel": GEMM_KERNEL},
        "roofline_rotate_quant": {"bound": "hbm", "achieved": round(main_res["rotate_quant"]["GB_s"], 1),
                                  "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                  "frac": round(main_res["rotate_quant"]["frac_hbm"], 4),
                                  "traffic": _traffic("rotate_quant", args.workload),
                                  "kernel": "rotate-quant (block rotation on MFMA, row absmax, INT4 codes)"},
    }
    for name, extra in extras.items():
        line[name] = {"workload": extra["workload"], "ms_per_step": round(extra["ms_per_step"], 5),
                      "tops": round(extra["tops"], 2),
                      "rotate_quant": {k: (round(v, 4) if isinstance(v, float) else v)
                                       for k, v in extra["rotate_quant"].items()},
                      "gemm": {k: (round(v, 4) if isinstance(v, float) else v)
                               for k, v in extra["gemm"].items()}}
        if "lowrank_down" in extra:
            line[name]["lowrank_down"] = {k: (round(v, 4) if isinstance(v, float) else v)
                                          for k, v in extra["lowrank_down"].items()}
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline(w, inp, np)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
