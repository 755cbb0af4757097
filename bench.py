#!/usr/bin/env python3
"""Benchmark of the W4A4 rotate/quantize linear on one MI355X.

One step = the whole hot path on one batch: fused rotate+quantize of the
activation rows, then the INT8-MFMA W4A4 GEMM with its fused epilogue (plus the
low-rank down projection when the workload has one), i.e. one w4a4_linear call.

Prints ONE JSON line.  `value` is whole-job throughput in TOPS (2*M*N*K per
step / step time) with all inputs resident in HBM.  Four independent input /
weight / output sets are cycled so that consecutive steps do not find their
operands in the 256 MB last-level cache.

Before anything is timed, the CPU leg (the same part of the run that times the
oracle for `cpu_baseline`) checks each workload's output against the oracle on
a sample of rows (all columns): codes and scales of those rows, and the output
bit for bit wherever the codes agree (1 ulp with the low-rank term); a
mismatch ends the run with an error.  The statistics go into the line.
--no-cpu skips the whole CPU leg (parity and baseline).

Each kernel is then timed alone on the stream it runs on, over max(steps, 50)
launches with a HIP event pair around every launch: their median (the figure
rocprofv3's average kernel duration agrees with, and the one
`roofline.achieved` divides the kernel's algorithmic work by), mean, p10 and
p90; plus the average over one event pair around the back-to-back launches
(ms_loop, which includes the gaps between kernels).

The line also carries the other four workloads (wide-K transposed-view fp16,
decode-like M=32, tiny fp32, large-K with smoothing, per-64-group scales and a
rank-32 term), each as a step and per kernel, and the INT8 mode (qmax = 127,
INT8 weights) on the prefill and wide-K shapes, and the SVDQuant variant (act_unsigned,
per-64-group activation scales) on the low-rank shape.

Usage: python bench.py [--gpus 1] [--steps 200] [--warmup 100] [--workload prefill]
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
FP6_PEAK_TOPS = 10100.0        # MI355X dense FP6/FP4 MFMA, published
MIN_KERNEL_LAUNCHES = 50
TRAFFIC_FILES = {  # kernel source -> committed counter summary
    "gemm": ("bit_quantized_linear_rotate_amd/csrc/gemm.hip",
             "profiles/gemm_pingpong_prefill_m8192_k3840_n3840_traffic.json"),
    "rotate_quant": ("bit_quantized_linear_rotate_amd/csrc/rq_row.hip",
                     "profiles/rotate_quant_row_prefill_m8192_k3840_g64_traffic.json"),
}
GEMM_NAMES = {"pingpong": "w4a4_gemm_pp_kernel", "ring3": "w4a4_gemm_ring3_kernel",
              "skinny": "w4a4_gemm_skinny_kernel",
              "tile128": "w4a4_gemm_kernel", "tile128_splitk": "w4a4_gemm_kernel (K chunks)"}
RQ_NAMES = {"row": "rq_row_kernel", "wave": "rq_wave_kernel", "colmajor": "rq_colmajor_kernel", "g256": "rq_g256_kernel",
            "reg": "rq_reg_kernel", "mfma_lds": "rq_mfma_kernel", "generic": "rq_generic_kernel"}


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


def _time_each(fn, n, torch, np):
    """Two passes of n calls each, HIP events on the current stream (the
    stream the binding launches on):
      * an event pair around every launch: ms_median (the figure
        rocprofv3's average kernel duration agrees with, and the one the
        roofline figures divide by), ms_mean, ms_p10, ms_p90;
      * ms_loop: one event pair around n back-to-back launches, divided by n
        (includes the gaps between consecutive kernels)."""
    st = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(n)]
    torch.cuda.synchronize()
    for i in range(n):
        ev[i][0].record(st)
        fn(i)
        ev[i][1].record(st)
    ev[-1][1].synchronize()
    a = np.asarray([x.elapsed_time(y) for x, y in ev], dtype=np.float64)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(st)
    for i in range(n):
        fn(i)
    e1.record(st)
    e1.synchronize()
    loop = e0.elapsed_time(e1) / n
    return {"ms_mean": float(a.mean()), "ms_median": float(np.median(a)), "ms_p10": float(np.percentile(a, 10)),
            "ms_p90": float(np.percentile(a, 90)), "ms_loop": float(loop), "launches": int(n)}


def _dtcode(torch, t):
    return {torch.bfloat16: 2, torch.float16: 1, torch.float32: 0}[t.dtype]


def cpu_leg_parity(w, inp, out, codes, scales, rows, np):
    """CPU baseline leg, parity part: the oracle on `rows` of the workload
    (all columns) against the GPU's output, codes and scales for the same rows
    (taken before the timed region); raises if they break the parity rule,
    returns the statistics."""
    import oracle
    ref = oracle.linear(inp, w.dtype, w.g, w.sw_dtype, w.sw_group, rows=rows)
    gc, gs = codes[rows], scales[rows]
    same_scale = (gs.view(np.uint32) == ref["scales"].view(np.uint32)) | (
        np.isnan(gs) & np.isnan(ref["scales"]))
    dc = np.abs(gc.astype(np.int32) - ref["codes"])
    go = out[rows]
    ro = ref["out"]
    if w.dtype == "f32":
        ia, ib = go.view(np.int32).astype(np.int64), ro.view(np.int32).astype(np.int64)
        top = 1 << 31
    else:
        ia, ib = go.view(np.int16).astype(np.int64), ro.view(np.int16).astype(np.int64)
        top = 1 << 15
    ia = np.where(ia < 0, -(ia + top), ia)
    ib = np.where(ib < 0, -(ib + top), ib)
    ulp = np.abs(ia - ib)
    exact_rows = same_scale & (dc.max(axis=1) == 0)
    tol = 1 if w.rank else 0
    ok = dc.max(initial=0) <= 1 and ulp[exact_rows].max(initial=0) <= tol
    res = {"rows": int(len(rows)), "cols": int(w.N),
           "codes_equal_frac": float((dc == 0).mean()), "code_flips": int((dc > 0).sum()),
           "rows_other_scale": int((~same_scale).sum()),
           "out_bit_exact_frac": float((ulp == 0).mean()),
           "out_max_ulp_rows_with_equal_codes": int(ulp[exact_rows].max(initial=0)),
           "rule": "codes within 1; outputs of rows whose codes match bit-exact"
                   + (" (1 ulp with the low-rank term)" if w.rank else ""),
           "pass": bool(ok)}
    if not ok:
        raise SystemExit(f"parity check failed on {w.name}: {res}")
    return res


def measure(name, steps, warmup, torch, np, w4, workloads, cpu=True):
    from bit_quantized_linear_rotate_amd import _binding as b
    w = workloads.WORKLOADS[name]
    inp = workloads.generate(w)
    base = _dev_inputs(w, inp, torch, np)
    sets = [_variant(base, i, torch) for i in range(4)]
    M, K, N, g = w.M, w.K, w.N, w.g
    rank = w.rank
    outs = [torch.empty((M, N), dtype=base["x"].dtype, device="cuda") for _ in sets]
    wss = [torch.empty((w4.w4a4_linear_workspace_size(M, K, N, rank),), dtype=torch.uint8,
                       device="cuda") for _ in sets]
    rq_kernel = w4.w4a4_rotate_quant_plan(base["x"], base["rot"], g, smooth=base["smooth"])
    gemm_kernel = w4.w4a4_gemm_plan(M, K, N, w.sw_group, lowrank=rank > 0)

    def step(i):
        s = sets[i % 4]
        w4.w4a4_linear(s["x"], s["rot"], g, s["w_packed"], s["w_scale"], w_scale_group=w.sw_group,
                       bias=s["bias"], smooth=s["smooth"], proj_down=s["proj_down"],
                       proj_up=s["proj_up"], workspace=wss[i % 4], out=outs[i % 4])

    # rotate+quantize alone (the kernel w4a4_linear launches first), through
    # the C ABI with prepared arguments; every return code is checked
    qbufs = [(torch.empty((M, K), dtype=torch.int8, device="cuda"),
              torch.empty((M,), dtype=torch.float32, device="cuda")) for _ in sets]
    lib = w4.lib()
    stream = torch.cuda.current_stream().cuda_stream

    def rq(i):
        s = sets[i % 4]
        c, sc = qbufs[i % 4]
        x = s["x"]
        rc = lib.w4a4_rotate_quant_rowwise(
            x.data_ptr(), _dtcode(torch, x), M, K, x.stride(0), x.stride(1), s["rot"].data_ptr(), g,
            s["smooth"].data_ptr() if s["smooth"] is not None else None, c.data_ptr(), sc.data_ptr(),
            None, stream)
        if rc:
            b._check(rc, "w4a4_rotate_quant_rowwise")

    def host(t):
        t = t.detach().cpu().contiguous()
        if t.dtype == torch.bfloat16:
            return t.view(torch.int16).numpy().view(np.uint16)
        return t.numpy()

    # ---- parity against the oracle (CPU leg), before anything is timed
    par = None
    if cpu:
        step(0)
        rq(0)
        torch.cuda.synchronize()
        rng = np.random.default_rng(7)
        nrow = min(M, 64)
        rows = np.sort(rng.choice(M, nrow, replace=False))
        if w.zero_row_frac > 0:    # the workload's planted zero rows join the sample
            zr = np.flatnonzero((inp["x"] == 0).all(axis=1))[:4]
            rows = np.unique(np.concatenate([rows, zr]))
        par = cpu_leg_parity(w, inp, host(outs[0]), host(qbufs[0][0]), host(qbufs[0][1]), rows, np)

    # ---- timed steps: exactly `steps` calls after `warmup` untimed ones,
    # synchronised on both sides
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    st = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(st)
    for i in range(steps):
        step(i)
    e1.record(st)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = e0.elapsed_time(e1) / steps

    nk = max(steps, MIN_KERNEL_LAUNCHES)
    for i in range(warmup):
        rq(i)
    t_rq = _time_each(rq, nk, torch, np)
    rq_bytes = M * K * base["x"].element_size() + M * K + 4 * M + 4 * g * g
    if w.smooth:
        rq_bytes += K * base["x"].element_size()

    # GEMM + epilogue alone, on the codes just produced, through the C ABI
    # with prepared arguments (the binding's own host time would otherwise
    # show in the loop average of a ~0.1 ms kernel)
    gws = w4.w4a4_gemm_workspace_size(M, N, K, 0)
    assert gws == 0, "the timed GEMM configurations need no workspace"
    odt = _dtcode(torch, outs[0])

    def gemm(i):
        s = sets[i % 4]
        c, sc = qbufs[i % 4]
        b_ = s["bias"]
        rc = lib.w4a4_gemm_from_codes(
            c.data_ptr(), sc.data_ptr(), M, K, s["w_packed"].data_ptr(), N, s["w_scale"].data_ptr(),
            _dtcode(torch, s["w_scale"]), w.sw_group, b_.data_ptr() if b_ is not None else None,
            _dtcode(torch, b_) if b_ is not None else 0, None, None, 0, 0, outs[i % 4].data_ptr(), odt,
            None, 0, None, 0, stream)
        if rc:
            b._check(rc, "w4a4_gemm_from_codes")
    for i in range(warmup):
        gemm(i)
    t_gemm = _time_each(gemm, nk, torch, np)
    ops = 2.0 * M * N * K
    # bytes the GEMM must move: codes, packed weights, scales, bias, output
    gemm_bytes = (M * K + N * K // 2 + 4 * M + base["w_scale"].numel() * base["w_scale"].element_size()
                  + (N * base["bias"].element_size() if base["bias"] is not None else 0)
                  + M * N * outs[0].element_size())
    # per-launch medians: the figure rocprofv3's kernel statistics agree
    # with (the mean carries the event pairs' own occasional delays)
    ms_rq, ms_gemm = t_rq["ms_median"], t_gemm["ms_median"]
    res = {
        "workload": f"{name}: M={M} K={K} N={N} g={g} {w.dtype}"
                    + (" transposed-view input" if w.transposed else "")
                    + (f" smooth+rank{rank}" if rank else "")
                    + (" per-64-group scales" if w.sw_group else ""),
        "ms_per_step": ms_step,
        "wall_s_timed_steps": wall,
        "tops": ops / (ms_step * 1e-3) / 1e12,
        "rotate_quant": {"kernel": RQ_NAMES.get(rq_kernel, rq_kernel), **t_rq,
                         "GB_s": rq_bytes / (ms_rq * 1e-3) / 1e9,
                         "frac_hbm": rq_bytes / (ms_rq * 1e-3) / 1e9 / HBM_PEAK_GBS,
                         "algorithmic_bytes": rq_bytes},
        "gemm": {"kernel": GEMM_NAMES.get(gemm_kernel, gemm_kernel), **t_gemm,
                 "TOPS": ops / (ms_gemm * 1e-3) / 1e12,
                 "frac_int8": ops / (ms_gemm * 1e-3) / 1e12 / INT8_PEAK_TOPS, "ops": ops,
                 "GB_s": gemm_bytes / (ms_gemm * 1e-3) / 1e9, "algorithmic_bytes": gemm_bytes},
    }
    if par is not None:
        res["parity"] = par
    if w.sw_group == 0 and rank == 0 and K % 128 == 0 and K >= 256 and M > 64:
        res["fp6"] = _bf6_leg(w, sets, outs, qbufs, steps, warmup, torch, np, w4, ops)
    if not w.transposed and w.dtype != "f32":
        res["hadamard"] = _hadamard_leg(w, sets, outs, wss, qbufs, steps, warmup, torch, np, w4, b, stream,
                                        rq_bytes, qmax=7)
    if rank:
        res["gemm"]["note"] = "low-rank term excluded from the GEMM-alone timing"
        # low-rank down projection alone (the first kernel of a low-rank step)
        lbufs = [torch.empty((M, rank), dtype=torch.float32, device="cuda") for _ in sets]

        def lrd(i):
            s = sets[i % 4]
            x = s["x"]
            rc = lib.w4a4_lowrank_down(x.data_ptr(), _dtcode(torch, x), M, K, x.stride(0), x.stride(1),
                                       s["proj_down"].data_ptr(), rank, lbufs[i % 4].data_ptr(), stream)
            if rc:
                b._check(rc, "w4a4_lowrank_down")

        for i in range(warmup):
            lrd(i)
        t_lrd = _time_each(lrd, nk, torch, np)
        lrd_bytes = M * K * base["x"].element_size() + K * rank * base["proj_down"].element_size() + 4 * M * rank
        res["lowrank_down"] = {"kernel": "lowrank down projection", **t_lrd,
                               "GB_s": lrd_bytes / (t_lrd["ms_median"] * 1e-3) / 1e9,
                               "frac_hbm": lrd_bytes / (t_lrd["ms_median"] * 1e-3) / 1e9 / HBM_PEAK_GBS,
                               "algorithmic_bytes": lrd_bytes}
    return w, inp, res


def _bf6_leg(w, sets, outs, qbufs, steps, warmup, torch, np, w4, ops):
    """The same GEMM on the FP6 matrix cores: the codes just produced and the
    weights as bf6 blocks (encoded once, outside the timed region), then the
    whole layer through w4a4_linear_bf6 (rotate-quant, bf6 encoding, GEMM)."""
    b6 = [(w4.w4a4_codes_to_bf6(c), sc, w4.w4a4_pack_weights_bf6(s["w_packed"]))
          for (c, sc), s in zip(qbufs, sets)]
    torch.cuda.synchronize()

    from bit_quantized_linear_rotate_amd import _binding as b
    lib = w4.lib()
    stream = torch.cuda.current_stream().cuda_stream
    M, K = sets[0]["x"].shape
    N = sets[0]["w_packed"].shape[0]
    odt = _dtcode(torch, outs[0])

    def gemm(i):
        c6, sc, w6 = b6[i % 4]
        s = sets[i % 4]
        bi = s["bias"]
        rc = lib.w4a4_gemm_bf6(c6.data_ptr(), sc.data_ptr(), M, K, w6.data_ptr(), N, s["w_scale"].data_ptr(),
                               _dtcode(torch, s["w_scale"]), bi.data_ptr() if bi is not None else None,
                               _dtcode(torch, bi) if bi is not None else 0, outs[i % 4].data_ptr(), odt, stream)
        if rc:
            b._check(rc, "w4a4_gemm_bf6")
    nk = max(steps, MIN_KERNEL_LAUNCHES)
    for i in range(warmup):
        gemm(i)
    t = _time_each(gemm, nk, torch, np)
    res = {"kernel": "w4a4_gemm_bf6_kernel (bf6 e3m2 operands, v_mfma_f32_16x16x128_f8f6f4)", **t,
           "TOPS": ops / (t["ms_median"] * 1e-3) / 1e12,
           "frac_int8_peak": ops / (t["ms_median"] * 1e-3) / 1e12 / INT8_PEAK_TOPS,
           "frac_fp6_peak": ops / (t["ms_median"] * 1e-3) / 1e12 / FP6_PEAK_TOPS}
    need = w4.w4a4_linear_bf6_workspace_size(M, K)
    wss = [torch.empty((need,), dtype=torch.uint8, device="cuda") for _ in sets]

    def step(i):
        s = sets[i % 4]
        w4.w4a4_linear_bf6(s["x"], s["rot"], w.g, b6[i % 4][2], s["w_scale"], bias=s["bias"],
                           smooth=s["smooth"], workspace=wss[i % 4], out=outs[i % 4])
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    st = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(st)
    for i in range(steps):
        step(i)
    e1.record(st)
    torch.cuda.synchronize()
    res["ms_per_step"] = e0.elapsed_time(e1) / steps
    res["tops_step"] = ops / (res["ms_per_step"] * 1e-3) / 1e12
    return res


def _hadamard_leg(w, sets, outs, wss, qbufs, steps, warmup, torch, np, w4, b, stream, rq_bytes, qmax):
    """The same workload with the rotation given by its structure (the
    normalized Hadamard the workload uses): rotate-quant alone through
    w4a4_rotate_quant_hadamard (fast Walsh-Hadamard kernel; the row-streaming
    kernel at g = 64 on many contiguous rows), and for INT4
    codes the whole layer through w4a4_linear_hadamard."""
    lib = w4.lib()
    M, K, g = w.M, w.K, w.g
    xc = _dtcode(torch, sets[0]["x"])

    def rq(i):
        s = sets[i % 4]
        c, sc = qbufs[i % 4]
        x = s["x"]
        sm = s.get("smooth")
        rc = lib.w4a4_rotate_quant_hadamard(x.data_ptr(), xc, M, K, x.stride(0), 1, g, None, None,
                                            sm.data_ptr() if sm is not None else None, qmax, c.data_ptr(),
                                            sc.data_ptr(), None, stream)
        if rc:
            b._check(rc, "w4a4_rotate_quant_hadamard")
    nk = max(steps, MIN_KERNEL_LAUNCHES)
    for i in range(warmup):
        rq(i)
    t = _time_each(rq, nk, torch, np)
    plan = w4.w4a4_rotate_quant_hadamard_plan(sets[0]["x"], g, qmax, smooth=sets[0].get("smooth"))
    name = {"row": "rq_row_kernel (R built from the signs, qmax %d)",
            "hadamard": "rq_hadamard_kernel (fast Walsh-Hadamard, qmax %d)"}[plan] % qmax
    out = {"kernel": name, **t,
           "GB_s": rq_bytes / (t["ms_median"] * 1e-3) / 1e9,
           "frac_hbm": rq_bytes / (t["ms_median"] * 1e-3) / 1e9 / HBM_PEAK_GBS}
    if qmax == 7:
        h = w4.Hadamard(g)

        def step(i):
            s = sets[i % 4]
            w4.w4a4_linear_hadamard(s["x"], h, s["w_packed"], s["w_scale"], w_scale_group=w.sw_group,
                                    bias=s["bias"], smooth=s["smooth"], proj_down=s["proj_down"],
                                    proj_up=s["proj_up"], workspace=wss[i % 4], out=outs[i % 4])
        for i in range(warmup):
            step(i)
        torch.cuda.synchronize()
        st = torch.cuda.current_stream()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(st)
        for i in range(steps):
            step(i)
        e1.record(st)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
        out["ms_per_step"] = ms
        out["tops"] = 2.0 * M * w.N * K / (ms * 1e-3) / 1e12
    return out


def measure_int8(name, steps, warmup, torch, np, w4, workloads, cpu=True):
    """The INT8 mode on the workload's shape: per-token INT8 codes (qmax =
    127) and the dynamic INT8 linear with (N, K) INT8 weights, per-channel
    weight scales in the workload's scale dtype.  The activations are the
    workload's values in contiguous rows.  Times the w8a8_linear step, the
    INT8 rotate-quant alone and the INT8 GEMM alone (same protocol as the
    W4A4 legs); the CPU leg checks sampled rows against the oracle's INT8
    linear first."""
    from bit_quantized_linear_rotate_amd import _binding as b
    w = workloads.WORKLOADS[name]
    inp = workloads.generate(w)
    M, K, N, g = w.M, w.K, w.N, w.g
    rng = np.random.default_rng(w.seed + 77)
    w8 = rng.integers(-127, 128, size=(N, K)).astype(np.int8)
    sw = workloads.f32_to_storage(rng.uniform(0.0005, 0.002, size=N).astype(np.float32), w.sw_dtype)
    x_host = np.ascontiguousarray(inp["x"])

    def d(a, dt=None):
        a = np.ascontiguousarray(a)
        if dt == "bf16":
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(a).cuda()
    base = dict(x=d(x_host, w.dtype), rot=torch.from_numpy(inp["rot"].astype(np.float32)).cuda(),
                w8=d(w8), w_scale=d(sw, w.sw_dtype), bias=d(inp["bias"], w.dtype) if w.bias else None)
    sets = [base] + [{k: (v.clone() if v is not None and k != "rot" else v) for k, v in base.items()}
                     for _ in range(3)]
    xdt = base["x"].dtype
    outs = [torch.empty((M, N), dtype=xdt, device="cuda") for _ in sets]
    need = w4.w8a8_linear_workspace_size(M, K, N)
    wss = [torch.empty((need,), dtype=torch.uint8, device="cuda") for _ in sets]
    rq_kernel = w4.w8a8_rotate_quant_plan(base["x"], base["rot"], g)
    lib = w4.lib()
    stream = torch.cuda.current_stream().cuda_stream
    xc, sc_, oc = _dtcode(torch, base["x"]), _dtcode(torch, base["w_scale"]), _dtcode(torch, outs[0])

    def step(i):
        s = sets[i % 4]
        x, b_ = s["x"], s["bias"]
        rc = lib.w8a8_linear(x.data_ptr(), xc, M, K, x.stride(0), 1, s["rot"].data_ptr(), g, None,
                             s["w8"].data_ptr(), N, s["w_scale"].data_ptr(), sc_,
                             b_.data_ptr() if b_ is not None else None, outs[i % 4].data_ptr(), oc,
                             wss[i % 4].data_ptr(), need, stream)
        if rc:
            b._check(rc, "w8a8_linear")

    qbufs = [(torch.empty((M, K), dtype=torch.int8, device="cuda"),
              torch.empty((M,), dtype=torch.float32, device="cuda")) for _ in sets]

    def rq(i):
        s = sets[i % 4]
        c, sc = qbufs[i % 4]
        x = s["x"]
        rc = lib.w8a8_rotate_quant_rowwise(x.data_ptr(), xc, M, K, x.stride(0), 1, s["rot"].data_ptr(), g,
                                           None, c.data_ptr(), sc.data_ptr(), None, stream)
        if rc:
            b._check(rc, "w8a8_rotate_quant_rowwise")

    assert w4.w8a8_gemm_workspace_size(M, N, K) == 0

    def gemm(i):
        s = sets[i % 4]
        c, sc = qbufs[i % 4]
        b_ = s["bias"]
        rc = lib.w8a8_gemm_from_codes(c.data_ptr(), sc.data_ptr(), M, K, s["w8"].data_ptr(), N,
                                      s["w_scale"].data_ptr(), sc_, b_.data_ptr() if b_ is not None else None,
                                      _dtcode(torch, b_) if b_ is not None else 0, outs[i % 4].data_ptr(), oc,
                                      None, 0, stream)
        if rc:
            b._check(rc, "w8a8_gemm_from_codes")

    par = None
    if cpu:
        import oracle
        step(0)
        rq(0)
        torch.cuda.synchronize()
        rows = np.sort(np.random.default_rng(7).choice(M, 32, replace=False))

        def host(t):
            t = t.detach().cpu().contiguous()
            return t.view(torch.int16).numpy().view(np.uint16) if t.dtype == torch.bfloat16 else t.numpy()
        out, gc, gs = host(outs[0])[rows], host(qbufs[0][0])[rows], host(qbufs[0][1])[rows]
        ref = oracle.linear_int8(x_host, inp["rot"], g, w8, sw, w.dtype, w.sw_dtype,
                                 bias=inp["bias"] if w.bias else None, rows=rows)
        same = gs.view(np.uint32) == ref["scales"].view(np.uint32)
        dc = np.abs(gc.astype(np.int32) - ref["codes"])
        exact = same & (dc.max(axis=1) == 0)
        ok = dc.max(initial=0) <= 1 and np.array_equal(out[exact].view(np.uint16),
                                                      ref["out"][exact].view(np.uint16))
        par = {"rows": int(len(rows)), "cols": int(N), "code_flips": int((dc > 0).sum()),
               "rows_other_scale": int((~same).sum()), "rows_bit_exact": int(exact.sum()),
               "rule": "codes within 1; outputs of rows whose codes match bit-exact", "pass": bool(ok)}
        if not ok:
            raise SystemExit(f"INT8 parity check failed on {name}: {par}")

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    st = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(st)
    for i in range(steps):
        step(i)
    e1.record(st)
    torch.cuda.synchronize()
    ms_step = e0.elapsed_time(e1) / steps
    nk = max(steps, MIN_KERNEL_LAUNCHES)
    for i in range(warmup):
        rq(i)
    t_rq = _time_each(rq, nk, torch, np)
    for i in range(warmup):
        gemm(i)
    t_gemm = _time_each(gemm, nk, torch, np)
    es = base["x"].element_size()
    rq_bytes = M * K * es + M * K + 4 * M + 4 * g * g
    ops = 2.0 * M * N * K
    gemm_bytes = (M * K + N * K + 4 * M + N * base["w_scale"].element_size()
                  + (N * es if w.bias else 0) + M * N * outs[0].element_size())
    ms_rq, ms_gemm = t_rq["ms_median"], t_gemm["ms_median"]
    res = {"workload": f"INT8 mode, {name} shape: M={M} K={K} N={N} g={g} {w.dtype}, contiguous rows, "
                       f"INT8 weights (N, K), per-channel {w.sw_dtype} weight scales"
                       + (", bias" if w.bias else ""),
           "ms_per_step": ms_step, "tops": ops / (ms_step * 1e-3) / 1e12,
           "rotate_quant": {"kernel": RQ_NAMES.get(rq_kernel, rq_kernel) + " (qmax 127)", **t_rq,
                            "GB_s": rq_bytes / (ms_rq * 1e-3) / 1e9,
                            "frac_hbm": rq_bytes / (ms_rq * 1e-3) / 1e9 / HBM_PEAK_GBS,
                            "algorithmic_bytes": rq_bytes},
           "gemm": {"kernel": GEMM_NAMES.get(w4.w8a8_gemm_plan(M, K, N), "?") + " (INT8 weights)", **t_gemm,
                    "TOPS": ops / (ms_gemm * 1e-3) / 1e12,
                    "frac_int8": ops / (ms_gemm * 1e-3) / 1e12 / INT8_PEAK_TOPS, "ops": ops,
                    "GB_s": gemm_bytes / (ms_gemm * 1e-3) / 1e9, "algorithmic_bytes": gemm_bytes}}
    if par is not None:
        res["parity"] = par
    res["hadamard"] = _hadamard_leg(w, [dict(s, smooth=None) for s in sets], outs, wss, qbufs, steps, warmup,
                                    torch, np, w4, b, stream, rq_bytes, qmax=127)
    return res


def measure_svdquant(steps, warmup, torch, np, w4, workloads, cpu=True):
    """The SVDQuant variant on the low-rank workload's shape and inputs
    (M=4096, K=16384, N=6144, bf16, smoothing, rank 32, per-64-group weight
    scales), as a post-GELU layer: activations floored at -0.17, the
    act_unsigned shift onto the unsigned grid, per-64-group activation
    scales, no rotation.  Times the layer step (w4a4_linear_svdquant), the
    quantizer alone and the GEMM alone; the CPU leg checks sampled rows
    against the oracle first."""
    from bit_quantized_linear_rotate_amd import _binding as b
    w = workloads.WORKLOADS["lowrank"]
    inp = workloads.generate(w)
    M, K, N, R = w.M, w.K, w.N, w.rank
    xf = np.maximum(workloads.storage_to_f32(inp["x"], w.dtype), np.float32(-0.17))
    x_host = workloads.f32_to_storage(xf, w.dtype)

    def d(a, dt=None):
        a = np.ascontiguousarray(a)
        if dt == "bf16":
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(a).cuda()
    base = dict(x=d(x_host, w.dtype), w_packed=d(inp["w_packed"]), w_scale=d(inp["s_w"], w.sw_dtype),
                smooth=d(inp["smooth"], w.dtype), down=d(inp["proj_down"], w.dtype), up=d(inp["proj_up"], w.dtype))
    sets = [base] + [{k: v.clone() for k, v in base.items()} for _ in range(3)]
    outs = [torch.empty((M, N), dtype=torch.bfloat16, device="cuda") for _ in sets]
    need = w4.w4a4_svdquant_workspace_size(M, K, N, R, 64, True)
    wss = [torch.empty((need,), dtype=torch.uint8, device="cuda") for _ in sets]
    qbufs = [(torch.empty((M, K), dtype=torch.int8, device="cuda"),
              torch.empty((M, K // 64), dtype=torch.float32, device="cuda"),
              torch.empty((M, R), dtype=torch.float32, device="cuda")) for _ in sets]
    lib = w4.lib()
    stream = torch.cuda.current_stream().cuda_stream

    def step(i):
        s_ = sets[i % 4]
        w4.w4a4_linear_svdquant(s_["x"], s_["w_packed"], s_["w_scale"], 64, smooth=s_["smooth"],
                                proj_down=s_["down"], proj_up=s_["up"], act_unsigned=True, act_group=64,
                                workspace=wss[i % 4])

    def quant(i):
        s_ = sets[i % 4]
        c, sc, _ = qbufs[i % 4]
        x = s_["x"]
        rc = lib.w4a4_quantize_svdquant(x.data_ptr(), 2, M, K, K, 1, s_["smooth"].data_ptr(), 1, 64,
                                        c.data_ptr(), sc.data_ptr(), stream)
        if rc:
            b._check(rc, "w4a4_quantize_svdquant")

    def gemm(i):
        s_ = sets[i % 4]
        c, sc, L = qbufs[i % 4]
        rc = lib.w4a4_gemm_svdquant(c.data_ptr(), sc.data_ptr(), 64, 1, M, K, s_["w_packed"].data_ptr(), N,
                                    s_["w_scale"].data_ptr(), 2, 64, None, 0, L.data_ptr(), s_["up"].data_ptr(),
                                    2, R, outs[i % 4].data_ptr(), 2, None, 0, stream)
        if rc:
            b._check(rc, "w4a4_gemm_svdquant")

    par = None
    if cpu:
        import oracle
        quant(0)
        qbufs[0][2].copy_(w4.w4a4_lowrank_down(sets[0]["x"], sets[0]["down"]))
        gemm(0)
        torch.cuda.synchronize()
        rows = np.sort(np.random.default_rng(7).choice(M, 24, replace=False))

        def host(t):
            t = t.detach().cpu().contiguous()
            return t.view(torch.int16).numpy().view(np.uint16) if t.dtype == torch.bfloat16 else t.numpy()
        gc, gs = host(qbufs[0][0])[rows], host(qbufs[0][1])[rows]
        ref = oracle.linear_svdquant(x_host, inp["w_packed"], inp["s_w"], w.dtype, w.sw_dtype, 64, inp["smooth"],
                                     None, inp["proj_down"], inp["proj_up"], act_unsigned=True, act_group=64,
                                     rows=rows)
        codes_ok = bool(np.array_equal(gc, ref["codes"]) and np.array_equal(gs.view(np.uint32),
                                                                            ref["scales"].view(np.uint32)))
        go = host(outs[0])[rows].astype(np.int64)
        ro = ref["out"].astype(np.int64)
        ia = np.where(go >= 0x8000, -(go - 0x8000), go)
        ib = np.where(ro >= 0x8000, -(ro - 0x8000), ro)
        ulp = np.abs(ia - ib)
        # the low-rank term is an fp32 sum on the GPU (L over K, l over R)
        # where the oracle rounds exact sums once: beyond one ulp an output
        # must lie within those sums' fp32 error bounds
        upv = np.abs(oracle.decode(w.dtype, inp["proj_up"]))
        S = np.abs(oracle.decode(w.dtype, x_host[rows])) @ np.abs(oracle.decode(w.dtype, inp["proj_down"]))
        bound = (R * 2.0 ** -23 * np.abs(ref["L"].astype(np.float64))) @ upv.T + (K * 2.0 ** -24 * S) @ upv.T
        diff = np.abs(oracle.decode(w.dtype, host(outs[0])[rows]) - oracle.decode(w.dtype, ref["out"]))
        ok = (ulp <= 1) | (diff <= bound)
        par = {"rows": int(len(rows)), "cols": int(N), "codes_scales_bit_exact": codes_ok,
               "out_bit_exact_frac": float((ulp == 0).mean()), "out_max_ulp": int(ulp.max()),
               "out_beyond_1ulp_within_lowrank_bound": int(((ulp > 1) & ok).sum()),
               "rule": "codes and scales bit-exact; outputs within 1 ulp, or within the fp32 summation "
                       "bound of the low-rank term",
               "pass": bool(codes_ok and ok.all())}
        if not par["pass"]:
            raise SystemExit(f"SVDQuant parity check failed: {par}")

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    st = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(st)
    for i in range(steps):
        step(i)
    e1.record(st)
    torch.cuda.synchronize()
    ms_step = e0.elapsed_time(e1) / steps
    nk = max(steps, MIN_KERNEL_LAUNCHES)
    for i in range(warmup):
        quant(i)
    t_q = _time_each(quant, nk, torch, np)
    for i in range(warmup):
        gemm(i)
    t_g = _time_each(gemm, nk, torch, np)
    q_bytes = M * K * 2 + K * 2 + M * K + M * (K // 64) * 4
    ops = 2.0 * M * N * K
    res = {"workload": f"SVDQuant layer, lowrank shape: M={M} K={K} N={N} bf16, act_unsigned shift, "
                       f"per-64-group activation and weight scales, smoothing, rank {R}, no rotation",
           "ms_per_step": ms_step, "tops": ops / (ms_step * 1e-3) / 1e12,
           "quantizer": {"kernel": "rq_svd_kernel (group 64, unsigned grid)", **t_q,
                         "GB_s": q_bytes / (t_q["ms_median"] * 1e-3) / 1e9,
                         "frac_hbm": q_bytes / (t_q["ms_median"] * 1e-3) / 1e9 / HBM_PEAK_GBS,
                         "algorithmic_bytes": q_bytes},
           "gemm": {"kernel": "w4a4_gemm_kernel (activation and weight group scales, low-rank term)", **t_g,
                    "TOPS": ops / (t_g["ms_median"] * 1e-3) / 1e12,
                    "frac_int8": ops / (t_g["ms_median"] * 1e-3) / 1e12 / INT8_PEAK_TOPS, "ops": ops}}
    if par is not None:
        res["parity"] = par
    return res


def stream_ceiling(w, steps, torch, np):
    """The HBM ceiling for rotate-quant's traffic on this device: a plain
    streaming kernel of this repository (bit_quantized_linear_rotate_amd/
    csrc/stream_probe.hip, no rotation, no quantizer) that reads the same M*K
    16-bit values and writes the same M*K + 4*M bytes, over four cycled
    buffer sets, at several grid sizes, with ordinary and with non-temporal
    stores; the best mean per launch counts."""
    import ctypes
    from bit_quantized_linear_rotate_amd import build as bld
    if not os.path.exists(bld.PROBE_LIB):
        return None
    L = ctypes.CDLL(bld.PROBE_LIB)
    L.w4a4_stream_probe.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p,
                                    ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    L.w4a4_stream_probe.restype = ctypes.c_int
    M, K = w.M, w.K
    xs = [torch.empty((M, K), dtype=torch.bfloat16, device="cuda").normal_() for _ in range(4)]
    cs = [torch.empty((M, K), dtype=torch.int8, device="cuda") for _ in range(4)]
    ss = [torch.empty((M,), dtype=torch.float32, device="cuda") for _ in range(4)]
    stream = torch.cuda.current_stream().cuda_stream
    nbytes = M * K * 2 + M * K + 4 * M
    best = None
    for nt in (0, 1):
        for grid in (2048, 4096, 8192, 16384):
            def run(i):
                rc = L.w4a4_stream_probe(xs[i % 4].data_ptr(), M * K, cs[i % 4].data_ptr(), ss[i % 4].data_ptr(),
                                         M, grid, nt, stream)
                if rc:
                    raise RuntimeError(f"stream probe: hip error {rc}")
            for i in range(5):
                run(i)
            t = _time_each(run, max(steps, MIN_KERNEL_LAUNCHES), torch, np)
            if best is None or t["ms_median"] < best[0]["ms_median"]:
                best = (t, grid, nt)
    t, grid, nt = best
    return {"kernel": "stream_probe_kernel (same bytes as rotate-quant, no arithmetic)",
            **t, "grid": grid, "nontemporal_stores": bool(nt), "bytes": nbytes,
            "GB_s": nbytes / (t["ms_median"] * 1e-3) / 1e9,
            "frac_hbm_peak": nbytes / (t["ms_median"] * 1e-3) / 1e9 / HBM_PEAK_GBS}


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


# --- counter summaries (host only): turns the rocprofv3 CSVs of the commands
# below into the text summaries under profiles/
PROFILE_COMMANDS = {
    "stats": "rocprofv3 --kernel-trace --stats --output-format csv -d $REPO/gpurun_out/prof_all -o run "
             "-- python3 $REPO/bench.py",
    "FETCH_SIZE": "rocprofv3 --pmc FETCH_SIZE --output-format csv -d $REPO/gpurun_out/pmcF -o f "
                  "-- python3 $REPO/bench.py --steps 3 --warmup 1 --no-cpu --copy-calibration",
    "WRITE_SIZE": "rocprofv3 --pmc WRITE_SIZE --output-format csv -d $REPO/gpurun_out/pmcW -o w "
                  "-- python3 $REPO/bench.py --steps 3 --warmup 1 --no-cpu --copy-calibration",
    "SQ": "rocprofv3 --pmc SQ_INSTS_VALU SQ_INSTS_MFMA SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CYCLES SQ_WAVES "
          "SQ_INSTS_LDS SQ_WAVE_CYCLES GRBM_GUI_ACTIVE --output-format csv -d $REPO/gpurun_out/pmcS -o s "
          "-- python3 $REPO/bench.py --steps 3 --warmup 1 --no-cpu",
}
N_XCD, N_SIMD = 8, 1024   # MI355X: GRBM_GUI_ACTIVE sums the 8 XCDs; 256 CUs x 4 SIMDs


def _profile_kernels():
    """(kernel name, summary stem, workload text, algorithmic bytes, ops,
    source file) of the kernels the summaries cover."""
    import workloads
    W = workloads.WORKLOADS
    es = {"bf16": 2, "f16": 2, "f32": 4}

    def rq_bytes(w):
        xs = es[w.dtype]
        return w.M * w.K * xs + w.M * w.K + 4 * w.M + 4 * w.g * w.g + (w.K * xs if w.smooth else 0)

    def gemm_bytes(w):
        sw = (w.K // 64 if w.sw_group else 1) * w.N * es[w.sw_dtype]
        return (w.M * w.K + w.N * w.K // 2 + 4 * w.M + sw + (w.N * es[w.dtype] if w.bias else 0)
                + w.M * w.N * es[w.dtype])

    def text(w):
        return (f"{w.name}: M={w.M} K={w.K} N={w.N} g={w.g} {w.dtype}"
                + (" transposed view" if w.transposed else "") + (" smoothing" if w.smooth else "")
                + (f" rank {w.rank}" if w.rank else "") + (" per-64-group scales" if w.sw_group else ""))
    p, wk, lr = W["prefill"], W["widek"], W["lowrank"]
    src = "bit_quantized_linear_rotate_amd/csrc/"
    return [
        ("void w4a4::rq_row_kernel<2, false, false, 4, 1, 7>", "rotate_quant_row_prefill_m8192_k3840_g64",
         text(p), rq_bytes(p), None, src + "rq_row.hip"),
        ("void w4a4::w4a4_gemm_pp_kernel<2>", "gemm_pingpong_prefill_m8192_k3840_n3840",
         text(p), gemm_bytes(p), 2.0 * p.M * p.N * p.K, src + "gemm.hip"),
        ("void w4a4::rq_colmajor_kernel<1, 256, false, false, 6>", "rotate_quant_colmajor_widek_m8192_k10240_g256",
         text(wk), rq_bytes(wk), None, src + "rotate_quant.hip"),
        ("void w4a4::w4a4_gemm_pp_kernel<1>", "gemm_pingpong_widek_m8192_k10240_n3840",
         text(wk), gemm_bytes(wk), 2.0 * wk.M * wk.N * wk.K, src + "gemm.hip"),
        ("void w4a4::rq_g256_kernel<2, true, 7, 1>", "rotate_quant_g256_lowrank_m4096_k16384",
         text(lr), rq_bytes(lr), None, src + "rotate_quant.hip"),
        ("void w4a4::w4a4_gemm_kernel<2, false, true, false, false>", "gemm_tile128_lowrank_m4096_k16384_n6144",
         text(lr), gemm_bytes(lr), 2.0 * lr.M * lr.N * lr.K, src + "gemm.hip"),
        ("void w4a4::lowrank_wide_kernel<2, 32>", "lowrank_down_lowrank_m4096_k16384_r32",
         text(lr), lr.M * lr.K * 2 + lr.K * lr.rank * 2 + 4 * lr.M * lr.rank, None, src + "lowrank.hip"),
        ("void (anonymous namespace)::stream_probe_kernel<true>", "stream_probe_nt_prefill_m8192_k3840",
         "streaming probe, the prefill rotate-quant's bytes (non-temporal stores)",
         p.M * p.K * 2 + p.M * p.K + 4 * p.M, None, src + "stream_probe.hip"),
        # INT8 mode (qmax 127, INT8 weights (N, K))
        ("void w4a4::rq_row_kernel<2, false, false, 4, 1, 127>", "rotate_quant_row_int8_prefill_m8192_k3840_g64",
         "INT8 mode, " + text(p), rq_bytes(p), None, src + "rq_row.hip"),
        ("void w4a4::w4a4_gemm_ring3_kernel<2, true>", "gemm_ring3_int8_weights_prefill_m8192_k3840_n3840",
         "INT8 mode, " + text(p) + ", INT8 weights",
         p.M * p.K + p.N * p.K + 4 * p.M + 2 * p.N + 2 * p.M * p.N, 2.0 * p.M * p.N * p.K, src + "gemm.hip"),
        # structured (Hadamard) rotation
        ("void w4a4::(anonymous namespace)::rq_hadamard_kernel<2, 256, true, 7, 2, 1>",
         "rotate_quant_hadamard_lowrank_m4096_k16384_g256", "Hadamard rotation, " + text(lr),
         lr.M * lr.K * 3 + 4 * lr.M + 2 * lr.K, None, src + "rq_hadamard.hip"),
        ("void w4a4::(anonymous namespace)::rq_hadamard_kernel<1, 256, false, 127, 2, 1>",
         "rotate_quant_hadamard_int8_widek_m8192_k10240_g256",
         "Hadamard rotation, INT8 mode, widek shape with contiguous rows (f16, g=256)",
         wk.M * wk.K * 3 + 4 * wk.M, None, src + "rq_hadamard.hip"),
        # SVDQuant variant
        ("void w4a4::(anonymous namespace)::rq_svd_kernel<2, 64, true, true, true>",
         "quantize_svdquant_lowrank_m4096_k16384_group64",
         "SVDQuant quantizer (act_unsigned shift, smoothing, per-64-group scales), lowrank shape",
         lr.M * lr.K * 3 + 2 * lr.K + 4 * lr.M * (lr.K // 64), None, src + "rq_svdquant.hip"),
        ("void w4a4::w4a4_gemm_kernel<2, false, true, false, true>",
         "gemm_tile128_svdquant_lowrank_m4096_k16384_n6144",
         "SVDQuant GEMM (activation and weight group scales, rank 32), lowrank shape",
         lr.M * lr.K + lr.N * lr.K // 2 + 4 * lr.M * (lr.K // 64) + 2 * (lr.K // 64) * lr.N + 2 * lr.M * lr.N
         + 4 * lr.M * lr.rank + 2 * lr.N * lr.rank, 2.0 * lr.M * lr.N * lr.K, src + "gemm.hip"),
        # FP6 (bf6) GEMM
        ("void w4a4::w4a4_gemm_bf6_kernel<2>", "gemm_bf6_prefill_m8192_k3840_n3840",
         "FP6 path, " + text(p) + ", bf6 codes and weights",
         p.M * p.K + p.N * p.K + 4 * p.M + 2 * p.N + 2 * p.M * p.N, 2.0 * p.M * p.N * p.K, src + "gemm.hip"),
    ]


def _short_name(k):
    """Kernel name without the return type and the parameter list."""
    k = k[5:] if k.startswith("void ") else k
    pre = "(anonymous namespace)::"
    head = pre if k.startswith(pre) else ""
    return head + k[len(head):].split("(")[0]


def summarize_profiles(d):
    """profiles/*.md and the two traffic .json files from the CSVs in
    directory d (prof_all/, pmcF/, pmcW/, pmcS/ as the commands above write
    them)."""
    import csv
    import glob
    import hashlib
    import statistics

    def one(pattern):
        f = glob.glob(os.path.join(d, pattern))
        if len(f) != 1:
            raise SystemExit(f"expected one file {pattern} under {d}, found {f}")
        return list(csv.DictReader(open(f[0])))

    def counters(rows):
        by = {}
        for r in rows:
            by.setdefault(r["Kernel_Name"], {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
        return by
    F = counters(one("pmcF/f_counter_collection.csv"))
    Wr = counters(one("pmcW/w_counter_collection.csv"))
    S = counters(one("pmcS/s_counter_collection.csv"))
    stats = {r["Name"]: r for r in one("prof_all/run_kernel_stats.csv")}
    copy = "__amd_rocclr_copyBuffer"
    cal_bytes = 256 << 20
    f_copy, w_copy = max(F[copy]["FETCH_SIZE"]), max(Wr[copy]["WRITE_SIZE"])
    f_scale, w_scale = cal_bytes / (f_copy * 1024), cal_bytes / (w_copy * 1024)
    out_dir = os.path.join(ROOT, "profiles")
    os.makedirs(out_dir, exist_ok=True)
    med = statistics.median
    rows_md = []
    for name, stem, wtext, alg, ops, srcf in _profile_kernels():
        full = [k for k in S if k.startswith(name)]
        if not full:
            continue
        k = full[0]
        st = stats.get(k)
        fb = med(F[k]["FETCH_SIZE"]) * 1024 * f_scale
        wb = med(Wr[k]["WRITE_SIZE"]) * 1024 * w_scale
        sq = {c: med(v) for c, v in S[k].items()}
        cyc = sq["GRBM_GUI_ACTIVE"] / N_XCD
        avg_ns = float(st["AverageNs"]) if st else None
        lines = [f"# `{_short_name(k)}` — {wtext}", "",
                 "Commands (`$REPO` is the repository root, run from `/tmp` with `TMPDIR=/tmp`), "
                 "then `python bench.py --summarize-profiles gpurun_out` on the host:", "", "```"]
        lines += [PROFILE_COMMANDS[c] for c in ("stats", "FETCH_SIZE", "WRITE_SIZE", "SQ")]
        lines += ["```", ""]
        if st:
            lines += [f"Kernel statistics (`--kernel-trace --stats`, the default bench run): {st['Calls']} calls, "
                      f"average {avg_ns / 1000:.2f} us, min {float(st['MinNs']) / 1000:.2f} us, "
                      f"max {float(st['MaxNs']) / 1000:.2f} us.", ""]
        lines += ["Counters, median per dispatch:", "", "| Counter | Value |", "|---|---|"]
        lines += [f"| FETCH_SIZE x 1024 x {f_scale:.4f} (bytes) | {fb:,.0f} |",
                  f"| WRITE_SIZE x 1024 x {w_scale:.4f} (bytes) | {wb:,.0f} |",
                  f"| algorithmic bytes | {alg:,} |",
                  f"| traffic / algorithmic | {(fb + wb) / alg:.3f} |"]
        for c in ("SQ_WAVES", "SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_LDS",
                  "SQ_BUSY_CYCLES", "SQ_WAVE_CYCLES", "GRBM_GUI_ACTIVE"):
            lines.append(f"| {c} | {sq[c]:,.0f} |")
        mfma_busy = sq["SQ_VALU_MFMA_BUSY_CYCLES"] / (cyc * N_SIMD)
        # SQ_INSTS_VALU counts the MFMA instructions too
        valu_busy = 4 * (sq["SQ_INSTS_VALU"] - sq["SQ_INSTS_MFMA"]) / (cyc * N_SIMD)
        lines += ["", "Derived (GRBM_GUI_ACTIVE / 8 = cycles of one XCD over the counter run's dispatch, "
                  "which the profiler serialises and can stretch; 1024 SIMDs):", "",
                  f"- cycles per XCD {cyc:,.0f}",
                  f"- MFMA busy {100 * mfma_busy:.1f}% of SIMD cycles (SQ_VALU_MFMA_BUSY_CYCLES)",
                  f"- non-MFMA VALU issue {100 * valu_busy:.1f}% of SIMD cycles (SQ_INSTS_VALU less "
                  f"SQ_INSTS_MFMA, 4 cycles per wave64 instruction)"]
        if avg_ns:
            lines.append(f"- algorithmic bytes / average duration: {alg / (avg_ns * 1e-9) / 1e9:,.0f} GB/s "
                         f"({100 * alg / (avg_ns * 1e-9) / 1e9 / HBM_PEAK_GBS:.1f}% of 8 TB/s)")
            if ops:
                lines.append(f"- ops / average duration: {ops / (avg_ns * 1e-9) / 1e12:,.0f} TOPS "
                             f"({100 * ops / (avg_ns * 1e-9) / 1e12 / INT8_PEAK_TOPS:.1f}% of the dense INT8 peak)")
        with open(os.path.join(out_dir, stem + ".md"), "w") as f:
            f.write("\n".join(lines) + "\n")
        rows_md.append((k, wtext, st))
        if stem in ("rotate_quant_row_prefill_m8192_k3840_g64", "gemm_pingpong_prefill_m8192_k3840_n3840"):
            with open(os.path.join(ROOT, srcf), "rb") as f:
                digest = hashlib.sha256(f.read()).hexdigest()
            rec = {"kernel": _short_name(k), "workload": "prefill", "source": srcf,
                   "source_sha256": digest, "fetch_bytes_per_launch": round(fb), "write_bytes_per_launch": round(wb),
                   "traffic_bytes_per_launch": round(fb + wb), "algorithmic_bytes_per_launch": alg,
                   "launches_counted": len(F[k]["FETCH_SIZE"]),
                   "calibration": {"copy_bytes": cal_bytes, "fetch_scale": round(f_scale, 4),
                                   "write_scale": round(w_scale, 4)},
                   "commands": [PROFILE_COMMANDS["FETCH_SIZE"], PROFILE_COMMANDS["WRITE_SIZE"]]}
            with open(os.path.join(out_dir, stem + "_traffic.json"), "w") as f:
                json.dump(rec, f, indent=1)
    # all kernels of the default run
    lines = ["# rocprofv3 kernel statistics — the default bench run (all five workloads)", "", "```",
             PROFILE_COMMANDS["stats"], "```", "",
             "| Kernel | Calls | Average us | Min us | Max us | Share |", "|---|---|---|---|---|---|"]
    for r in sorted(stats.values(), key=lambda r: -float(r["TotalDurationNs"])):
        lines.append(f"| `{_short_name(r['Name'])}` | {r['Calls']} | {float(r['AverageNs']) / 1000:.2f} | "
                     f"{float(r['MinNs']) / 1000:.2f} | {float(r['MaxNs']) / 1000:.2f} | "
                     f"{float(r['Percentage']):.1f}% |")
    with open(os.path.join(out_dir, "kernel_stats_all_workloads.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    print(f"wrote {len(rows_md) * 1 + 1} summaries under profiles/")


def _rounded(d):
    return {k: (round(v, 5) if isinstance(v, float) else _rounded(v) if isinstance(v, dict) else v)
            for k, v in d.items()}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default="prefill")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-extra", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--summarize-profiles", metavar="DIR",
                    help="write profiles/ from the rocprofv3 CSVs under DIR (host only) and exit")
    args = ap.parse_args()
    if args.summarize_profiles:
        summarize_profiles(args.summarize_profiles)
        return
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
    cpu = not args.no_cpu
    w, inp, main_res = measure(args.workload, args.steps, args.warmup, torch, np, w4, workloads,
                               cpu=cpu)
    print(f"# {args.workload}: {main_res['ms_per_step']:.4f} ms/step", file=sys.stderr, flush=True)
    extras = {}
    if not args.no_extra and args.workload == "prefill":
        for name in ("widek", "decode", "tiny", "lowrank"):
            _, _, extras[name] = measure(name, max(10, args.steps // 2), args.warmup, torch, np, w4,
                                         workloads, cpu=cpu)
            print(f"# {name}: {extras[name]['ms_per_step']:.4f} ms/step", file=sys.stderr, flush=True)
        extras["svdquant_lowrank"] = measure_svdquant(max(10, args.steps // 2), args.warmup, torch, np, w4,
                                                      workloads, cpu=cpu)
        print(f"# svdquant lowrank: {extras['svdquant_lowrank']['ms_per_step']:.4f} ms/step", file=sys.stderr,
              flush=True)
        for name in ("prefill", "widek"):
            extras["int8_" + name] = measure_int8(name, max(10, args.steps // 2), args.warmup, torch, np, w4,
                                                  workloads, cpu=cpu)
            print(f"# int8 {name}: {extras['int8_' + name]['ms_per_step']:.4f} ms/step", file=sys.stderr,
                  flush=True)
    ceiling = stream_ceiling(w, args.steps, torch, np) if w.dtype == "bf16" else None
    g = main_res["gemm"]
    rq = main_res["rotate_quant"]
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
        "parity": main_res.get("parity"),
        "rotate_quant": _rounded(rq),
        "gemm": _rounded(g),
        "roofline": {"bound": "mfma", "achieved": round(g["TOPS"], 2), "peak": INT8_PEAK_TOPS,
                     "unit": "TOPS", "frac": round(g["frac_int8"], 4),
                     "traffic": _traffic("gemm", args.workload),
                     "kernel": g["kernel"] + " (INT8 MFMA GEMM + fused scale/bias/cast epilogue)",
                     "per_launch_ms": "median of per-launch HIP event pairs"},
        "roofline_rotate_quant": {"bound": "hbm", "achieved": round(rq["GB_s"], 1),
                                  "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                  "frac": round(rq["frac_hbm"], 4),
                                  "traffic": _traffic("rotate_quant", args.workload),
                                  "kernel": rq["kernel"] + " (block rotation on MFMA, row absmax, INT4 codes)",
                                  "measured_stream_ceiling_GB_s": round(ceiling["GB_s"], 1) if ceiling else None,
                                  "frac_of_measured_ceiling": round(rq["GB_s"] / ceiling["GB_s"], 4)
                                  if ceiling else None},
        "stream_ceiling": _rounded(ceiling) if ceiling else None,
    }
    if "hadamard" in main_res:
        line["hadamard"] = _rounded(main_res["hadamard"])
    if "fp6" in main_res:
        line["fp6"] = _rounded(main_res["fp6"])
    for name, extra in extras.items():
        line[name] = {"workload": extra["workload"], "ms_per_step": round(extra["ms_per_step"], 5),
                      "tops": round(extra["tops"], 2), "parity": extra.get("parity"),
                      "gemm": _rounded(extra["gemm"])}
        for part in ("rotate_quant", "quantizer"):
            if part in extra:
                line[name][part] = _rounded(extra[part])
        if "lowrank_down" in extra:
            line[name]["lowrank_down"] = _rounded(extra["lowrank_down"])
        if "hadamard" in extra:
            line[name]["hadamard"] = _rounded(extra["hadamard"])
        if "fp6" in extra:
            line[name]["fp6"] = _rounded(extra["fp6"])
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline(w, inp, np)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
