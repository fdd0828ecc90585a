"""Benchmark of libsgemm on one MI355X.

A step is one sgemm_f32 call on the headline workload: M = N = K = 5120,
row-major fp32, A and B uniform on [-1, 1), C preloaded uniform, alpha = 1.5,
beta = 0.5 (the largest point of the square sweep).  Inputs are resident in
HBM before timing starts.  The line printed also carries:
  * roofline: the MFMA tile kernel's achieved fp32 rate against the MI355X
    dense fp32 matrix peak, from HIP events around the timed launches, and
    the HBM traffic per launch measured with rocprofv3 counters when the
    stored counter summary matches the current kernel sources;
  * parity: the whole output of one more launch of the headline compared
    with the CPU reference, element by element (max err/tol, pass);
  * cpu_baseline: the CPU reference's wall time on the host cores for that
    same whole product (the reference the parity check uses);
  * squares: 256^3 (alpha 1, beta 0), 1024^3 (alpha 1, beta 0, C preloaded)
    and every point of the square sweep 256 ... 5120 step 256 (alpha 1.5,
    beta 0.5), each timed like the headline, launches back to back, and
    each with its own parity check and CPU reference time;
  * device_copy: a plain device-to-device copy's bandwidth, the measured
    ceiling for mixed read and write traffic;
  * im2col: the six convolution-as-GEMM shapes, each timed back to back over
    rotating copies of its operands (and, for comparison, one launch at a
    time after a cache flush), with TFLOPS and the HBM bandwidth the
    algorithmic bytes imply, a parity check and the CPU reference's time;
  * conv: the convolution readings of the im2col shapes, as sconv2d_f32
    (implicit GEMM), as sgemm_im2col_f32 alone and as the lowered path
    (im2col, then sgemm_f32), with the roofline fraction of the algorithmic
    bytes (input + filters + output), a parity check and the CPU reference
    convolution's time;
  * valu_comparison and ladder: the vector-FMA kernels on the headline
    workload, the register-tile comparison kernel and each rung of the
    pages' SIMT optimisation ladder (naive ... double-buffered);
    ladder_im2col: the rungs that match page 2's five kernels on its six
    im2col shapes.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-check] [--no-im2col]
                       [--no-valu] [--no-ladder] [--no-squares] [--no-conv]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import workloads  # noqa: E402

METRIC = "SGEMM TFLOPS at 5120³ + im2col shapes; % of FP32 peak / HBM roofline"
PEAK_FP32_TFLOPS = 157.3   # MI355X dense fp32 matrix peak, and its fp32 vector peak
PEAK_HBM_GBPS = 8000.0     # MI355X HBM3E
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_counters.json")


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def source_hash() -> str:
    """Hash of the kernel sources, to tell whether stored counters still apply."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "fp32_gemm_04_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def stored_traffic(name):
    """HBM bytes per call of configuration `name` from the committed counter
    records (scaled FETCH_SIZE + WRITE_SIZE), or None if there is none or it
    was taken on other kernel sources."""
    try:
        with open(TRAFFIC_FILE) as f:
            records = json.load(f)
    except (OSError, ValueError):
        return None
    for rec in records:
        if rec.get("config") == name and rec.get("source_hash") == source_hash():
            if "FETCH_SIZE_bytes" in rec and "WRITE_SIZE_bytes" in rec:
                return round(rec["FETCH_SIZE_bytes"] + rec["WRITE_SIZE_bytes"])
    return None


def time_steps(fn, steps, warmup, stream):
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(steps):
        fn()
    end.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps  # ms


def device_operands(case):
    import torch
    A, B, C = workloads.operands(case, integer=False)
    dA = torch.from_numpy(A).cuda()
    dB = torch.from_numpy(B).cuda()
    if C is None:
        dC = torch.zeros((case.M, case.N), dtype=torch.float32, device="cuda")
    else:
        dC = torch.from_numpy(C).cuda()
    return A, B, C, dA, dB, dC


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def device_copy(stream):
    """Measured device-to-device copy bandwidth (a plain stream of reads and
    writes, the ceiling to set the skinny shapes beside): 512 MiB copies back
    to back between two buffer pairs for about 0.1 s, bytes read + written."""
    import torch
    n = 512 * 1024 * 1024 // 4
    xs = [torch.ones(n, dtype=torch.float32, device="cuda") for _ in range(2)]
    ys = [torch.empty(n, dtype=torch.float32, device="cuda") for _ in range(2)]
    for i in range(20):
        ys[i % 2].copy_(xs[i % 2])
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    reps = 100
    e0.record(stream)
    for i in range(reps):
        ys[i % 2].copy_(xs[i % 2])
    e1.record(stream)
    torch.cuda.synchronize()
    sec = e0.elapsed_time(e1) * 1e-3 / reps
    del xs, ys
    torch.cuda.empty_cache()
    return {"bytes_each_way": n * 4, "us": round(sec * 1e6, 1),
            "gbps": round(2 * n * 4 / sec / 1e9, 1),
            "frac_hbm_peak": round(2 * n * 4 / sec / 1e9 / PEAK_HBM_GBPS, 4)}


def verify(sg, case, call_args, A, B, C, dC, stream, lib=None):
    """Parity of the launch configuration just timed, and the CPU reference's
    own time on the same product.

    C is reset to its initial contents (NaN where the case does not preload
    C: beta is 0 there, so C must not be read), the library runs the product
    once, and every element of the output is compared with the CPU
    reference: |gpu - ref| <= 1e-5 * (|alpha| * sum|a*b| + |beta*c|) + 1e-6.
    The reference call is timed with the host wall clock; it computes the
    whole product, sum|a*b| included, on every host core OpenMP is given."""
    import torch
    import oracle
    lib = lib or oracle.load()
    if C is None:
        dC.fill_(float("nan"))
    else:
        dC.copy_(torch.from_numpy(C))
    torch.cuda.synchronize()
    rc = sg.sgemm_f32(*call_args)
    if rc != 0:
        raise RuntimeError(sg.sgemm_status_string(rc))
    torch.cuda.synchronize()
    out = dC.cpu().numpy()
    t0 = time.perf_counter()
    ref, absdot = oracle.sgemm(A, B, C, case.alpha, case.beta, with_absdot=True, lib=lib)
    secs = time.perf_counter() - t0
    tol = oracle.tolerance(case.alpha, case.beta, absdot, C)
    del absdot
    err = np.abs(out.astype(np.float64) - ref.astype(np.float64))
    bits = bool(np.array_equal(out.view(np.uint32), ref.view(np.uint32)))
    ratio = err / tol
    del err, tol
    worst = float(np.nanmax(ratio)) if ratio.size else 0.0
    ok = bool(np.all(ratio <= 1.0))  # NaN fails
    del ratio
    parity = {"elements": int(out.size), "pass": ok, "max_err_over_tol": round(worst, 4),
              "bit_identical_to_reference": bits}
    threads = oracle.num_threads(lib)
    cpu = {"s": round(secs, 3), "tflops": round(case.flops / secs / 1e12, 5),
           "threads": threads, "kind": "oracle", "work": "whole product with sum|a*b|"}
    return parity, cpu


def cpu_baseline(case, cpu):
    """The CPU reference's time on the headline product (whole product,
    measured by verify() in the same run), as the cpu_baseline object."""
    return {"value": cpu["tflops"], "unit": "TFLOPS", "cores": cpu["threads"], "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": "the whole %dx%dx%d product (alpha=%g, beta=%g) with its per-element "
                      "sum|a*b|, %.1f s" % (case.M, case.N, case.K, case.alpha, case.beta,
                                            cpu["s"])}


def square_timing(sg, args, stream):
    """A square configuration's time per launch (ms) and launch count: back
    to back for about 50 ms (clocks up, the launch pipeline full), then about
    20 ms of launches between two HIP events, as for the headline."""
    import torch

    def step():
        rc = sg.sgemm_f32(*args)
        if rc != 0:
            raise RuntimeError(sg.sgemm_status_string(rc))

    step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    step()
    torch.cuda.synchronize()
    once = max(time.perf_counter() - t0, 1e-6)
    t_end = time.perf_counter() + 0.05
    while time.perf_counter() < t_end:
        for _ in range(10):
            step()
        torch.cuda.synchronize()
    steps = int(min(2000, max(10, 0.02 / once)))
    return time_steps(step, steps, 0, stream), steps


def im2col_operand_sets(case, dA, dB, dC, stream):
    """Enough copies of the operands (at least 1.6 GB in all) that launches
    over them in turn read their inputs from HBM; the calls' arguments."""
    footprint = 4 * (case.M * case.K + case.K * case.N + case.M * case.N)
    nset = max(2, -(-1600 * 1024 * 1024 // footprint))
    sets = [(dA, dB, dC)] + [(dA.clone(), dB.clone(), dC.clone()) for _ in range(nset - 1)]
    calls = [(case.M, case.N, case.K, case.alpha, a.data_ptr(), case.K, b.data_ptr(),
              case.N, case.beta, c.data_ptr(), case.N, stream.cuda_stream) for a, b, c in sets]
    return sets, calls


def im2col_steady(sg, calls, stream, n=None):
    """Steady-state time per launch (ms) over the operand sets in turn: about
    0.1 s of back-to-back launches to bring the clocks up, then three runs of
    about 0.15 s of launches between two HIP events; the median run, and the
    launches per run."""
    import torch
    nset = len(calls)
    rc = sg.sgemm_f32(*calls[0])
    if rc != 0:
        raise RuntimeError(sg.sgemm_status_string(rc))
    t_end = time.perf_counter() + 0.1
    i = 0
    while time.perf_counter() < t_end:
        for _ in range(10):
            sg.sgemm_f32(*calls[i % nset])
            i += 1
        torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    if n is None:
        e0.record(stream)
        for c in calls:
            sg.sgemm_f32(*c)
        e1.record(stream)
        torch.cuda.synchronize()
        n = max(nset, int(0.15 / max(e0.elapsed_time(e1) * 1e-3 / nset, 1e-6)))
    runs = []
    for _ in range(3):
        e0.record(stream)
        for k in range(n):
            sg.sgemm_f32(*calls[k % nset])
        e1.record(stream)
        torch.cuda.synchronize()
        runs.append(e0.elapsed_time(e1) / n)
    return float(np.median(runs)), n


def bench_squares(sg, stream, check=True, known=None):
    """The square configurations: 256^3, 1024^3 and the sweep 256 ... 5120,
    each timed by square_timing."""
    import torch
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    out = []
    for case in [workloads.SMALL, workloads.SQUARE1024] + workloads.SWEEP:
        log("square", case.name)
        A, B, C, dA, dB, dC = device_operands(case)
        args = (case.M, case.N, case.K, case.alpha, dA.data_ptr(), case.K, dB.data_ptr(),
                case.N, case.beta, dC.data_ptr(), case.N, stream.cuda_stream)

        ms, steps = square_timing(sg, args, stream)
        tflops = case.flops / (ms * 1e-3) / 1e12
        entry = {"shape": [case.M, case.N, case.K], "alpha": case.alpha, "beta": case.beta,
                 "steps": steps, "us": round(ms * 1e3, 2), "tflops": round(tflops, 2),
                 "frac_fp32_peak": round(tflops / PEAK_FP32_TFLOPS, 4),
                 "kernel": sg.sgemm_plan(0, case.M, case.N, case.K, case.K, case.N, case.N,
                                         case.alpha, cus)[1]}
        if check and known and case.name in known:  # the headline, verified already
            entry["parity"], entry["cpu"] = known[case.name]
        elif check:
            log("verify", case.name)
            entry["parity"], entry["cpu"] = verify(sg, case, args, A, B, C, dC, stream)
        if check:
            entry["gpu_over_cpu"] = round(tflops / entry["cpu"]["tflops"], 1)
        out.append(entry)
        del dA, dB, dC
        torch.cuda.empty_cache()
    return out


def bench_im2col(sg, stream, reps, check=True):
    """Each im2col shape, timed two ways.

    `us` (the figure the fractions use): the steady state of back-to-back
    launches over enough copies of the operands (at least 1.6 GB in all) that
    every launch reads its inputs from HBM (im2col_steady).  Each launch also
    pays for writing back what the one before it left dirty in the caches.

    `us_tuned`: the same steady state after sgemm_tune (the library's
    autotuner) chose the kernel for the shape; `tuned_variant` is its choice
    (0: the selector's own).

    `us_single_flushed`: one launch between two events after a 512 MB read that
    evicts the caches, median of `reps`.  This reads low for kernels that
    write C with plain stores: up to the memory-side cache's size of C can
    still be dirty there when the launch ends, and the next flush writes it
    back outside the timed region."""
    import torch
    flush = torch.ones(512 * 1024 * 1024 // 4, dtype=torch.float32, device="cuda")
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    out = []
    for case in workloads.SKINNY + workloads.MID:
        log("im2col", case.name)
        A, B, C, dA, dB, dC = device_operands(case)
        sets, calls = im2col_operand_sets(case, dA, dB, dC, stream)
        nset = len(calls)
        ms, n = im2col_steady(sg, calls, stream)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        single = []
        for _ in range(reps):
            flush.sum()  # evict the caches without leaving dirty lines behind
            e0.record(stream)
            sg.sgemm_f32(*calls[0])
            e1.record(stream)
            torch.cuda.synchronize()
            single.append(e0.elapsed_time(e1))
        ms_single = float(np.median(single))
        # The library's autotuner on the same operands (sgemm_tune), then the
        # same steady-state timing with its choice; the table is reset after.
        rc, tuned_variant, _ = sg.sgemm_tune(*calls[0], 5)
        assert rc == 0, sg.sgemm_status_string(rc)
        ms_tuned, _ = im2col_steady(sg, calls, stream, n)
        sg.sgemm_tune_reset()
        tflops = case.flops / (ms * 1e-3) / 1e12
        gbps = case.alg_bytes / (ms * 1e-3) / 1e9
        roof_us = max(case.alg_bytes / (PEAK_HBM_GBPS * 1e9), case.flops / (PEAK_FP32_TFLOPS * 1e12)) * 1e6
        _, plan = sg.sgemm_plan(0, case.M, case.N, case.K, case.K, case.N, case.N, case.alpha, cus)
        entry = {}
        if check:
            log("verify", case.name)
            entry["parity"], entry["cpu"] = verify(sg, case, calls[0], A, B, C, dC, stream)
            entry["gpu_over_cpu"] = round(tflops / entry["cpu"]["tflops"], 1)
        out.append({"shape": [case.M, case.N, case.K], "us": round(ms * 1e3, 2),
                    "launches": n, "operand_sets": nset,
                    "tflops": round(tflops, 2), "hbm_gbps": round(gbps, 1),
                    "frac_hbm_peak": round(gbps / PEAK_HBM_GBPS, 4),
                    "frac_fp32_peak": round(tflops / PEAK_FP32_TFLOPS, 4),
                    "frac_roofline": round(roof_us / (ms * 1e3), 4),
                    "us_single_flushed": round(ms_single * 1e3, 2),
                    "frac_roofline_single_flushed": round(roof_us / (ms_single * 1e3), 4),
                    "us_tuned": round(ms_tuned * 1e3, 2), "tuned_variant": tuned_variant,
                    "frac_roofline_tuned": round(roof_us / (ms_tuned * 1e3), 4),
                    "kernel": plan, "traffic": stored_traffic(case.name), **entry})
        del dA, dB, dC, sets, calls
        torch.cuda.empty_cache()
    return out


def steady_state(launch, nset, stream, n=None):
    """Steady-state time per call (ms) of launch(i), i cycling over nset
    operand sets: about 0.1 s of back-to-back calls to bring the clocks up,
    then three runs of about 0.15 s between two HIP events; the median run,
    and the calls per run."""
    import torch
    launch(0)
    t_end = time.perf_counter() + 0.1
    i = 0
    while time.perf_counter() < t_end:
        for _ in range(10):
            launch(i % nset)
            i += 1
        torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    if n is None:
        e0.record(stream)
        for k in range(nset):
            launch(k)
        e1.record(stream)
        torch.cuda.synchronize()
        n = max(nset, int(0.15 / max(e0.elapsed_time(e1) * 1e-3 / nset, 1e-6)))
    runs = []
    for _ in range(3):
        e0.record(stream)
        for k in range(n):
            launch(k % nset)
        e1.record(stream)
        torch.cuda.synchronize()
        runs.append(e0.elapsed_time(e1) / n)
    return float(np.median(runs)), n


def bench_conv(sg, stream, check=True):
    """The convolution readings of the im2col shapes, three ways each:
    sconv2d_f32 (implicit GEMM: the input, the filters and the output cross
    HBM once), sgemm_im2col_f32 alone (the im2col matrix written), and the
    lowered path (sgemm_im2col_f32, then sgemm_f32 on the matrix).  Steady
    state over rotating input and output copies (at least 1.6 GB), as for
    the im2col shapes.  The convolution's whole output is compared with the
    CPU reference convolution, whose time is reported."""
    import torch
    import oracle
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    out = []
    for case in workloads.CONV_STEMS + workloads.CONV_MID:
        log("conv", case.name)
        g = case.geometry
        X, Wt, dX, dW, dY, conv = conv_sets(sg, case, stream)
        nset = len(dX)
        ms, n = steady_state(conv, nset, stream)
        _, plan = sg.sconv2d_plan(0, *g, cus)
        roof_us = max(case.alg_bytes / (PEAK_HBM_GBPS * 1e9),
                      case.flops / (PEAK_FP32_TFLOPS * 1e12)) * 1e6
        tflops = case.flops / (ms * 1e-3) / 1e12
        entry = {"name": case.name, "geometry": dict(zip(
            ["batch", "C", "H", "W", "M", "R", "S", "sh", "sw", "ph", "pw"], g)),
            "gemm_shape": [case.M, case.N, case.K], "kernel": plan,
            "us": round(ms * 1e3, 2), "calls": n, "operand_sets": nset,
            "tflops": round(tflops, 2), "alg_bytes": case.alg_bytes,
            "hbm_gbps": round(case.alg_bytes / (ms * 1e-3) / 1e9, 1),
            "frac_fp32_peak": round(tflops / PEAK_FP32_TFLOPS, 4),
            "frac_roofline": round(roof_us / (ms * 1e3), 4)}
        if plan.split()[0] in ("gemm", "tap", "direct", "tile"):
            # The other implicit forms on the same sets, for comparison: the
            # 16-tap direct form, the register-staged tile kernel and the
            # general 64 x 64 kernel.
            forms = [("general_us", sg.SCONV_VARIANT_GENERAL)]
            if plan.split()[0] in ("gemm", "tap", "direct"):
                forms.insert(0, ("tile_us", sg.SCONV_VARIANT_TILE))
            if plan.split()[0] in ("gemm", "tap"):
                forms.insert(0, ("direct_us", sg.SCONV_VARIANT_DIRECT))
            for key, v in forms:
                def other(i, v=v):
                    rc = sg.sconv2d_f32_variant(v, *g, 1.0, dX[i].data_ptr(), dW.data_ptr(),
                                                case.K, 0.0, dY[i].data_ptr(), case.N,
                                                stream.cuda_stream)
                    if rc != 0:
                        raise RuntimeError(sg.sgemm_status_string(rc))
                o_ms, _ = steady_state(other, nset, stream)
                entry[key] = round(o_ms * 1e3, 2)
        if check:
            log("verify", case.name)
            conv(0)
            torch.cuda.synchronize()
            got = dY[0].cpu().numpy()
            t0 = time.perf_counter()
            ref, absdot = oracle.conv2d(X, Wt, case.R, case.S, (case.sh, case.sw),
                                        (case.ph, case.pw))
            secs = time.perf_counter() - t0
            tol = oracle.tolerance(1.0, 0.0, absdot, None)
            ratio = np.abs(got.astype(np.float64) - ref.astype(np.float64)) / tol
            del absdot, tol
            entry["parity"] = {"elements": int(got.size), "pass": bool(np.all(ratio <= 1.0)),
                               "max_err_over_tol": round(float(np.nanmax(ratio)), 4)}
            entry["cpu"] = {"s": round(secs, 3), "tflops": round(case.flops / secs / 1e12, 5),
                            "threads": oracle.num_threads(), "kind": "oracle",
                            "work": "whole direct convolution with sum|w*x|"}
            entry["gpu_over_cpu"] = round(tflops / entry["cpu"]["tflops"], 1)
            del got, ref, ratio
        del dY
        torch.cuda.empty_cache()
        # The lowered path: im2col matrix, then the product.
        B = [torch.empty((case.K, case.N), dtype=torch.float32, device="cuda") for _ in range(2)]
        Y = torch.empty((case.M, case.N), dtype=torch.float32, device="cuda")

        def im2col(i):
            rc = sg.sgemm_im2col_f32(case.batch, case.C, case.H, case.W, case.R, case.S,
                                     case.sh, case.sw, case.ph, case.pw, dX[i % nset].data_ptr(),
                                     B[i % 2].data_ptr(), case.N, stream.cuda_stream)
            if rc != 0:
                raise RuntimeError(sg.sgemm_status_string(rc))

        def lowered(i):
            im2col(i)
            rc = sg.sgemm_f32(case.M, case.N, case.K, 1.0, dW.data_ptr(), case.K,
                              B[i % 2].data_ptr(), case.N, 0.0, Y.data_ptr(), case.N,
                              stream.cuda_stream)
            if rc != 0:
                raise RuntimeError(sg.sgemm_status_string(rc))

        im_ms, _ = steady_state(im2col, 2 * nset, stream)
        low_ms, _ = steady_state(lowered, 2 * nset, stream)
        im_bytes = 4.0 * (X.size + case.K * case.N)
        entry.update({"im2col_us": round(im_ms * 1e3, 2),
                      "im2col_hbm_gbps": round(im_bytes / (im_ms * 1e-3) / 1e9, 1),
                      "lowered_us": round(low_ms * 1e3, 2),
                      "lowered_over_conv": round(low_ms / ms, 3)})
        out.append(entry)
        del dX, B, Y, dW
        torch.cuda.empty_cache()
    return out


def bench_ladder(sg, case, call_args, stream, mfma_tflops):
    """Each rung of the pages' SIMT ladder (sgemm_f32_variant(SGEMM_VARIANT_LADDER + r))
    on the headline workload: one untimed launch, then the median of a few
    timed ones (the first rungs take a quarter of a second per launch)."""
    import torch
    out = []
    for r, name in enumerate(sg.LADDER_RUNG_NAMES):
        v = sg.SGEMM_VARIANT_LADDER + r
        log("ladder rung", r, name)
        rc = sg.sgemm_f32_variant(v, *call_args)
        assert rc == 0, sg.sgemm_status_string(rc)
        torch.cuda.synchronize()
        times = []
        for _ in range(3 if r < 2 else 9):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            sg.sgemm_f32_variant(v, *call_args)
            e1.record(stream)
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1))
        ms = float(np.median(times))
        tf = case.flops / (ms * 1e-3) / 1e12
        out.append({"rung": r, "name": name, "ms": round(ms, 3), "tflops": round(tf, 2),
                    "frac_fp32_vector_peak": round(tf / PEAK_FP32_TFLOPS, 4),
                    "mfma_over_rung": round(mfma_tflops / tf, 2)})
    return out


def bench_ladder_im2col(sg, stream):
    """The ladder rungs that match the five kernels page 2 times on the six
    im2col shapes (naive, coalesced, LDS tiles, 1-D and 2-D thread tiles):
    median of 3 launches each, in microseconds."""
    import torch
    out = []
    for case in workloads.SKINNY + workloads.MID:
        log("ladder im2col", case.name)
        _, _, _, dA, dB, dC = device_operands(case)
        args = (case.M, case.N, case.K, case.alpha, dA.data_ptr(), case.K, dB.data_ptr(),
                case.N, case.beta, dC.data_ptr(), case.N, stream.cuda_stream)
        row = {"shape": [case.M, case.N, case.K]}
        for r in range(5):
            v = sg.SGEMM_VARIANT_LADDER + r
            rc = sg.sgemm_f32_variant(v, *args)
            assert rc == 0, sg.sgemm_status_string(rc)
            times = []
            for _ in range(3):
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                sg.sgemm_f32_variant(v, *args)
                e1.record(stream)
                torch.cuda.synchronize()
                times.append(e0.elapsed_time(e1))
            row[sg.LADDER_RUNG_NAMES[r] + "_us"] = round(float(np.median(times)) * 1e3, 1)
        out.append(row)
        del dA, dB, dC
        torch.cuda.empty_cache()
    return out


def config_by_name(name):
    for case in workloads.ALL + workloads.CONV_STEMS + workloads.CONV_MID:
        if case.name == name:
            return case
    raise SystemExit("no configuration named %r (names: %s)" % (name, ", ".join(
        c.name for c in workloads.ALL + workloads.CONV_STEMS + workloads.CONV_MID)))


def conv_sets(sg, case, stream, nset=None, variant=0):
    """Rotating input/output copies of a convolution reading (at least
    1.6 GB in all, unless nset is given) and a launch(i) running
    sconv2d_f32_variant(variant) (0: what sconv2d_f32 picks) on set i."""
    import torch
    X, Wt = workloads.conv_operands(case)
    dW = torch.from_numpy(Wt).cuda()
    per_set = 4 * (X.size + case.M * case.N)
    if nset is None:
        nset = int(min(64, max(2, -(-1600 * 1024 * 1024 // per_set))))
    dX = [torch.from_numpy(X).cuda()]
    dX += [dX[0].clone() for _ in range(nset - 1)]
    dY = [torch.zeros((case.M, case.N), dtype=torch.float32, device="cuda") for _ in range(nset)]

    def launch(i):
        rc = sg.sconv2d_f32_variant(variant, *case.geometry, 1.0, dX[i].data_ptr(),
                                    dW.data_ptr(), case.K, 0.0, dY[i].data_ptr(), case.N,
                                    stream.cuda_stream)
        if rc != 0:
            raise RuntimeError(sg.sgemm_status_string(rc))
    return X, Wt, dX, dW, dY, launch


def profile_config(sg, name, stream, min_launches=50):
    """One configuration timed exactly as the full run times it (square_timing,
    or im2col_steady over rotating operand sets), for a kernel-trace run of
    its own.  The timed launches are the process's last library launches;
    the line printed says how many there were and what the HIP events gave."""
    import torch
    case = config_by_name(name)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    if isinstance(case, workloads.ConvCase):
        _, _, dX, _, _, launch = conv_sets(sg, case, stream)
        ms, n = steady_state(launch, len(dX), stream)
        print(json.dumps({"profile_config": name, "shape": [case.M, case.N, case.K],
                          "geometry": list(case.geometry), "flops": case.flops,
                          "alg_bytes": case.alg_bytes, "timed_launches": 3 * n,
                          "us_event": round(ms * 1e3, 3),
                          "kernel": sg.sconv2d_plan(0, *case.geometry, cus)[1],
                          "source_hash": source_hash()}), flush=True)
        return
    _, _, _, dA, dB, dC = device_operands(case)
    if case in workloads.SKINNY + workloads.MID:
        sets, calls = im2col_operand_sets(case, dA, dB, dC, stream)
        ms, n = im2col_steady(sg, calls, stream)
        timed = 3 * n
    else:
        args = (case.M, case.N, case.K, case.alpha, dA.data_ptr(), case.K, dB.data_ptr(),
                case.N, case.beta, dC.data_ptr(), case.N, stream.cuda_stream)

        def step():
            rc = sg.sgemm_f32(*args)
            if rc != 0:
                raise RuntimeError(sg.sgemm_status_string(rc))
        ms, steps = square_timing(sg, args, stream)
        if steps < min_launches:
            ms = time_steps(step, min_launches, 0, stream)
            steps = min_launches
        timed = steps
    print(json.dumps({"profile_config": name, "shape": [case.M, case.N, case.K],
                      "alpha": case.alpha, "beta": case.beta, "flops": case.flops,
                      "alg_bytes": case.alg_bytes, "timed_launches": timed,
                      "us_event": round(ms * 1e3, 3),
                      "kernel": sg.sgemm_plan(0, case.M, case.N, case.K, case.K, case.N, case.N,
                                              case.alpha, cus)[1],
                      "source_hash": source_hash()}), flush=True)


def summarize_profiles(root):
    """Markdown table from profile_config runs under rocprofv3: `root`/NAME.json
    holds the line profile_config printed, `root`/NAME/ the kernel trace
    (CSV).  For each library kernel, the mean duration over the timed
    launches (the last ones of the process) is set beside the HIP-event time
    per call of the same run."""
    import csv
    import glob
    rows = []
    for jpath in sorted(glob.glob(os.path.join(root, "*.json"))):
        with open(jpath) as f:
            lines = [l for l in f.read().splitlines() if l.startswith("{")]
        if not lines:
            continue
        rec = json.loads(lines[-1])
        name = rec["profile_config"]
        traces = glob.glob(os.path.join(root, name, "**", "*kernel_trace.csv"), recursive=True)
        if not traces:
            rows.append((name, rec, [], "no kernel trace"))
            continue
        with open(traces[0], newline="") as f:
            reader = csv.DictReader(f)
            keys = {k.lower(): k for k in reader.fieldnames}
            kn, ks, ke = keys["kernel_name"], keys["start_timestamp"], keys["end_timestamp"]
            disp = [(r[kn], int(r[ks]), int(r[ke])) for r in reader]
        disp.sort(key=lambda d: d[1])
        lib = [d for d in disp if "sgemm::" in d[0]]  # the library's kernels only
        per = {}
        for kname, t0, t1 in lib:
            per.setdefault(kname, []).append(t1 - t0)
        kernels = []
        for kname, durs in per.items():
            last = durs[-rec["timed_launches"]:]
            kernels.append((kname, len(last), float(np.mean(last)) / 1e3))
        kernels.sort(key=lambda k: -k[2])
        rows.append((name, rec, kernels, ""))
    out = ["| config | kernel | timed dispatches | rocprof mean (us) | sum per call (us) | "
           "HIP events per call (us) | fraction of roofline (rocprof) |",
           "|---|---|---|---|---|---|---|"]
    for name, rec, kernels, note in rows:
        if not kernels:
            out.append("| %s | %s | | | | %.2f | |" % (name, note, rec["us_event"]))
            continue
        per_call = sum(k[2] * k[1] for k in kernels) / rec["timed_launches"]
        roof = max(rec["alg_bytes"] / (PEAK_HBM_GBPS * 1e3), rec["flops"] / (PEAK_FP32_TFLOPS * 1e6))
        for i, (kname, n, us) in enumerate(kernels):
            short = kname if len(kname) < 90 else kname[:87] + "..."
            if i == 0:
                out.append("| %s | `%s` | %d | %.2f | %.2f | %.2f | %.4f |"
                           % (name, short, n, us, per_call, rec["us_event"], roof / per_call))
            else:
                out.append("| | `%s` | %d | %.2f | | | |" % (short, n, us))
    return "\n".join(out)


def conv_traffic_probe(sg, case, stream):
    """As traffic_probe, for a convolution reading: three 1 GiB copies, then
    three sconv2d_f32 calls on one input/output set."""
    import torch
    n = (1 << 30) // 4
    x = torch.ones(n, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    for _ in range(3):
        y.copy_(x)
    torch.cuda.synchronize()
    del x, y
    _, _, dX, _, _, launch = conv_sets(sg, case, stream, nset=1)
    for _ in range(3):
        launch(0)
    torch.cuda.synchronize()
    reads = 4.0 * (case.batch * case.C * case.H * case.W + case.M * case.K)
    print(json.dumps({"traffic_probe": True, "config": case.name, "copy_bytes_each_way": n * 4,
                      "shape": [case.M, case.N, case.K], "geometry": list(case.geometry),
                      "algorithmic_bytes": case.alg_bytes, "algorithmic_read_bytes": reads,
                      "algorithmic_write_bytes": 4.0 * case.M * case.N,
                      "kernel": sg.sconv2d_plan(0, *case.geometry, 256)[1],
                      "launches": 3, "source_hash": source_hash()}), flush=True)


kNumXcdCounted = 8  # GRBM_GUI_ACTIVE comes summed over the MI355X's 8 XCDs


def summarize_counters(root):
    """Counter passes over traffic_probe (or any run of a configuration):
    `root`/NAME_PASS/ holds the counter CSV of one pass for configuration
    NAME.  For the library's kernels, each counter's median over the
    dispatches, and per MFMA instruction the other instruction counts.
    Returns markdown."""
    import csv
    import glob
    per = {}  # config -> {counter: [values]}
    for d in sorted(glob.glob(os.path.join(root, "*_*"))):
        if not os.path.isdir(d):
            continue
        files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
        if not files:
            continue
        name = os.path.basename(d).rsplit("_", 1)[0]
        vals, durs = {}, {}
        with open(files[0], newline="") as f:
            reader = csv.DictReader(f)
            keys = {k.lower(): k for k in reader.fieldnames}
            for r in reader:
                if "sgemm::" not in r[keys["kernel_name"]]:
                    continue
                did = int(r[keys["dispatch_id"]])
                key = (r[keys["counter_name"]], did)
                vals[key] = vals.get(key, 0.0) + float(r[keys["counter_value"]])
                if "start_timestamp" in keys:
                    durs[did] = int(r[keys["end_timestamp"]]) - int(r[keys["start_timestamp"]])
        for (cname, did), v in vals.items():
            per.setdefault(name, {}).setdefault(cname, []).append(v)
            if cname == "GRBM_GUI_ACTIVE" and did in durs:
                # Active cycles are counted per XCD (8), summed here.
                per[name].setdefault("clock_GHz", []).append(v / kNumXcdCounted / durs[did])
        if durs:
            per[name].setdefault("duration_us (counted run)", []).extend(d / 1e3 for d in durs.values())
    out = []
    for name, counters in per.items():
        med = {c: float(np.median(v)) for c, v in counters.items()}
        out.append("### %s\n" % name)
        out.append("| counter | median per call |")
        out.append("|---|---|")
        for c in sorted(med):
            out.append("| %s | %.6g |" % (c, med[c]))
        mf = med.get("SQ_INSTS_MFMA")
        if mf:
            ratios = ["%s %.2f" % (c[9:] if c.startswith("SQ_INSTS_") else c, med[c] / mf)
                      for c in ("SQ_INSTS_VALU", "SQ_INSTS_SALU", "SQ_INSTS_VMEM_RD",
                                "SQ_INSTS_VMEM_WR", "SQ_INSTS_LDS", "SQ_INSTS_SMEM") if c in med]
            out.append("\nPer MFMA instruction: " + ", ".join(ratios) + ".")
        out.append("")
    return "\n".join(out)


def traffic_probe(sg, case, call_args, stream):
    """Launch sequence for the HBM-traffic counter passes (run under rocprofv3
    --pmc FETCH_SIZE, then WRITE_SIZE): three plain copies of 1 GiB, whose
    true read and write bytes are known, then three launches of the workload
    (the headline, or an im2col shape).  The copy's counter values give the
    scale from counter to bytes."""
    import torch
    n = (1 << 30) // 4
    x = torch.ones(n, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    for _ in range(3):
        y.copy_(x)
    torch.cuda.synchronize()
    for _ in range(3):
        rc = sg.sgemm_f32(*call_args)
        if rc != 0:
            raise RuntimeError(sg.sgemm_status_string(rc))
    torch.cuda.synchronize()
    reads = 4.0 * (case.M * case.K + case.K * case.N) + (4.0 * case.M * case.N if case.beta else 0)
    print(json.dumps({"traffic_probe": True, "config": case.name, "copy_bytes_each_way": n * 4,
                      "shape": [case.M, case.N, case.K], "alpha": case.alpha, "beta": case.beta,
                      "algorithmic_bytes": case.alg_bytes, "algorithmic_read_bytes": reads,
                      "algorithmic_write_bytes": 4.0 * case.M * case.N,
                      "kernel": sg.sgemm_plan(0, case.M, case.N, case.K, case.K, case.N, case.N,
                                              case.alpha, 256)[1],
                      "launches": 3, "source_hash": source_hash()}), flush=True)


def summarize_traffic(root):
    """HBM traffic per launch from counter passes over traffic_probe: for
    config NAME, `root`/NAME.json holds the probe's line and
    `root`/NAME_FETCH_SIZE/ and `root`/NAME_WRITE_SIZE/ the counter CSVs of
    one pass each.  Counter values are scaled by what the same counter reads
    for the probe's plain copies of known size.  Returns (markdown, records)."""
    import csv
    import glob

    def counter(path_dir, name):
        files = glob.glob(os.path.join(path_dir, "**", "*counter_collection.csv"), recursive=True)
        if not files:
            return None
        vals = {}  # dispatch -> (kernel, value)
        with open(files[0], newline="") as f:
            reader = csv.DictReader(f)
            keys = {k.lower(): k for k in reader.fieldnames}
            for r in reader:
                if r[keys["counter_name"]] != name:
                    continue
                d = int(r[keys["dispatch_id"]])
                k, v = vals.get(d, (r[keys["kernel_name"]], 0.0))
                vals[d] = (k, v + float(r[keys["counter_value"]]))
        return [vals[d] for d in sorted(vals)]

    records = []
    for jpath in sorted(glob.glob(os.path.join(root, "*.json"))):
        with open(jpath) as f:
            lines = [l for l in f.read().splitlines() if l.startswith("{")]
        if not lines:
            continue
        rec = json.loads(lines[-1])
        if not rec.get("traffic_probe"):
            continue
        name = rec["config"]
        out = dict(rec)
        for cname in ("FETCH_SIZE", "WRITE_SIZE"):
            vals = counter(os.path.join(root, "%s_%s" % (name, cname)), cname)
            if not vals:
                continue
            # The probe's 1 GiB copies are the three largest copies of the run
            # (operand set-up may add smaller ones).
            copies = sorted((v for k, v in vals if "copyBuffer" in k), reverse=True)[:3]
            lib = [(k, v) for k, v in vals if "sgemm::" in k]
            if not copies or not lib:
                continue
            expect_kib = rec["copy_bytes_each_way"] / 1024.0
            scale = expect_kib / float(np.median(copies))
            # Per call: every library kernel of one call (stream-K: two).
            per_kernel = {}
            for k, v in lib:
                per_kernel.setdefault(k, []).append(v)
            per_call_kib = sum(float(np.median(v)) for v in per_kernel.values())
            out[cname + "_KiB"] = round(per_call_kib, 1)
            out[cname + "_scale"] = round(scale, 4)
            out[cname + "_bytes"] = per_call_kib * 1024.0 * scale
            out["kernels"] = sorted(k.split("(")[0] for k in per_kernel)
        records.append(out)
    md = ["| config | kernels | FETCH_SIZE KiB | WRITE_SIZE KiB | read MB (scaled) | "
          "algorithmic read MB | written MB (scaled) | algorithmic write MB | traffic / algorithmic |",
          "|---|---|---|---|---|---|---|---|---|"]
    for r in records:
        if "FETCH_SIZE_bytes" not in r or "WRITE_SIZE_bytes" not in r:
            md.append("| %s | counters missing | | | | | | | |" % r["config"])
            continue
        tot = r["FETCH_SIZE_bytes"] + r["WRITE_SIZE_bytes"]
        md.append("| %s | %s | %.0f | %.0f | %.1f | %.1f | %.1f | %.1f | %.2f |" % (
            r["config"], ", ".join("`%s`" % k for k in r["kernels"]), r["FETCH_SIZE_KiB"],
            r["WRITE_SIZE_KiB"], r["FETCH_SIZE_bytes"] / 1e6, r["algorithmic_read_bytes"] / 1e6,
            r["WRITE_SIZE_bytes"] / 1e6, r["algorithmic_write_bytes"] / 1e6,
            tot / r["algorithmic_bytes"]))
    return "\n".join(md), records


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--no-check", "--no-cpu", dest="no_check", action="store_true",
                    help="skip the parity checks against the CPU reference and its timing")
    ap.add_argument("--no-im2col", action="store_true", help="skip the im2col shapes")
    ap.add_argument("--im2col-reps", type=int, default=20)
    ap.add_argument("--variant", type=int, default=0, help="force a kernel family (tuning)")
    ap.add_argument("--no-valu", action="store_true", help="skip the VALU-kernel comparison")
    ap.add_argument("--no-ladder", action="store_true", help="skip the SIMT-ladder table")
    ap.add_argument("--no-squares", action="store_true", help="skip the square sweep")
    ap.add_argument("--no-conv", action="store_true", help="skip the convolution readings")
    ap.add_argument("--profile-config", metavar="NAME",
                    help="only time the named configuration as the full run does (for a "
                         "kernel-trace run of its own)")
    ap.add_argument("--summarize-profiles", metavar="DIR",
                    help="print the markdown summary of profile-config runs under DIR (no GPU)")
    ap.add_argument("--traffic-probe", nargs="?", const="headline", default=None,
                    metavar="NAME|M,N,K",
                    help="only run the launch sequence for the HBM-traffic counter passes "
                         "(the headline, a configuration by name, or the im2col shape M,N,K)")
    ap.add_argument("--summarize-traffic", metavar="DIR",
                    help="print the markdown summary of traffic counter passes under DIR (no GPU)")
    ap.add_argument("--summarize-counters", metavar="DIR",
                    help="print the markdown summary of counter passes under DIR (no GPU)")
    ap.add_argument("--traffic-json", metavar="FILE",
                    help="with --summarize-traffic: also write the per-config records as JSON")
    args = ap.parse_args()

    if args.summarize_profiles:
        print(summarize_profiles(args.summarize_profiles))
        return 0
    if args.summarize_counters:
        print(summarize_counters(args.summarize_counters))
        return 0
    if args.summarize_traffic:
        md, records = summarize_traffic(args.summarize_traffic)
        print(md)
        if args.traffic_json:
            with open(args.traffic_json, "w") as f:
                json.dump(records, f, indent=1)
        return 0
    if args.gpus != 1:
        print("bench.py runs on one GPU only: libsgemm has no multi-GPU path (the product "
              "would split N across GPUs, B and C in column blocks, with no collective).",
              file=sys.stderr)
        return 2

    import torch
    import fp32_gemm_04_amd as sg

    torch.cuda.set_device(0)
    props = torch.cuda.get_device_properties(0)
    if args.profile_config:
        profile_config(sg, args.profile_config, torch.cuda.current_stream())
        return 0
    case = workloads.HEADLINE
    if args.traffic_probe not in (None, "headline"):
        if "," in args.traffic_probe:
            want = [int(v) for v in args.traffic_probe.split(",")]
            found = [c for c in workloads.SKINNY + workloads.MID if [c.M, c.N, c.K] == want]
            if not found:
                print("no im2col shape %s" % args.traffic_probe, file=sys.stderr)
                return 2
            case = found[0]
        else:
            case = config_by_name(args.traffic_probe)
            if isinstance(case, workloads.ConvCase):
                conv_traffic_probe(sg, case, torch.cuda.current_stream())
                return 0
    log("device", props.name, "CUs", props.multi_processor_count)
    A, B, C, dA, dB, dC = device_operands(case)
    stream = torch.cuda.current_stream()
    call_args = (case.M, case.N, case.K, case.alpha, dA.data_ptr(), case.K, dB.data_ptr(),
                 case.N, case.beta, dC.data_ptr(), case.N, stream.cuda_stream)

    if args.traffic_probe is not None:
        traffic_probe(sg, case, call_args, stream)
        return 0

    def step():
        rc = sg.sgemm_f32_variant(args.variant, *call_args)
        if rc != 0:
            raise RuntimeError(sg.sgemm_status_string(rc))

    # Clocks up before the counted warm-up: the inputs were just drawn on the
    # host while the GPU sat idle.  About 0.3 s of back-to-back launches.
    t_end = time.perf_counter() + 0.3
    while time.perf_counter() < t_end:
        for _ in range(10):
            step()
        torch.cuda.synchronize()
    log("timing %d steps after %d warmup" % (args.steps, args.warmup))
    ms = time_steps(step, args.steps, args.warmup, stream)
    tflops = case.flops / (ms * 1e-3) / 1e12
    _, plan = sg.sgemm_plan(args.variant, case.M, case.N, case.K, case.K, case.N, case.N,
                            case.alpha, props.multi_processor_count)
    traffic = stored_traffic(case.name)
    roofline = {"bound": "mfma", "achieved": round(tflops, 3), "peak": PEAK_FP32_TFLOPS,
                "unit": "TFLOP/s", "frac": round(tflops / PEAK_FP32_TFLOPS, 4),
                "traffic": traffic, "kernel": plan,
                "algorithmic_flops_per_launch": case.flops,
                "avg_launch_ms": round(ms, 4)}

    result = {
        "metric": METRIC, "value": round(tflops, 3), "unit": "TFLOPS", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "sgemm M=N=K=5120 row-major fp32, alpha=1.5, beta=0.5, "
                               "C preloaded, uniform[-1,1) inputs",
                   "M": case.M, "N": case.N, "K": case.K, "alpha": case.alpha,
                   "beta": case.beta, "device": props.name},
        "roofline": roofline,
    }
    if not args.no_valu:
        # The vector-FMA register-tile kernel on the same workload, for comparison.
        def valu_step():
            rc = sg.sgemm_f32_variant(sg.SGEMM_VARIANT_VALU, *call_args)
            if rc != 0:
                raise RuntimeError(sg.sgemm_status_string(rc))
        log("timing the VALU kernel")
        vms = time_steps(valu_step, max(3, args.steps // 5), 3, stream)
        vtf = case.flops / (vms * 1e-3) / 1e12
        result["valu_comparison"] = {
            "kernel": sg.sgemm_plan(sg.SGEMM_VARIANT_VALU, case.M, case.N, case.K, case.K, case.N,
                                    case.N, case.alpha, props.multi_processor_count)[1],
            "tflops": round(vtf, 3), "ms_per_step": round(vms, 4),
            "frac_fp32_peak": round(vtf / PEAK_FP32_TFLOPS, 4),
            "mfma_over_valu": round(tflops / vtf, 3)}
    if not args.no_ladder:
        result["ladder"] = bench_ladder(sg, case, call_args, stream, tflops)
        result["ladder_im2col"] = bench_ladder_im2col(sg, stream)
    known = {}
    if not args.no_check and args.variant == 0:
        log("verify the headline; CPU reference time")
        parity, cpu = verify(sg, case, call_args, A, B, C, dC, stream)
        result["parity"] = parity
        result["cpu_baseline"] = cpu_baseline(case, cpu)
        known[case.name] = (parity, cpu)
    del A, B, C
    if not args.no_squares:
        result["squares"] = bench_squares(sg, stream, check=not args.no_check, known=known)
    if not args.no_im2col:
        result["device_copy"] = device_copy(stream)
        result["im2col"] = bench_im2col(sg, stream, args.im2col_reps, check=not args.no_check)
    if not args.no_conv:
        result["conv"] = bench_conv(sg, stream, check=not args.no_check)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
