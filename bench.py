#!/usr/bin/env python3
"""Benchmark of the attention hot path on one MI355X.

A step is one pass of the workload's whole path over one batch of synthetic
input.  The default workload is the bf16 causal forward at B=2, H=32, N=8192,
d=128 (one fa_fwd per step); with --workload a fwd+bwd workload steps through
the forward and the backward stages (fa_bwd_dq, which also forms delta, then
fa_bwd_dkdv -- exactly what fa_bwd enqueues for bf16).  Inputs are resident in
device memory before the timed region starts.  The timed steps run back to
back between two HIP events on the stream the kernels run on (no event between
kernels: recording one makes the next kernel start cold); a step of several
kernels also times each kernel alone, `steps` launches between two events, so
per-kernel durations are measured live.

After the timed steps the other workloads are timed the same way and reported
in the same JSON line: the bf16 causal forward+backward at B=2, H=16, N=4096,
d=128 (per-kernel times and fractions of peak), the forward-only workloads
(bf16 N=2048 d=64, fp8 N=16384 d=128 with per-tensor scales and with e8m0
block scales), two runs with an additive bias on the scores (the N=8192
forward with a dense bias, the N=4096 forward and backward with a
sliding-window bias), the launch-bound float32 workload (N=128, in
microseconds), the HBM-bound delta kernel, and the CPU oracle on a bounded
sample of the main workload on this host's cores.

Prints ONE JSON line.  Only N=1 GPU is supported (--gpus > 1 exits).
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_TFLOPS = {"bf16": 2516.6, "fp8": 5033.2, "fp32": 157.3}  # dense, 256 CU x 2.4 GHz
PEAK_HBM_GBS = 8000.0
METRIC = "attention fwd/bwd TFLOPS (bf16, fp8) and % of MI355X MFMA peak"
MAIN = "bf16_causal_fwd_b2h32n8192d128"
FWDBWD_EXTRA = "bf16_causal_fwdbwd_b2h16n4096d128"
EXTRA = ["bf16_causal_fwd_b2h32n8192d128", "bf16_fwd_b4h16n2048d64", "fp8_fwd_b1h32n16384d128"]
MX_EXTRA = ("mxfp8_fwd_b1h32n16384d128", (1, 32, 16384, 128))
# Additive bias on the scores (one [N, N] float32 bias shared by every batch
# entry and head): (name, shape, causal, bias kind, window, with backward)
BIAS_EXTRA = [
    ("bf16_causal_fwd_densebias_b2h32n8192d128", (2, 32, 8192, 128), True, "dense", 0, False),
    ("bf16_causal_fwdbwd_windowbias_b2h16n4096d128", (2, 16, 4096, 128), True, "window", 1023,
     True),
]


# The sources each timed kernel is built from (with the build flags): a
# counter figure stays valid while these files are unchanged.
STAGE_SOURCES = {
    "fwd": ["csrc/fwd_bf16.hip", "csrc/fa_device.h", "csrc/fa_kernels.h", "build.py"],
    "delta": ["csrc/f32_kernels.hip", "csrc/fa_device.h", "csrc/fa_kernels.h", "build.py"],
    "dkdv": ["csrc/bwd_bf16.hip", "csrc/fa_device.h", "csrc/fa_kernels.h", "build.py"],
    "dq": ["csrc/bwd_bf16.hip", "csrc/fa_device.h", "csrc/fa_kernels.h", "build.py"],
}


def source_hash(stage: str) -> str:
    """sha256 over the files a stage's kernel is built from (name + bytes)."""
    import hashlib

    h = hashlib.sha256()
    for rel in STAGE_SOURCES[stage]:
        h.update(rel.encode())
        with open(os.path.join(ROOT, "exact_io_aware_11_amd", rel), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(workload: str, stage: str):
    """HBM bytes per launch of `stage` on `workload` from the committed
    rocprofv3 counter summary (FETCH_SIZE and WRITE_SIZE, scaled by a
    copy-kernel calibration), or None if none was taken for that pair or it
    was taken on other sources of that kernel."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    try:
        with open(path) as fh:
            t = json.load(fh)
    except (OSError, ValueError):
        return None
    st = t.get("workloads", {}).get(workload, {}).get("stages", {}).get(stage)
    if st is None or stage not in STAGE_SOURCES:
        return None
    if st.get("source_sha256") != source_hash(stage):
        return None
    return st["bytes_per_launch"]


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def device_inputs(w, with_dout):
    import torch

    import fa_inputs

    inp = fa_inputs.make_inputs(w.shape, w.dtype, seed=42, with_dout=with_dout)

    def dev(a):
        t = torch.from_numpy(a)
        if w.dtype == "bf16":
            t = t.view(torch.int16).view(torch.bfloat16)
        return t.cuda()

    q, k, v = dev(inp.q), dev(inp.k), dev(inp.v)
    do = dev(inp.dout) if with_dout else None
    return inp, q, k, v, do


def algorithmic_work(w):
    """Per-stage algorithmic FLOPs (bytes for the delta kernel)."""
    import exact_io_aware_11_amd as fa

    B, H, N, d, c = w.B, w.H, w.N, w.d, w.causal
    per_product = 2.0 * B * H * N * N * d / (2 if c else 1)
    elt = {"fp32": 4, "bf16": 2, "fp8": 1}[w.dtype]
    return {
        "fwd": fa.flops_fwd(B, H, N, d, c),
        # dK/dV kernel: S recompute, dV, dP, dK; dQ kernel: the dQ product
        # (its S and dP recomputes, and for bf16 delta, are not counted)
        "dkdv": 4 * per_product,
        "dq": 1 * per_product,
        # delta kernel: reads O and dO, writes one float per row
        "delta_bytes": 2.0 * B * H * N * d * elt + 4.0 * B * H * N,
    }


def warm_until(fn, seconds):
    """Repeat fn until `seconds` of wall time have passed.  The GPU's power
    management raises the shader clock over the first few hundred ms of
    sustained load; timing before that measures the ramp, not the kernel."""
    import torch

    t0 = time.perf_counter()
    n = 0
    while True:
        fn()
        n += 1
        if n % 4 == 0:
            torch.cuda.synchronize()
            if time.perf_counter() - t0 >= seconds:
                return n


def time_main(w, steps, warmup, warm_s=0.0):
    import torch

    import exact_io_aware_11_amd as fa

    inp, q, k, v, do = device_inputs(w, w.backward)
    B, H, N, d = w.shape
    odt = torch.float32 if w.dtype == "fp32" else torch.bfloat16
    o = torch.empty((B, H, N, d), dtype=odt, device="cuda")
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    if w.backward:
        dq, dk, dv = (torch.empty_like(q) for _ in range(3))
        ws = torch.empty(fa.fa_bwd_workspace_size(B, H, N, d), dtype=torch.uint8, device="cuda")
    # the stages fa_bwd enqueues: for bf16 the dQ kernel forms delta itself
    bwd_stages = ["dq", "dkdv"] if w.dtype == "bf16" else ["delta", "dkdv", "dq"]
    stages = ["fwd"] + (bwd_stages if w.backward else [])
    calls = {"delta": fa.fa_bwd_delta, "dkdv": fa.fa_bwd_dkdv, "dq": fa.fa_bwd_dq}

    args = (q, k, v, o, do, lse, dq, dk, dv, ws, w.scale, w.causal) if w.backward else None

    def run_stage(s):
        if s == "fwd":
            fa.fa_fwd(q, k, v, o, lse, w.scale, w.causal, descale=inp.descale)
        else:
            calls[s](*args)

    def step():
        for s in stages:
            run_stage(s)

    # The timed steps run back to back between two events, with no event in
    # between: recording one between two kernels makes the next start cold
    # (~45 us on the N=8192 forward), which would be timed as the step's.  A
    # step of one kernel is therefore its average launch duration (gaps
    # included).  A step of several kernels is timed the same way, and each
    # kernel's average launch duration comes from `steps` launches of that
    # kernel alone between two events right after (each stage only reads what
    # the stages before it wrote, so repeating it changes nothing).
    # Every event is created (recorded once) before the warm-up, so nothing is
    # allocated between the warm-up and the timed steps and the GPU does not
    # sit idle there.  (After an idle gap of tens of ms the chip boosts its
    # clock, overshoots its power limit and takes ~20 launches of this kernel
    # to settle: steps timed in that window measure the power controller.)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    sev = {s: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for s in stages}
    for e in [start, end] + [x for pair in sev.values() for x in pair]:
        e.record()
    for _ in range(warmup):
        step()
    n_warm, tw = 0, time.perf_counter()
    if warm_s > 0:
        n_warm = warm_until(step, warm_s)
    torch.cuda.synchronize()
    step_s = (time.perf_counter() - tw) / n_warm if n_warm else 0.0
    # A queue of about 40 ms of untimed steps ahead of the start event: the
    # host then enqueues the timed steps while the GPU is still busy, so a
    # stall of the host thread (seen on fresh machines: 30+ ms inside the
    # loop, the GPU idle meanwhile and then ramping its clock back) cannot
    # leave the GPU without work inside the timed region.  The timed region
    # is still exactly `steps` steps between two events on the stream.
    ahead = min(200, int(math.ceil(0.04 / step_s))) if step_s > 0 else 0
    for _ in range(ahead):
        step()
    t0 = time.perf_counter()
    start.record()
    for _ in range(steps):
        step()
    end.record()
    if len(stages) > 1:
        for s in stages:
            a, b = sev[s]
            a.record()
            for _ in range(steps):
                run_stage(s)
            b.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    total_ms = start.elapsed_time(end)
    if len(stages) == 1:
        per = {stages[0]: total_ms / steps}
    else:
        per = {s: sev[s][0].elapsed_time(sev[s][1]) / steps for s in stages}
    return total_ms / steps, wall, per


def time_calls(fn, reps, warmup, warm_s=0.0, batches=5):
    """Mean and median time per call of fn after warm-up: `batches` batches
    of about reps/batches back-to-back calls, each batch between two events
    (an event between every two calls would be timed too: recording one makes
    the next kernel start cold, ~45 us on the N=8192 forward); the mean over
    all calls and the median of the batch means."""
    import torch

    batches = max(1, min(batches, reps))
    per_batch = max(1, reps // batches)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(batches)]
    for a, b in evs:  # created before the warm-up (see time_main)
        a.record()
        b.record()
    for _ in range(warmup):
        fn()
    n_warm, tw = 0, time.perf_counter()
    if warm_s > 0:
        n_warm = warm_until(fn, warm_s)
    torch.cuda.synchronize()
    if n_warm:  # ~40 ms of untimed calls queued ahead (see time_main)
        per = (time.perf_counter() - tw) / n_warm
        for _ in range(min(200, int(math.ceil(0.04 / per)))):
            fn()
    for a, b in evs:
        a.record()
        for _ in range(per_batch):
            fn()
        b.record()
    torch.cuda.synchronize()
    ms = sorted(a.elapsed_time(b) / per_batch for a, b in evs)
    return sum(ms) / len(ms), ms[len(ms) // 2]


def time_delta(w, reps, warmup, warm_s=0.0):
    """The standalone delta kernel (fa_bwd_delta: delta_i = dO_i . O_i, HBM-bound) on the
    workload's shape; the bf16 backward forms delta inside its dQ kernel instead.  Thirty
    back-to-back calls between two events, cycling over six (O, dO) pairs -- 384 MiB at the
    default shape, more than the 256 MB last-level cache -- so that every call reads HBM and
    the event overhead is spread; returns the mean and median time per call."""
    import torch

    import exact_io_aware_11_amd as fa

    B, H, N, d = w.shape
    g = torch.Generator(device="cuda").manual_seed(7)
    pairs = [tuple(torch.randn((B, H, N, d), generator=g, device="cuda").to(torch.bfloat16)
                   for _ in range(2)) for _ in range(6)]
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    ws = torch.empty(fa.fa_bwd_workspace_size(B, H, N, d), dtype=torch.uint8, device="cuda")
    calls = 30

    def run():
        for i in range(calls):
            o, do = pairs[i % len(pairs)]
            # (q, k, v and the gradients are neither read nor written by this stage)
            fa.fa_bwd_delta(o, o, o, o, do, lse, o, o, o, ws, w.scale, w.causal)

    mean, med = time_calls(run, reps, warmup, warm_s)
    del pairs, lse, ws
    torch.cuda.empty_cache()
    return mean / calls, med / calls


def time_fwd_only(w, reps, warmup, warm_s=0.0):
    import torch

    import exact_io_aware_11_amd as fa

    inp, q, k, v, _ = device_inputs(w, False)
    B, H, N, d = w.shape
    o = torch.empty((B, H, N, d), dtype=torch.bfloat16 if w.dtype != "fp32" else torch.float32,
                    device="cuda")
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    res = time_calls(lambda: fa.fa_fwd(q, k, v, o, lse, w.scale, w.causal, descale=inp.descale),
                     reps, warmup, warm_s)
    del q, k, v, o, lse
    torch.cuda.empty_cache()
    return res


SCHEDULES = ["interleaved", "pingpong", "rows64"]


def time_schedules(reps, rounds=3, warm_s=0.5):
    """The forward schedules (FA_FWD_SCHEDULE) on the headline shape, causal
    and not: the same inputs, the schedules timed in turn for `rounds` rounds
    of `reps` back-to-back calls (so clock drift hits all alike); per schedule
    the median of its rounds' means."""
    import statistics

    import torch

    import exact_io_aware_11_amd as fa
    import fa_inputs

    w = fa_inputs.WORKLOADS[MAIN]
    inp, q, k, v, _ = device_inputs(w, False)
    o = torch.empty(w.shape, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(w.shape[:3], dtype=torch.float32, device="cuda")
    out = {}
    saved = os.environ.get("FA_FWD_SCHEDULE")
    try:
        for causal in (True, False):
            ms = {sched: [] for sched in SCHEDULES}
            for r in range(rounds):
                for sched in SCHEDULES:
                    os.environ["FA_FWD_SCHEDULE"] = sched
                    mean, _ = time_calls(
                        lambda: fa.fa_fwd(q, k, v, o, lse, w.scale, causal, descale=inp.descale),
                        reps, 2, warm_s if r == 0 else 0.0)
                    ms[sched].append(mean)
            flops = fa.flops_fwd(w.B, w.H, w.N, w.d, causal)
            name = w.name if causal else w.name.replace("_causal", "")
            out[name] = {}
            for sched in SCHEDULES:
                m = statistics.median(ms[sched])
                out[name][sched] = {"ms": round(m, 4),
                                    "TFLOP/s": round(flops / (m * 1e-3) / 1e12, 1)}
    finally:
        if saved is None:
            os.environ.pop("FA_FWD_SCHEDULE", None)
        else:
            os.environ["FA_FWD_SCHEDULE"] = saved
    del q, k, v, o, lse
    torch.cuda.empty_cache()
    return out


def measure_mfma_rates(warm_s=0.5, reps=10):
    """The matrix-core rate on realistic operand bits (fa_measure_mfma_rate:
    pure 32x32 products on pseudo-random per-lane data, two waves per SIMD on
    every CU), after warm-up: the measured ceiling beside the published peak."""
    import torch

    import exact_io_aware_11_amd as fa

    cus = torch.cuda.get_device_properties(0).multi_processor_count
    blocks, iters = 8 * cus, 2048
    out = torch.empty(blocks * 512, dtype=torch.float32, device="cuda")
    rates = {}
    for name, fp8 in (("bf16", False), ("fp8", True)):
        flops = fa.fa_measure_mfma_rate(out, blocks, iters, fp8)
        mean, _ = time_calls(lambda: fa.fa_measure_mfma_rate(out, blocks, iters, fp8), reps, 2,
                             warm_s)
        rates[name] = round(flops / (mean * 1e-3) / 1e12, 1)
    del out
    return rates


def time_small_fp32(reps=50):
    """The float32 workload (one head, N=128, d=64, fwd+bwd): four 32-row
    workgroups per kernel, so launch latency dominates; reported in microseconds."""
    import torch

    import exact_io_aware_11_amd as fa

    w = __import__("fa_inputs").WORKLOADS["fp32_fwdbwd_b1h1n128d64"]
    inp, q, k, v, do = device_inputs(w, True)
    B, H, N, d = w.shape
    o = torch.empty((B, H, N, d), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    dq, dk, dv = (torch.empty_like(q) for _ in range(3))
    ws = torch.empty(fa.fa_bwd_workspace_size(B, H, N, d), dtype=torch.uint8, device="cuda")
    f_mean, f_med = time_calls(lambda: fa.fa_fwd(q, k, v, o, lse, w.scale, w.causal), reps, 5)
    b_mean, b_med = time_calls(
        lambda: fa.fa_bwd(q, k, v, o, do, lse, dq, dk, dv, ws, w.scale, w.causal), reps, 5)
    return {"fwd_us": round(f_mean * 1e3, 2), "fwd_us_median": round(f_med * 1e3, 2),
            "bwd_us": round(b_mean * 1e3, 2), "bwd_us_median": round(b_med * 1e3, 2),
            "note": "event-timed on the stream; launch-bound (4 workgroups per kernel)"}


def time_fwd_mx(shape, reps, warmup, warm_s=0.0):
    """The microscaled fp8 forward (one e8m0 scale per 32 elements along each
    product's contraction) on the same shape as the per-tensor fp8 line."""
    import torch

    import exact_io_aware_11_amd as fa
    import fa_inputs

    B, H, N, d = shape
    mx = fa_inputs.make_mx_inputs(shape, seed=42)
    q, k, v, qs, ks, vs = (torch.from_numpy(a).cuda() for a in (mx.q, mx.k, mx.v, mx.qs, mx.ks,
                                                                 mx.vs))
    o = torch.empty(shape, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    scale = 1.0 / math.sqrt(d)
    res = time_calls(lambda: fa.fa_fwd_mxfp8(q, k, v, qs, ks, vs, o, lse, scale, False),
                     reps, warmup, warm_s)
    del q, k, v, qs, ks, vs, o, lse
    torch.cuda.empty_cache()
    return res


def time_bias(shape, causal, kind, window, backward, reps, warmup, warm_s=0.0):
    """fa_fwd_bias (and fa_bwd_bias) with a shared [N, N] bias drawn by
    fa_inputs.draw_bias (N(0,1); "dense": 10 % -inf, "window": -inf before the
    last window+1 keys).  The kernels apply the bias element by element, so the
    algorithmic FLOPs are those of the unbiased problem."""
    import torch

    import exact_io_aware_11_amd as fa
    import fa_inputs

    B, H, N, d = shape
    inp = fa_inputs.make_inputs(shape, "bf16", seed=42, with_dout=backward)

    def dev(a):
        return torch.from_numpy(a).view(torch.int16).view(torch.bfloat16).cuda()

    q, k, v = dev(inp.q), dev(inp.k), dev(inp.v)
    bias = torch.from_numpy(fa_inputs.draw_bias((1, 1), N, seed=7, kind=kind,
                                                window=window)).cuda()[..., :N]
    o = torch.empty(shape, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    scale = 1.0 / math.sqrt(d)
    out = {}
    mean, med = time_calls(lambda: fa.fa_fwd_bias(q, k, v, bias, o, lse, scale, causal),
                           reps, warmup, warm_s)
    out["fwd"] = {"ms": round(mean, 4), "ms_median": round(med, 4),
                  "TFLOP/s": round(fa.flops_fwd(B, H, N, d, causal) / (mean * 1e-3) / 1e12, 1)}
    if backward:
        do = dev(inp.dout)
        dq, dk, dv = (torch.empty_like(q) for _ in range(3))
        ws = torch.empty(fa.fa_bwd_workspace_size(B, H, N, d), dtype=torch.uint8, device="cuda")
        mean, med = time_calls(
            lambda: fa.fa_bwd_bias(q, k, v, bias, o, do, lse, dq, dk, dv, ws, scale, causal),
            reps, warmup, warm_s)
        out["bwd"] = {"ms": round(mean, 4), "ms_median": round(med, 4),
                      "TFLOP/s": round(fa.flops_bwd(B, H, N, d, causal) / (mean * 1e-3) / 1e12,
                                       1)}
        del do, dq, dk, dv, ws
    del q, k, v, bias, o, lse
    torch.cuda.empty_cache()
    return out


IO_COMPARE = ["bf16_fwd_b4h16n2048d64", "bf16_causal_fwdbwd_b2h16n4096d128"]


def time_io_compare(reps, warmup, warm_s=0.0):
    """The forward by fa_fwd (S and P stay on chip) and by fa_std_fwd, the
    standard attention that writes S (float32) and P (bf16) to device memory
    and reads them back, on the same inputs.  Returns per-workload times and
    the algorithmic device-memory bytes of each: Q, K, V read once, O and LSE
    written once, plus for the standard form S written and read and P written
    and read (N x ldp entries per head)."""
    import torch

    import exact_io_aware_11_amd as fa
    import fa_inputs

    out = {}
    for name in IO_COMPARE:
        w = fa_inputs.WORKLOADS[name]
        _, q, k, v, _ = device_inputs(w, False)
        B, H, N, d = w.shape
        o = torch.empty_like(q)
        lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
        ws = torch.empty(fa.fa_std_workspace_size(B, H, N, d), dtype=torch.uint8, device="cuda")
        f_mean, f_med = time_calls(lambda: fa.fa_fwd(q, k, v, o, lse, w.scale, w.causal), reps,
                                   warmup, warm_s)
        s_mean, s_med = time_calls(
            lambda: fa.fa_std_fwd(q, k, v, o, lse, ws, w.scale, w.causal), reps, warmup, warm_s)
        ldp = (N + 63) // 64 * 64
        io = 4 * B * H * N * d * 2 + 4 * B * H * N  # Q, K, V, O (bf16) and LSE
        nn = B * H * N * ldp
        std_io = io + 2 * nn * 4 + 2 * nn * 2      # + S written, read; P written, read
        flops = fa.flops_fwd(B, H, N, d, w.causal)
        out[name] = {"flash_ms": round(f_mean, 4), "flash_ms_median": round(f_med, 4),
                     "flash_TFLOP/s": round(flops / (f_mean * 1e-3) / 1e12, 1),
                     "standard_ms": round(s_mean, 4), "standard_ms_median": round(s_med, 4),
                     "standard_TFLOP/s": round(flops / (s_mean * 1e-3) / 1e12, 1),
                     "speedup": round(s_mean / f_mean, 2),
                     "algorithmic_bytes_flash": io, "algorithmic_bytes_standard": std_io}
        log(f"io comparison {name}: {out[name]}")
        del q, k, v, o, lse, ws
        torch.cuda.empty_cache()
    return out


def cpu_baseline(w, max_heads):
    """The oracle as it stands on a bounded sample: whole heads of the workload."""
    import numpy as np

    import exact_io_aware_11_amd as fa
    import fa_inputs
    import oracle

    oracle.build(force=False)
    inp = fa_inputs.make_inputs((1, max_heads, w.N, w.d), w.dtype, seed=42,
                                with_dout=w.backward)

    def exact(a, s=1.0):
        if w.dtype == "fp32":
            return a.astype(np.float64)
        if w.dtype == "bf16":
            return oracle.decode_bf16(a)
        return oracle.decode_e4m3fn(a, s)

    qs, ks, vs = (exact(x, s) for x, s in zip((inp.q, inp.k, inp.v), inp.descale))
    threads = oracle.default_threads()
    t0 = time.perf_counter()
    oracle.attn_fwd(qs, ks, vs, w.scale, w.causal, nthreads=threads)
    flops = fa.flops_fwd(1, max_heads, w.N, w.d, w.causal)
    if w.backward:
        oracle.attn_bwd(qs, ks, vs, exact(inp.dout), w.scale, w.causal, nthreads=threads)
        flops += fa.flops_bwd(1, max_heads, w.N, w.d, w.causal)
    sec = time.perf_counter() - t0
    return {"value": flops / sec / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "seconds": round(sec, 3),
            "sample": f"{max_heads} of {w.B * w.H} heads at full N={w.N}, d={w.d} "
                      f"({'fwd+bwd' if w.backward else 'fwd'}), float64 naive oracle"}


def calibrate_copy(nbytes: int = 1 << 30, reps: int = 3):
    """A plain device-to-device copy of known size: each launch reads and
    writes nbytes.  Profiling it with the HBM byte counters gives the factor
    that turns counter readings into bytes."""
    import torch

    src = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        dst.copy_(src)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / reps
    print(json.dumps({"copy_bytes_read": nbytes, "copy_bytes_written": nbytes, "reps": reps,
                      "ms": round(ms, 4), "GB/s": round(2 * nbytes / (ms * 1e-3) / 1e9, 1)}),
          flush=True)


def step_report(w, ms, per):
    """Whole-step TFLOP/s, per-kernel figures and the roofline of the dominant
    kernel (the one with the largest share of the step) for one timed workload."""
    work = algorithmic_work(w)
    total_flops = work["fwd"] + (work["dkdv"] + work["dq"] if w.backward else 0.0)
    peak = PEAK_TFLOPS[w.dtype]
    kernels = {}
    for s, t in per.items():
        if s == "delta":
            gbs = work["delta_bytes"] / (t * 1e-3) / 1e9
            kernels[s] = {"ms": round(t, 4), "GB/s": round(gbs, 1),
                          "frac_hbm": round(gbs / PEAK_HBM_GBS, 4)}
        else:
            tf = work[s] / (t * 1e-3) / 1e12
            kernels[s] = {"ms": round(t, 4), "TFLOP/s": round(tf, 1), "frac": round(tf / peak, 4)}
            if s == "dq":  # it also recomputes S and dP: three products executed, one credited
                kernels[s]["executed_TFLOP/s"] = round(3 * tf, 1)
    dom = max(per, key=per.get)
    if dom == "delta":
        ach = work["delta_bytes"] / (per[dom] * 1e-3) / 1e9
        roof = {"kernel": "delta", "bound": "hbm", "achieved": round(ach, 1),
                "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(ach / PEAK_HBM_GBS, 4)}
    else:
        ach = work[dom] / (per[dom] * 1e-3) / 1e12
        roof = {"kernel": dom, "bound": "mfma", "achieved": round(ach, 1), "peak": peak,
                "unit": "TFLOP/s", "frac": round(ach / peak, 4)}
    roof["traffic"] = measured_traffic(w.name, dom)
    return total_flops / (ms * 1e-3) / 1e12, kernels, roof


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--warm-seconds", type=float, default=1.5,
                    help="after the warmup steps, keep stepping (untimed) until this much "
                         "wall time has passed, so that the shader clock has settled")
    ap.add_argument("--workload", default=MAIN)
    ap.add_argument("--no-extra", action="store_true", help="skip the forward-only workloads")
    ap.add_argument("--rate-probe", action="store_true",
                    help="time the matrix-core rate probe also with --no-extra")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-heads", type=int, default=0,
                    help="heads the CPU oracle runs (0: all B*H heads of the workload)")
    ap.add_argument("--io-compare", action="store_true",
                    help="only time fa_fwd against the standard attention fa_std_fwd (S and P "
                         "in device memory) on the two IO-comparison workloads")
    ap.add_argument("--hbm-calibrate", action="store_true",
                    help="only run a plain 1 GiB device copy (reference for HBM counters)")
    ap.add_argument("--bias-only", action="store_true",
                    help="only time the workloads with an additive bias (for profiling them)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: every (batch, head) is independent, so "
              "several GPUs would each run this same kernel on their share of heads; "
              "there is no multi-GPU mode.", file=sys.stderr)
        sys.exit(2)

    import torch

    if args.hbm_calibrate:
        calibrate_copy()
        return

    import exact_io_aware_11_amd as fa  # noqa: F401  (fails loudly without libfa.so)
    import fa_inputs

    if args.io_compare:
        print(json.dumps({"io_comparison": time_io_compare(max(3, args.steps), args.warmup)}),
              flush=True)
        return

    if args.bias_only:
        out = {}
        for name, shape, causal, kind, window, backward in BIAS_EXTRA:
            out[name] = time_bias(shape, causal, kind, window, backward, max(3, args.steps),
                                  args.warmup, args.warm_seconds)
        print(json.dumps({"bias_workloads": out}), flush=True)
        return

    w = fa_inputs.WORKLOADS[args.workload]
    log(f"workload {w.name} steps={args.steps} warmup={args.warmup}")
    ms, wall, per = time_main(w, args.steps, args.warmup, args.warm_seconds)
    value, kernels, roof = step_report(w, ms, per)
    peak = PEAK_TFLOPS[w.dtype]
    log(f"step {ms:.3f} ms  {value:.1f} TFLOP/s  kernels {kernels}")

    fwdbwd = {}
    if not args.no_extra and w.name != FWDBWD_EXTRA:
        x = fa_inputs.WORKLOADS[FWDBWD_EXTRA]
        x_ms, _, x_per = time_main(x, args.steps, min(args.warmup, 3),
                                   min(args.warm_seconds, 1.0))
        x_value, x_kernels, x_roof = step_report(x, x_ms, x_per)
        fwdbwd[x.name] = {"ms_per_step": round(x_ms, 4), "TFLOP/s": round(x_value, 1),
                          "frac_of_peak": round(x_value / PEAK_TFLOPS[x.dtype], 4),
                          "passes": "fwd+bwd", "kernels": x_kernels, "roofline": x_roof}
        log(f"{x.name}: step {x_ms:.3f} ms {x_value:.1f} TFLOP/s kernels {x_kernels}")

    extra = {}
    bias_lines = {}
    hbm_lines = {}
    if not args.no_extra:
        for name in EXTRA:
            if name == w.name:
                continue
            x = fa_inputs.WORKLOADS[name]
            mean, med = time_fwd_only(x, reps=max(10, args.steps // 2), warmup=3,
                                      warm_s=min(args.warm_seconds, 1.0))
            tf = fa.flops_fwd(x.B, x.H, x.N, x.d, x.causal) / (mean * 1e-3) / 1e12
            extra[name] = {"ms": round(mean, 4), "ms_median": round(med, 4),
                           "TFLOP/s": round(tf, 1),
                           "frac_of_peak": round(tf / PEAK_TFLOPS[x.dtype], 4),
                           "peak": PEAK_TFLOPS[x.dtype]}
            log(f"{name}: {mean:.3f} ms {tf:.1f} TFLOP/s")
        name, shape = MX_EXTRA
        mean, med = time_fwd_mx(shape, reps=max(10, args.steps // 2), warmup=3,
                                warm_s=min(args.warm_seconds, 1.0))
        tf = fa.flops_fwd(*shape, False) / (mean * 1e-3) / 1e12
        extra[name] = {"ms": round(mean, 4), "ms_median": round(med, 4), "TFLOP/s": round(tf, 1),
                       "frac_of_peak": round(tf / PEAK_TFLOPS["fp8"], 4),
                       "peak": PEAK_TFLOPS["fp8"]}
        log(f"{name}: {mean:.3f} ms {tf:.1f} TFLOP/s")
        small = time_small_fp32()
        extra["fp32_fwdbwd_b1h1n128d64"] = small
        log(f"fp32_fwdbwd_b1h1n128d64: {small}")
        for name, shape, causal, kind, window, backward in BIAS_EXTRA:
            r = time_bias(shape, causal, kind, window, backward, reps=max(10, args.steps // 2),
                          warmup=3, warm_s=min(args.warm_seconds, 1.0))
            bias_lines[name] = r
            log(f"{name}: {r}")
        xd = w if w.backward else fa_inputs.WORKLOADS[FWDBWD_EXTRA]
        if xd.dtype == "bf16":  # (for fp32 the delta kernel is a stage of the step)
            work = algorithmic_work(xd)
            mean, med = time_delta(xd, reps=max(10, args.steps // 2), warmup=3,
                                   warm_s=min(args.warm_seconds, 1.0))
            gbs = work["delta_bytes"] / (mean * 1e-3) / 1e9
            hbm_lines["delta"] = {"ms": round(mean, 4), "ms_median": round(med, 4),
                                  "GB/s": round(gbs, 1), "peak": PEAK_HBM_GBS,
                                  "frac_hbm": round(gbs / PEAK_HBM_GBS, 4),
                                  "bytes": work["delta_bytes"],
                                  "shape": list(xd.shape),
                                  "note": "fa_bwd_delta on this shape (reads O and dO, "
                                          "writes delta; the bf16 fa_bwd forms delta in dQ): 30 "
                                          "back-to-back calls over 6 buffer pairs, per call"}
            log(f"delta kernel: {hbm_lines['delta']}")

    io_cmp = None
    schedules = None
    if not args.no_extra:
        io_cmp = time_io_compare(reps=max(5, args.steps // 4), warmup=2,
                                 warm_s=min(args.warm_seconds, 0.5))
        schedules = time_schedules(reps=max(5, args.steps // 4))
        log(f"forward schedules: {schedules}")

    measured = None
    if not args.no_extra or args.rate_probe:
        measured = measure_mfma_rates()
        log(f"measured matrix-core rates (TFLOP/s): {measured}")
        roof["measured_peak"] = measured[w.dtype] if w.dtype in measured else None
        if roof["unit"] == "TFLOP/s" and roof["measured_peak"]:
            roof["frac_of_measured_peak"] = round(roof["achieved"] / roof["measured_peak"], 4)
        for x in fwdbwd.values():
            r = x["roofline"]
            if r["unit"] == "TFLOP/s" and measured.get("bf16"):
                r["measured_peak"] = measured["bf16"]
                r["frac_of_measured_peak"] = round(r["achieved"] / measured["bf16"], 4)
        for name, x in extra.items():
            dt = "fp8" if name.startswith(("fp8", "mxfp8")) else "bf16"
            if "TFLOP/s" in x and dt in measured:
                x["frac_of_measured_peak"] = round(x["TFLOP/s"] / measured[dt], 4)

    cpu = None
    if not args.no_cpu:
        log("timing the CPU oracle on a sample")
        cpu = cpu_baseline(w, args.cpu_heads or w.B * w.H)
        log(f"cpu oracle: {cpu}")

    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "warm_seconds": args.warm_seconds,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": w.dtype, "data": "synthetic: N(0,1) float32 draws, seed 42, cast to the "
                                  "workload's format",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "N": w.N, "d": w.d,
                   "causal": w.causal, "passes": "fwd+bwd" if w.backward else "fwd",
                   "scale": w.scale, "parallelism": "single GPU",
                   "forward_schedule": os.environ.get("FA_FWD_SCHEDULE") or "interleaved"},
        "frac_of_peak": round(value / peak, 4),
        "kernels": kernels,
        "roofline": roof,
        "fwdbwd_workloads": fwdbwd,
        "forward_workloads": extra,
        "bias_workloads": bias_lines,
        "hbm_kernels": hbm_lines,
        "io_comparison": io_cmp,
        "forward_schedules": schedules,
        "mfma_rate_measured": None if measured is None else dict(
            measured, unit="TFLOP/s",
            note="pure 32x32 matrix-core products on pseudo-random operands, every CU, warm "
                 "clock (fa_measure_mfma_rate): what the chip sustains within its power budget"),
        "cpu_baseline": cpu,
        "wall_s_timed": round(wall, 4),
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
