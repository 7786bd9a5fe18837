#!/usr/bin/env python3
"""Benchmark of the adaLN hot path on one MI355X.

A step is one pass of the GLM-Image (1, 4096, 4096) bf16 pair:
    h   = ln_modulate(x, scale, shift, eps=1e-5)
    out = residual_gate_add(x, gate, h)
with inputs resident in HBM.  About 50 ms of back-to-back steps bring the
device's clocks to their steady state after the host-side setup, then W
untimed warm-up steps, then K timed steps between a synchronize on both
sides.  Buffers rotate over enough sets (>= 1 GiB in total) that the 256 MB
MALL cannot serve a step from cache.

The step time comes from HIP events on the launch stream around the K
timed steps.  Each kernel's average duration comes from its own loop of
back-to-back launches over the same rotated buffers (after two passes over
every set and about 50 ms of the same launches), between events on the
same stream; the roofline object reports the ln_modulate kernel (the
kernel the headline metric names).  The CPU oracle
(fixed-order fp32 mode) is timed on the host on the same step.

Prints ONE JSON line on stdout; everything else goes to stderr.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0  # MI355X HBM3E, published
METRIC = "µs/call + achieved HBM GB/s (% of peak), ln_modulate bf16 (1,4096,4096)"

# HBM bytes per ln_modulate launch from rocprofv3 byte counters, valid only
# while the kernel sources are the ones the counters were taken on
TRAFFIC_RECORD = os.path.join(ROOT, "profiles", "ln_modulate_1x4096x4096_traffic.txt")
TRAFFIC_SOURCES = ["modulate_ln_amd/csrc/ln_modulate.hip", "modulate_ln_amd/csrc/ln_row.hpp",
                   "modulate_ln_amd/csrc/mw_row.hpp", "modulate_ln_amd/csrc/device_common.hpp"]


def source_sha256(paths) -> str:
    import hashlib

    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic():
    """Bytes per launch: FETCH_SIZE and WRITE_SIZE (KiB per dispatch) of the kernel,
    each scaled by the same counter's reading for a plain copy of known size.
    None when there is no record or the kernel changed since it was taken."""
    if not os.path.exists(TRAFFIC_RECORD):
        return None
    rec = {}
    for line in open(TRAFFIC_RECORD):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            rec[k.strip()] = v.strip()
    try:
        if rec["source_sha256"] != source_sha256(TRAFFIC_SOURCES):
            return None
        copy_bytes = float(rec["copy_bytes_each_way"])
        rd = float(rec["fetch_kib_per_dispatch"]) / float(rec["copy_fetch_kib_per_dispatch"]) * copy_bytes
        wr = float(rec["write_kib_per_dispatch"]) / float(rec["copy_write_kib_per_dispatch"]) * copy_bytes
    except (KeyError, ValueError, ZeroDivisionError):
        return None
    return int(round(rd + wr))


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def lnm_bytes(R: int, D: int, B: int) -> int:
    # one read + one write of every activation element, plus the scale and shift rows
    return 2 * R * D * 2 + 2 * B * D * 2


def rga_bytes(R: int, D: int, B: int) -> int:
    # residual and update read, out written, plus the gate rows
    return 3 * R * D * 2 + B * D * 2


def fused_bytes(R: int, D: int, B: int) -> int:
    # residual and update read, new residual and normalized output written, plus gate/scale/shift rows
    return 4 * R * D * 2 + 3 * B * D * 2


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--buffers", type=int, default=12, help="rotated buffer sets (>= 1 GiB total)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="skip the other workloads' timings")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="wall-time budget of the CPU baseline")
    args = ap.parse_args()

    if args.gpus != 1:
        log("bench.py measures one GPU: the adaLN path is row-local and its kernels run on one device; "
            "--gpus %d is not supported (run with --gpus 1)." % args.gpus)
        return 2

    import numpy as np
    import torch

    import modulate_ln_amd as m
    from modulate_ln_amd import workloads as W

    if not torch.cuda.is_available():
        log("bench.py needs a GPU")
        return 2
    m._native.lib()  # fail loudly if the HIP library is missing
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)

    # ---- the headline workload ------------------------------------------------
    wl = W.glm_square()
    eps = wl.meta["eps"]
    t = wl.tensors
    B, S, D = t["x"].shape
    R = B * S
    scale, shift, gate = t["scale"].to(dev), t["shift"].to(dev), t["gate"].to(dev)
    x0 = t["x"].to(dev)
    NB = max(1, args.buffers)
    xs = [x0.clone() for _ in range(NB)]
    hs = [torch.empty_like(x0) for _ in range(NB)]
    outs = [torch.empty_like(x0) for _ in range(NB)]
    lnm_calls = [m.ln_modulate(xs[i], scale, shift, eps, out=hs[i], prepare=True) for i in range(NB)]
    rga_calls = [m.residual_gate_add(xs[i], gate, hs[i], out=outs[i], prepare=True) for i in range(NB)]
    footprint = NB * 3 * x0.numel() * 2
    log("workload %s, %d rotated buffer sets (%.2f GiB)" % (wl.name, NB, footprint / 2 ** 30))

    K, Wm = args.steps, args.warmup
    # device warm-up before the W warm-up steps: back-to-back steps until their time is steady
    # (at least STEP_WARMUP_MIN_MS, at most STEP_WARMUP_MAX_MS), so the timed steps do not run
    # while the clocks are still rising from the host-side setup above (measured: a kernel
    # takes ~10 % longer in its first tens of milliseconds of back-to-back work than from then
    # on, and on some boxes far longer; a ramp that slow changes too little from one chunk to
    # the next for the steadiness test alone, hence the floor)
    def step_call(i):
        lnm_calls[i % NB]()
        rga_calls[i % NB]()

    warm_ms = warm_until_steady(step_call, stream, min_ms=STEP_WARMUP_MIN_MS, max_ms=STEP_WARMUP_MAX_MS)
    for i in range(Wm):
        lnm_calls[i % NB]()
        rga_calls[i % NB]()
    torch.cuda.synchronize()

    # timed region: K steps, events on the launch stream at both ends only
    e_start, e_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e_start.record(stream)
    for i in range(K):
        lnm_calls[i % NB]()
        rga_calls[i % NB]()
    e_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_ms = e_start.elapsed_time(e_end) / K

    # per-kernel duration: each kernel alone over the same rotated buffers, 20
    # repetitions x 50 back-to-back launches bracketed by events on the launch
    # stream, the median repetition
    lnm_us = time_loop(lnm_calls, 1000, stream)
    rga_us = time_loop(rga_calls, 1000, stream)
    lb, rb = lnm_bytes(R, D, B), rga_bytes(R, D, B)
    step_gbps = (lb + rb) / (step_ms * 1e-3) / 1e9
    lnm_gbps = lb / (lnm_us * 1e-6) / 1e9
    rga_gbps = rb / (rga_us * 1e-6) / 1e9
    log("step %.2f us (wall %.2f us/step); alone: ln_modulate %.2f us (%.0f GB/s), residual_gate_add %.2f us (%.0f GB/s)"
        % (step_ms * 1e3, wall / K * 1e6, lnm_us, lnm_gbps, rga_us, rga_gbps))

    result = {
        "metric": METRIC,
        "value": round(step_gbps, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": Wm,
        "ms_per_step": round(step_ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) x with 1% x20 outliers, N(0,0.1) adaLN rows; see workloads.glm_square)",
        "config": {"workload": "ln_modulate + residual_gate_add, x (1,4096,4096) bf16, eps 1e-5",
                   "B": B, "S": S, "D": D, "rotated_buffer_sets": NB, "device_warmup_ms": round(warm_ms, 1),
                   "step_bytes": lb + rb},
        "us_per_call": {"ln_modulate": round(lnm_us, 3), "residual_gate_add": round(rga_us, 3)},
        "achieved_GBps": {"ln_modulate": round(lnm_gbps, 1), "residual_gate_add": round(rga_gbps, 1)},
        "roofline": {"bound": "hbm", "kernel": "ln_modulate", "achieved": round(lnm_gbps, 1),
                     "peak": PEAK_HBM_GBPS, "unit": "GB/s", "frac": round(lnm_gbps / PEAK_HBM_GBPS, 4),
                     "algorithmic_bytes": lb, "traffic": measured_traffic()},
    }

    # same buffers every call (67 MB fits the 256 MB MALL): reported apart, not the headline
    hot_us = time_loop(lnm_calls[:1], 1000, stream)
    result["ln_modulate_hot_same_buffer"] = {"us": round(hot_us, 3), "GBps": round(lb / hot_us / 1e3, 1),
                                             "note": "one buffer set reused, possibly MALL-assisted"}
    # host cost of a call: a marshalled call (ctypes only) and the full binding
    n_host = 200
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(n_host):
        lnm_calls[i % NB]()
    host_prepared = (time.perf_counter() - t0) / n_host * 1e6
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(n_host):
        m.ln_modulate(xs[i % NB], scale, shift, eps, out=hs[i % NB])
    host_binding = (time.perf_counter() - t0) / n_host * 1e6
    torch.cuda.synchronize()
    result["host_us_per_call"] = {"ln_modulate_prepared": round(host_prepared, 2),
                                  "ln_modulate_binding": round(host_binding, 2)}
    log("hot same-buffer ln_modulate %.2f us; host per call: prepared %.2f us, binding %.2f us"
        % (hot_us, host_prepared, host_binding))

    # ---- a plain copy of the same size: the achievable streaming bandwidth ----
    cp_src = [torch.empty(2 * x0.numel(), dtype=torch.bfloat16, device=dev) for _ in range(4)]
    cp_dst = [torch.empty_like(cp_src[0]) for _ in range(4)]
    for i in range(8):
        cp_dst[i % 4].copy_(cp_src[i % 4])
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    n_cp = 100
    for i in range(n_cp):
        cp_dst[i % 4].copy_(cp_src[i % 4])
    e1.record(stream)
    torch.cuda.synchronize()
    cp_us = 1000.0 * e0.elapsed_time(e1) / n_cp
    cp_gbps = 2 * cp_src[0].numel() * 2 / (cp_us * 1e-6) / 1e9
    result["copy_reference"] = {"bytes": 2 * cp_src[0].numel() * 2, "us": round(cp_us, 3),
                                "GBps": round(cp_gbps, 1),
                                "ln_modulate_frac_of_copy": round(lnm_gbps / cp_gbps, 4)}
    del cp_src, cp_dst
    log("copy %.1f GB/s; ln_modulate at %.1f%% of copy, %.1f%% of peak"
        % (cp_gbps, 100 * lnm_gbps / cp_gbps, 100 * lnm_gbps / PEAK_HBM_GBPS))
    result["stream_reference"] = stream_reference(dev, stream, log)

    if not args.no_extra:
        result["other_workloads"] = other_workloads(m, W, dev, stream, log)

    # ---- CPU baseline: the oracle on the same step ----------------------------
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(W, wl, lb + rb, args.cpu_seconds, log)

    del xs, hs, outs
    print(json.dumps(result), flush=True)
    return 0


def stream_reference(dev, stream, log, nbytes=1 << 30):
    """Streaming rates of torch's own kernels on 1 GiB buffers (far past the MALL): write-only
    (fill), a copy (read + write), and torch's float32 sum -- a reduction kernel, reported for
    context only: it is not a read-only ceiling (plain read-only streams measured 6.6-7.1 TB/s
    on this part).  Context for `roofline`: HBM writes run well below the 8 TB/s peak, so a
    stream that writes as much as it reads tops out near the copy rate."""
    import torch

    a = torch.empty(nbytes // 2, dtype=torch.bfloat16, device=dev)
    b = torch.empty_like(a)
    a.fill_(1.0)
    b.copy_(a)

    def ms_per(fn, reps=10):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    out = {"bytes": nbytes}
    for name, fn, moved in (("write_only_fill", lambda: a.fill_(2.0), nbytes),
                            ("torch_sum_fp32_reduction", lambda: a.sum(dtype=torch.float32), nbytes),
                            ("copy", lambda: b.copy_(a), 2 * nbytes)):
        ms = ms_per(fn)
        out[name] = {"ms": round(ms, 4), "GBps": round(moved / (ms * 1e-3) / 1e9, 1)}
    del a, b
    log("torch streams (1 GiB): write-only fill %.0f GB/s, fp32 sum (a reduction) %.0f GB/s, copy %.0f GB/s"
        % (out["write_only_fill"]["GBps"], out["torch_sum_fp32_reduction"]["GBps"], out["copy"]["GBps"]))
    return out


DEVICE_WARMUP_MS = 50.0       # at least this much back-to-back work before a measurement
DEVICE_WARMUP_MAX_MS = 1000.0  # ... and at most this much while the call time still moves
STEP_WARMUP_MIN_MS = 1000.0    # before the headline step loop: a floor a slow ramp cannot pass
STEP_WARMUP_MAX_MS = 3000.0    # ... and the bound there
WARMUP_CHUNK_MS = 20.0
WARMUP_TOL = 0.01


def warm_until_steady(call, stream, min_ms=DEVICE_WARMUP_MS, max_ms=DEVICE_WARMUP_MAX_MS):
    """Issue back-to-back calls (call(i) launches the i-th) in chunks of about WARMUP_CHUNK_MS
    until, after at least min_ms, two consecutive chunks take the same time per call within
    WARMUP_TOL, or max_ms have passed; returns the milliseconds spent.  Some boxes leave the
    clocks low for far longer than the tens of milliseconds most need (one measured the
    headline at 13.7 µs for the first seconds of the run, 11.4 µs once a long workload had
    run), so a fixed warm-up is either too short there or wasted elsewhere."""
    import torch

    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    k = 0

    def run_chunk(n):  # n back-to-back calls; their milliseconds on the device
        nonlocal k
        e0.record(stream)
        for _ in range(n):
            call(k)
            k += 1
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1)

    return steady_chunks(run_chunk, min_ms, max_ms)


def steady_chunks(run_chunk, min_ms, max_ms, chunk_ms=WARMUP_CHUNK_MS, tol=WARMUP_TOL):
    """The loop of warm_until_steady, apart from the device: run_chunk(n) runs n calls and
    returns their milliseconds.  10 calls size the chunks to about chunk_ms; then chunks until,
    after at least min_ms in all, two in a row agree per call within tol, or max_ms have
    passed.  Returns the milliseconds spent."""
    spent = run_chunk(10)
    n = int(max(1, min(20000, chunk_ms / max(spent / 10, 1e-4))))
    prev = None
    while True:
        ms = run_chunk(n)
        spent += ms
        per = ms / n
        if spent >= max_ms or (spent >= min_ms and prev is not None and abs(per - prev) <= tol * prev):
            return spent
        prev = per


def time_loop(calls, n, stream, reps=20):
    """µs per launch of back-to-back calls (rotating through calls): `reps` repetitions of
    n // reps launches each, events on the launch stream around every repetition, the
    median repetition reported.  Warm-up: two passes over every buffer set (at least 10
    calls), so no set is touched for the first time inside the timed region, then
    back-to-back calls until their time per call is steady (warm_until_steady), so the
    device's clocks have left the state the host-side setup between measurements leaves
    them in."""
    import statistics

    import torch

    for i in range(max(10, 2 * len(calls))):
        calls[i % len(calls)]()
    warm_until_steady(lambda i: calls[i % len(calls)](), stream)
    reps = max(1, min(reps, n))
    per = max(1, n // reps)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    torch.cuda.synchronize()
    k = 0
    ev[0].record(stream)
    for r in range(reps):
        for _ in range(per):
            calls[k % len(calls)]()
            k += 1
        ev[r + 1].record(stream)
    torch.cuda.synchronize()
    return statistics.median(1000.0 * ev[r].elapsed_time(ev[r + 1]) / per for r in range(reps))


def other_workloads(m, W, dev, stream, log):
    """The other workload shapes, each timed over back-to-back calls (buffers rotated
    so every set of calls touches >= 1 GiB)."""
    import torch

    res = {}

    def rot(nbytes):
        return max(2, min(64, -(-(1 << 30) // max(nbytes, 1))))

    # (1,256,512) ln_modulate: launch-bound, report us only
    wl = W.ln_small()
    t = {k: v.to(dev) for k, v in wl.tensors.items()}
    calls = [m.ln_modulate(t["x"], t["scale"], t["shift"], 1e-6, prepare=True)]
    us = time_loop(calls, 2000, stream)
    res["ln_modulate_1x256x512"] = {"us": round(us, 3), "GBps": round(lnm_bytes(256, 512, 1) / us / 1e3, 1)}

    # Sana (2,1024,2240) transposed input
    wl = W.sana_transposed()
    xt = wl.tensors["xt"].to(dev)
    emb = wl.tensors["emb"].to(dev)
    nb = rot(2 * xt.numel() * 2)
    xts = [xt.clone() for _ in range(nb)]
    outs = [torch.empty(2, 1024, 2240, dtype=torch.bfloat16, device=dev) for _ in range(nb)]
    calls = [m.ln_modulate(xts[i].transpose(1, 2), emb[:, 5], emb[:, 0], 1e-6, out=outs[i], prepare=True)
             for i in range(nb)]
    us = time_loop(calls, 500, stream)
    b = lnm_bytes(2048, 2240, 2)
    res["ln_modulate_2x1024x2240_transposed"] = {"us": round(us, 3), "GBps": round(b / us / 1e3, 1),
                                                  "pages_H200_us": 14.3}
    # the same calls with a workspace (ln_modulate_ws: whole-line reads, 8 blocks per 64 tokens)
    ws = m.ln_modulate_workspace(xts[0].transpose(1, 2))
    calls = [m.ln_modulate(xts[i].transpose(1, 2), emb[:, 5], emb[:, 0], 1e-6, out=outs[i], workspace=ws,
                           prepare=True) for i in range(nb)]
    us = time_loop(calls, 500, stream)
    res["ln_modulate_2x1024x2240_transposed_ws"] = {"us": round(us, 3), "GBps": round(b / us / 1e3, 1),
                                                     "pages_H200_us": 14.3}
    # and with the library's own array (ln_modulate_noalloc)
    calls = [m.ln_modulate_noalloc(xts[i].transpose(1, 2), emb[:, 5], emb[:, 0], 1e-6, out=outs[i], prepare=True)
             for i in range(nb)]
    us = time_loop(calls, 500, stream)
    res["ln_modulate_2x1024x2240_transposed_noalloc"] = {"us": round(us, 3), "GBps": round(b / us / 1e3, 1)}
    xcs = [xt.transpose(1, 2).contiguous() for _ in range(nb)]
    calls = [m.ln_modulate(xcs[i], emb[:, 5], emb[:, 0], 1e-6, out=outs[i], prepare=True) for i in range(nb)]
    us = time_loop(calls, 500, stream)
    res["ln_modulate_2x1024x2240_contiguous"] = {"us": round(us, 3), "GBps": round(b / us / 1e3, 1)}
    del xts, xcs, outs

    # (1,4096,4096) stored transposed, with and without a workspace
    g = torch.Generator().manual_seed(4096)
    xt = W.normal((1, 4096, 4096), g).to(dev)
    sc = W.normal((1, 4096), g, std=0.1).to(dev)
    sh = W.normal((1, 4096), g, std=0.1).to(dev)
    nb = rot(2 * xt.numel() * 2)
    xts = [xt.clone() for _ in range(nb)]
    outs = [torch.empty(1, 4096, 4096, dtype=torch.bfloat16, device=dev) for _ in range(nb)]
    ws = m.ln_modulate_workspace(xt.transpose(1, 2))
    b = lnm_bytes(4096, 4096, 1)
    for tag, w in (("", None), ("_ws", ws)):
        calls = [m.ln_modulate(xts[i].transpose(1, 2), sc, sh, 1e-6, out=outs[i], workspace=w, prepare=True)
                 for i in range(nb)]
        us = time_loop(calls, 300, stream)
        res["ln_modulate_1x4096x4096_transposed" + tag] = {"us": round(us, 3), "GBps": round(b / us / 1e3, 1)}
    del xts, outs, calls

    # GLM-Image q/k heads (1,4360,32,128)
    wl = W.glm_qk()
    t = {k: v.to(dev) for k, v in wl.tensors.items()}
    nb = rot(4 * t["q"].numel() * 2)
    qs = [t["q"].clone() for _ in range(nb)]
    ks = [t["k"].clone() for _ in range(nb)]
    calls = [m.qk_head_layernorm(qs[i], ks[i], t["wq"], t["bq"], t["wk"], t["bk"], 1e-6, prepare=True)
             for i in range(nb)]
    us = time_loop(calls, 200, stream)
    b = 4 * t["q"].numel() * 2 + 4 * 128 * 2
    res["qk_head_layernorm_1x4360x32x128"] = {"us": round(us, 3), "GBps": round(b / us / 1e3, 1),
                                               "pages_H200_eager_us": 301.0}
    del qs, ks, calls

    # bias + tanh-GELU (16384, 12288)
    wl = W.wan_bias_gelu()
    x = wl.tensors["x"].to(dev)
    bias = wl.tensors["bias"].to(dev)
    xs2 = [x, x.clone()]
    outs = [torch.empty_like(x) for _ in range(2)]
    calls = [m.bias_gelu_tanh(xs2[i], bias, out=outs[i], prepare=True) for i in range(2)]
    us = time_loop(calls, 50, stream)
    b = 2 * x.numel() * 2 + x.shape[1] * 2
    res["bias_gelu_tanh_16384x12288"] = {"us": round(us, 3), "GBps": round(b / us / 1e3, 1)}
    del xs2, outs, x

    # RMSNorm variants on the same shapes: (1,4096,4096) rows, (1,4360,32,128) q/k heads
    wl = W.glm_square()
    t = {k: v.to(dev) for k, v in wl.tensors.items()}
    nb = rot(lnm_bytes(4096, 4096, 1))
    xs_ = [t["x"].clone() for _ in range(nb)]
    outs = [torch.empty_like(t["x"]) for _ in range(nb)]
    calls = [m.rmsnorm_scale_shift(xs_[i], t["scale"], t["shift"], 1e-5, out=outs[i], prepare=True)
             for i in range(nb)]
    us = time_loop(calls, 500, stream)
    res["rmsnorm_scale_shift_1x4096x4096"] = {"us": round(us, 3),
                                              "GBps": round(lnm_bytes(4096, 4096, 1) / us / 1e3, 1)}
    del xs_, outs, calls
    wl = W.glm_qk()
    t = {k: v.to(dev) for k, v in wl.tensors.items()}
    nb = rot(4 * t["q"].numel() * 2)
    qs = [t["q"].clone() for _ in range(nb)]
    ks = [t["k"].clone() for _ in range(nb)]
    calls = [m.qk_rmsnorm(qs[i], ks[i], t["wq"], t["wk"], 1e-6, prepare=True) for i in range(nb)]
    us = time_loop(calls, 200, stream)
    b = 4 * t["q"].numel() * 2 + 2 * 128 * 2
    res["qk_rmsnorm_1x4360x32x128"] = {"us": round(us, 3), "GBps": round(b / us / 1e3, 1)}
    del qs, ks, calls

    # ln_modulate into static FP8, and the single-rounding fold, (1,4096,4096)
    wl = W.glm_square()
    t = {k: v.to(dev) for k, v in wl.tensors.items()}
    nb = rot(3 * 4096 * 4096)
    xs_ = [t["x"].clone() for _ in range(nb)]
    q8 = [torch.empty((1, 4096, 4096), dtype=torch.float8_e4m3fn, device=dev) for _ in range(nb)]
    qscale = torch.tensor([0.05], dtype=torch.float32, device=dev)
    calls = [m.ln_modulate_fp8(xs_[i], t["scale"], t["shift"], qscale, 1e-5, out=q8[i], prepare=True)
             for i in range(nb)]
    us = time_loop(calls, 500, stream)
    b = 3 * 4096 * 4096 + 2 * 4096 * 2
    res["ln_modulate_fp8_1x4096x4096"] = {"us": round(us, 3), "GBps": round(b / us / 1e3, 1)}
    del q8, calls
    outs = [torch.empty_like(t["x"]) for _ in range(nb)]
    calls = [m.ln_modulate_fold(xs_[i], t["scale"], t["shift"], 1e-5, out=outs[i], prepare=True) for i in range(nb)]
    us = time_loop(calls, 500, stream)
    res["ln_modulate_fold_1x4096x4096"] = {"us": round(us, 3),
                                           "GBps": round(lnm_bytes(4096, 4096, 1) / us / 1e3, 1)}
    del xs_, outs, calls

    # modulate_scale_shift (1,4096,4096): one adaLN row per sample, then one per token
    wl = W.glm_square()
    t = {k: v.to(dev) for k, v in wl.tensors.items()}
    nb = rot(lnm_bytes(4096, 4096, 1))
    xs_ = [t["x"].clone() for _ in range(nb)]
    outs = [torch.empty_like(t["x"]) for _ in range(nb)]
    calls = [m.modulate_scale_shift(xs_[i], t["scale"], t["shift"], out=outs[i], prepare=True) for i in range(nb)]
    us = time_loop(calls, 500, stream)
    res["modulate_scale_shift_1x4096x4096"] = {"us": round(us, 3),
                                               "GBps": round(lnm_bytes(4096, 4096, 1) / us / 1e3, 1)}
    g = torch.Generator().manual_seed(1)
    sc_tok = W.normal((1, 4096, 4096), g, std=0.1).to(dev)
    sh_tok = W.normal((1, 4096, 4096), g, std=0.1).to(dev)
    nb2 = rot(4 * 4096 * 4096 * 2)
    calls = [m.modulate_scale_shift(xs_[i % nb], sc_tok, sh_tok, out=outs[i % nb], prepare=True) for i in range(nb2)]
    us = time_loop(calls, 300, stream)
    b = 4 * 4096 * 4096 * 2
    res["modulate_scale_shift_1x4096x4096_per_token_rows"] = {"us": round(us, 3), "GBps": round(b / us / 1e3, 1)}
    del xs_, outs, calls, sc_tok, sh_tok

    # temb_table_slices at the Wan 704x1280, 121-frame size: (1,109120,6,3072) -> 8 GB of fp32
    wl = W.wan_temb()
    table = wl.tensors["table"].to(dev)
    temb = W.tile(wl.tensors["temb_frame"].to(dev), wl.meta["frames"])
    Bt, Lt, Mt, Dt = temb.shape
    out_t = torch.empty((Mt, Bt, Lt, Dt), dtype=torch.float32, device=dev)
    call = m.temb_table_slices(table, temb, out=out_t, prepare=True)
    us = time_loop([call], 10, stream, reps=5)
    b = Bt * Lt * Mt * Dt * (2 + 4) + Mt * Dt * 4
    entry = {"ms": round(us / 1e3, 4), "GBps": round(b / us / 1e3, 1)}
    del out_t

    def eager():
        return [c.contiguous() for c in (table[None, None] + temb.float()).chunk(Mt, dim=2)]

    eager()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(3):
        eager()
    e1.record(stream)
    torch.cuda.synchronize()
    entry["torch_eager_chunks_contiguous_ms"] = round(e0.elapsed_time(e1) / 3, 4)
    res["temb_table_slices_1x109120x6x3072"] = entry
    del temb, table

    # the gated residual update fused with ln_modulate, (1,4096,4096)
    wl = W.glm_square()
    t = {k: v.to(dev) for k, v in wl.tensors.items()}
    R, D = 4096, 4096
    nb = rot(fused_bytes(R, D, 1))
    rs = [t["x"].clone() for _ in range(nb)]
    us_ = [t["update"].clone() for _ in range(nb)]
    ros = [torch.empty_like(t["x"]) for _ in range(nb)]
    hs = [torch.empty_like(t["x"]) for _ in range(nb)]
    calls = [m.residual_gate_add_ln_modulate(rs[i], t["gate"], us_[i], t["scale"], t["shift"], 1e-5,
                                             residual_out=ros[i], out=hs[i], prepare=True) for i in range(nb)]
    us = time_loop(calls, 300, stream)
    res["residual_gate_add_ln_modulate_1x4096x4096"] = {"us": round(us, 3),
                                                        "GBps": round(fused_bytes(R, D, 1) / us / 1e3, 1)}
    del rs, us_, ros, hs, calls

    # rows longer than 4096 elements (W = 2..16 waves per row) at the same 2^24 elements: D % 8 == 4
    # (4100, W = 2, V = 4), 16384 (W = 4), 65536 (W = 16); the fused residual update at D = 16384
    g = torch.Generator().manual_seed(2)
    for D in (4100, 16384, 65536):
        S = (1 << 24) // D
        x = W.normal((1, S, D), g).to(dev)
        sc = W.normal((1, D), g, std=0.1).to(dev)
        sh = W.normal((1, D), g, std=0.1).to(dev)
        nb = rot(lnm_bytes(S, D, 1))
        xs_ = [x.clone() for _ in range(nb)]
        outs = [torch.empty_like(x) for _ in range(nb)]
        calls = [m.ln_modulate(xs_[i], sc, sh, 1e-6, out=outs[i], prepare=True) for i in range(nb)]
        us = time_loop(calls, 500, stream)
        res["ln_modulate_1x%dx%d" % (S, D)] = {"us": round(us, 3), "GBps": round(lnm_bytes(S, D, 1) / us / 1e3, 1),
                                               "waves_per_row": m.order_for(1, D).W}
        if D == 16384:
            gate = W.normal((1, D), g, std=0.5).to(dev)
            ups = [W.normal((1, S, D), g).to(dev)] * nb
            ros = [torch.empty_like(x) for _ in range(nb)]
            calls = [m.residual_gate_add_ln_modulate(xs_[i], gate, ups[i], sc, sh, 1e-6, residual_out=ros[i],
                                                     out=outs[i], prepare=True) for i in range(nb)]
            us = time_loop(calls, 300, stream)
            res["residual_gate_add_ln_modulate_1x%dx%d" % (S, D)] = {
                "us": round(us, 3), "GBps": round(fused_bytes(S, D, 1) / us / 1e3, 1)}
            del ups, ros
        del xs_, outs, calls, x

    # 20-block DiT chain on (4,4096,3072)
    wl = W.dit_chain()
    x = wl.tensors["x"].to(dev)
    embs = [e.to(dev) for e in wl.tensors["embs"]]
    h = torch.empty_like(x)
    R, D = 4 * 4096, 3072

    def chain_ms(calls, reps=5):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        for c in calls:
            c()
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(reps):
            for c in calls:
                c()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    # two ln_modulate and two residual_gate_add per block: 80 launches per pass
    calls = []
    for emb in embs:
        for j in (0, 3):
            calls.append(m.ln_modulate(x, emb[:, j + 1], emb[:, j], 1e-6, out=h, prepare=True))
            calls.append(m.residual_gate_add(x, emb[:, j + 2], h, out=x, prepare=True))
    ms = chain_ms(calls)
    b = 40 * (lnm_bytes(R, D, 4) + rga_bytes(R, D, 4))
    res["dit_chain_20_blocks_4x4096x3072"] = {"ms": round(ms, 4), "GBps": round(b / ms / 1e6, 1),
                                              "launches": len(calls)}
    # each gated residual add fused with the ln_modulate that reads its result: 41 launches
    calls = [m.ln_modulate(x, embs[0][:, 1], embs[0][:, 0], 1e-6, out=h, prepare=True)]
    for i, emb in enumerate(embs):
        calls.append(m.residual_gate_add_ln_modulate(x, emb[:, 2], h, emb[:, 4], emb[:, 3], 1e-6, residual_out=x,
                                                     out=h, prepare=True))
        if i + 1 < len(embs):
            nxt = embs[i + 1]
            calls.append(m.residual_gate_add_ln_modulate(x, emb[:, 5], h, nxt[:, 1], nxt[:, 0], 1e-6,
                                                         residual_out=x, out=h, prepare=True))
        else:
            calls.append(m.residual_gate_add(x, emb[:, 5], h, out=x, prepare=True))
    ms_f = chain_ms(calls)
    b = lnm_bytes(R, D, 4) + 39 * fused_bytes(R, D, 4) + rga_bytes(R, D, 4)
    # the same 41 launches captured once in a HIP graph and replayed
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        cap = torch.cuda.current_stream(dev).cuda_stream
        for c in calls:
            rc = c.fn(*(c.args[:-1] + (cap,)))
            if rc != m._native.OK:
                raise m.AdalnError(c.name + " (captured)", rc)
    graph.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(5):
        graph.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    ms_g = e0.elapsed_time(e1) / 5
    res["dit_chain_20_blocks_4x4096x3072_fused_residual"] = {
        "ms": round(ms_f, 4), "GBps": round(b / ms_f / 1e6, 1), "launches": len(calls),
        "speedup_vs_unfused": round(ms / ms_f, 3), "hip_graph_replay_ms": round(ms_g, 4)}
    del graph
    for k, v in res.items():
        log("%-40s %s" % (k, v))
    return res


def cpu_baseline(W, wl, step_bytes, budget_s, log):
    """The oracle on the same step: fixed-order fp32 mode on every host thread over the full
    step, repeated for ~budget_s of wall time (the reported value), plus both modes on one
    thread and on every thread over a bounded slice of rows (the detail)."""
    from oracle import oracle as orc

    t = wl.tensors
    B, S, D = t["x"].shape
    x = W.bits(t["x"].reshape(B * S, D))
    sc, sh, g = W.bits(t["scale"]), W.bits(t["shift"]), W.bits(t["gate"])
    eps = wl.meta["eps"]
    orc._load()
    all_threads = len(os.sched_getaffinity(0))
    orc.set_threads(all_threads)
    threads = orc.get_threads()

    def step(xr, mode):
        h, _, _ = orc.ln_modulate(xr, sc, sh, xr.shape[0], eps, mode, V=8, L=64)
        orc.residual_gate_add(xr, g, h, xr.shape[0], mode)

    reps = 0
    t0 = time.perf_counter()
    while True:
        step(x, orc.FP32)
        reps += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    gbps = step_bytes * reps / dt / 1e9
    log("cpu oracle: %d step(s) in %.2f s on %d threads -> %.2f GB/s" % (reps, dt, threads, gbps))

    detail = {}
    rows = 512  # a slice of the step's rows: bytes scale with the row count
    xs = x[:rows].copy()
    slice_bytes = step_bytes * rows // (B * S)
    for mode, mname in ((orc.FP32, "fp32_fixed"), (orc.FP64, "fp64_two_pass")):
        for nt in (1, threads):
            orc.set_threads(nt)
            n = 0
            t1 = time.perf_counter()
            while n < 2 or time.perf_counter() - t1 < 0.5:
                step(xs, mode)
                n += 1
            d = time.perf_counter() - t1
            detail["%s_%dt" % (mname, nt)] = {"GBps": round(slice_bytes * n / d / 1e9, 3), "threads": nt}
    orc.set_threads(threads)
    log("cpu oracle detail (%d-row slices): %s" % (rows, detail))
    return {"value": round(gbps, 3), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": "full (1,4096,4096) ln_modulate + residual_gate_add step x%d (fp32 fixed-order mode)" % reps,
            "ms_per_step": round(1000 * dt / reps, 2), "detail": detail}


if __name__ == "__main__":
    sys.exit(main())
