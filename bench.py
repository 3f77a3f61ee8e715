"""Benchmark: MXFP6 GEMM TFLOPS on the DiT MLP (one MI355X).

A step is one forward pass of the MLP hot path over 20480 tokens:
  mx_quantize(x)                     bf16 [20480, 3072] -> E2M3 codes + scales
  h = mx_gemm(x_mx, W1, GELU -> MX)  fc1 20480 x 3072 x 12288, E2M3 intermediate
  y = mx_gemm(h, W2, bf16 out)       fc2 20480 x 12288 x 3072
with weights pre-quantized once (untimed) and inputs resident in HBM; the
steps rotate over three independent sets of inputs, intermediates, outputs and
weight copies, so no step finds its operands in the 256 MB last-level cache
from the previous one.  value = 2*M*N*K summed over both GEMMs / step time
(wall clock over the timed steps).  Each kernel is also timed per launch with
HIP events on its stream (median, min, mean).  The GEMMs' launch
configurations come from the tuning table shipped with the package.

Measured beside it, each on rotating buffer sets, median and min per call:
the projection-shaped GEMM (4096 x 3072 x 3072, activations quantized in the
call, bf16 out) as a call and as the GEMM kernel alone; the skinny split-K path
(M in {16, 8} x 16384 x 13312, E3M2 weights, S in {16, 8}) per call and for the
split-K kernel alone; the tiny 256^3 GEMM; the step with the quantize-once
producer (RMSNorm + modulation + MX) in place of mx_quantize; the SwiGLU
variant of the MLP; the producer alone and feeding the stacked QKV + gate
projection; fc1's shape in each operand format; the matrix instruction's rate
with nothing else in the loop (the practical ceiling on this board); and the
CPU oracle, on a bounded sample of the MLP step (cpu_baseline) and of each
workload (oracle_ms beside the GPU time).

Prints one JSON line.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import microscaled_precision_gemm_amd as mx  # noqa: E402
from microscaled_precision_gemm_amd import synthetic as syn  # noqa: E402
from microscaled_precision_gemm_amd import tuning  # noqa: E402

METRIC = "MXFP6 GEMM TFLOPS + % of 10.1 PF MFMA peak (DiT MLP 20480x3072x12288)"
PEAK_MXFP6_TFLOPS = 10100.0
PEAK_HBM_GBS = 8000.0

# rocprofv3 names of the two GEMM instantiations <W fmt, A fmt, out kind, epilogue, out fmt>
# (E2M3 x E2M3; fc1: MX out + GELU, fc2: bf16 out, no epilogue)
# demangled GEMM kernel names: gemm_kernel<weights, activations, output kind, epilogue,
# output format, tile width, waves>; fc1 = E2M3 x E2M3 -> GELU-tanh -> MX E2M3, fc2 = -> bf16
KERNEL_PREFIX = {"fc1": "gemm_kernel<2, 2, 2, 1, 2", "fc2": "gemm_kernel<2, 2, 1, 0, 2"}


def kernel_name(gemm: str, config) -> str:
    tile_n, waves = (256, 4) if config is None else (int(config.tile_n), int(config.waves))
    return f"{KERNEL_PREFIX[gemm]}, {tile_n}, {waves}>"
# the sources the GEMM kernel is built from: measured HBM traffic is only reported
# while they are unchanged since the counters were taken
GEMM_SOURCES = ["gemm_kernel.h", "internal.h", "mx_device.h", "gemm_we2m3_e2m3.hip"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemm_fc1_fc2_hbm_traffic.txt")


def _events(n):
    return [torch.cuda.Event(enable_timing=True) for _ in range(n)]


SETS = 3  # independent buffer sets the timed loops rotate over


def stats(ms) -> dict:
    """Median, min and mean of per-launch times (ms)."""
    a = np.asarray(ms, dtype=np.float64)
    return {"median": round(float(np.median(a)), 4), "min": round(float(a.min()), 4), "mean": round(float(a.mean()), 4)}


def time_batches(fn, iters: int, batches: int = 5) -> dict:
    """Back-to-back rate: `batches` runs of `iters` calls fn(i) between one
    pair of HIP events each; ms per call of each batch (median, min, mean).
    For calls of a few microseconds this is the cost of the call in a stream
    of work; bracketing each call with its own events adds the events' own
    gaps (about 2 us measured) to every call."""
    settle(lambda: fn(0), 0.1)
    out = []
    for b in range(batches):
        e0, e1 = _events(2)
        e0.record()
        for i in range(iters):
            fn(b * iters + i)
        e1.record()
        torch.cuda.synchronize()
        out.append(e0.elapsed_time(e1) / iters)
    return stats(out)


def time_calls(fn, iters: int, settle_s: float = 0.2) -> list:
    """Per-call times (ms) of fn(i) for i = 0 .. iters-1, each between HIP
    events on the current stream, after an untimed settle."""
    settle(lambda: fn(0), settle_s)
    evs = [_events(2) for _ in range(iters)]
    torch.cuda.synchronize()
    for i in range(iters):
        evs[i][0].record()
        fn(i)
        evs[i][1].record()
    torch.cuda.synchronize()
    return [e[0].elapsed_time(e[1]) for e in evs]


SETTLE_S = 0.5


def settle(fn, seconds: float = SETTLE_S):
    """Run `fn` untimed for about `seconds` before the warm-up steps: from idle
    the GPU takes tens of milliseconds of sustained load to reach its steady
    clocks, so the first GEMMs after setup run up to ~20 % slower."""
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(10):
            fn()
        torch.cuda.synchronize()


def bench_mlp(table, steps: int, warmup: int, tune: bool = True):
    fc1, fc2 = syn.WORKLOADS["fc1"], syn.WORKLOADS["fc2"]
    m, d, hdim = fc1.m, fc1.k, fc1.n
    dev = torch.device("cuda:0")
    x_host, w1_host, w2_host = syn.make_a(fc1), syn.make_w(fc1), syn.make_w(fc2)
    # SETS independent sets: inputs, quantized inputs, intermediates, outputs and weight copies
    xs = [x_host.to(dev) for _ in range(SETS)]
    w1s = [mx.mx_quantize(w1_host.to(dev), "e2m3") for _ in range(SETS)]
    w2s = [mx.mx_quantize(w2_host.to(dev), "e2m3") for _ in range(SETS)]
    xqs = [mx.MXTensor.empty(m, d, "e2m3", "tiled", dev) for _ in range(SETS)]
    hs = [mx.MXTensor.empty(m, hdim, "e2m3", "tiled", dev) for _ in range(SETS)]
    ys = [torch.empty((m, d), dtype=torch.bfloat16, device=dev) for _ in range(SETS)]
    # the producer variant's parameters: gain, two conditionings of 10240 tokens
    gam = torch.ones(d, dtype=torch.float32, device=dev)
    shift = torch.zeros((2, d), dtype=torch.float32, device=dev)
    scale = torch.zeros((2, d), dtype=torch.float32, device=dev)
    # per-shape launch configurations from the tuning table: tuned here, untimed,
    # on these operands, unless the table (read from a file) already holds them
    cfg1 = table.lookup(m, hdim, d, epilogue="gelu_tanh", out_kind="mx")
    cfg2 = table.lookup(m, d, hdim, epilogue="none", out_kind="bf16")
    tuned = {}
    if tune and (cfg1 is None or cfg2 is None):
        mx.mx_quantize(xs[0], "e2m3", "tiled", out=xqs[0])
        tuned["fc1"] = tuning.tune_gemm(table, xqs[0], w1s[0], out_kind="mx", epilogue="gelu_tanh")
        h_t = mx.mx_gemm(xqs[0], w1s[0], out_kind="mx", epilogue="gelu_tanh")
        tuned["fc2"] = tuning.tune_gemm(table, h_t, w2s[0], out_kind="bf16")
        del h_t
        cfg1 = table.lookup(m, hdim, d, epilogue="gelu_tanh", out_kind="mx")
        cfg2 = table.lookup(m, d, hdim, epilogue="none", out_kind="bf16")
    elif tune:
        key1 = tuning.gemm_key(m, hdim, d, "e2m3", "e2m3", "gelu_tanh", "mx", "e2m3", tuning.device_name())
        key2 = tuning.gemm_key(m, d, hdim, "e2m3", "e2m3", "none", "bf16", "e2m3", tuning.device_name())
        tuned = {"fc1": table.entries[key1], "fc2": table.entries[key2]}
    else:
        cfg1 = cfg2 = None  # the library's shape rule
    if cfg1 is None:
        cfg1 = mx.mx_gemm_select_config(m, hdim, d, epilogue="gelu_tanh", out_kind="mx")
    if cfg2 is None:
        cfg2 = mx.mx_gemm_select_config(m, d, hdim, epilogue="none", out_kind="bf16")
    torch.cuda.synchronize()

    def step(i, ev=None, producer=False):
        j = i % SETS
        if ev is not None:
            ev[0].record()
        if producer:
            mx.mx_rmsnorm_quantize(xs[j], gam, shift, scale, 10240, 1e-6, "e2m3", out=xqs[j])
        else:
            mx.mx_quantize(xs[j], "e2m3", "tiled", out=xqs[j])
        if ev is not None:
            ev[1].record()
        mx.mx_gemm(xqs[j], w1s[j], out_kind="mx", epilogue="gelu_tanh", out=hs[j], config=cfg1)
        if ev is not None:
            ev[2].record()
        mx.mx_gemm(hs[j], w2s[j], out_kind="bf16", out=ys[j], config=cfg2)
        if ev is not None:
            ev[3].record()

    def run(producer: bool):
        it = [0]

        def one():
            step(it[0], producer=producer)
            it[0] += 1

        settle(one)
        for i in range(warmup):
            step(i, producer=producer)
        torch.cuda.synchronize()
        evs = [_events(4) for _ in range(steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            step(i, evs[i], producer=producer)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        q = [e[0].elapsed_time(e[1]) for e in evs]
        f1 = [e[1].elapsed_time(e[2]) for e in evs]
        f2 = [e[2].elapsed_time(e[3]) for e in evs]
        return wall * 1e3 / steps, q, f1, f2

    ms_step, q_ms, f1_ms, f2_ms = run(False)
    p_step, p_ms, pf1_ms, pf2_ms = run(True)
    flops_gemm = 2.0 * m * d * hdim
    return {
        "wall_ms_per_step": ms_step,
        "quantize": stats(q_ms), "fc1": stats(f1_ms), "fc2": stats(f2_ms),
        "quantize_ms": float(np.mean(q_ms)),
        "fc1_ms": float(np.mean(f1_ms)),
        "fc2_ms": float(np.mean(f2_ms)),
        "producer_step": {"ms_per_step": round(p_step, 4), "producer": stats(p_ms), "fc1": stats(pf1_ms),
                          "fc2": stats(pf2_ms)},
        "flops_per_step": 2 * flops_gemm,
        "flops_per_gemm": flops_gemm,
        "quantize_bytes": m * d * 2 + m * d * 3 // 4 + m * d // 32,
        "fc1_bytes": m * d * 3 // 4 + m * d // 32 + hdim * d * 3 // 4 + hdim * d // 32 + m * hdim * 3 // 4 + m * hdim // 32,
        "fc2_bytes": m * hdim * 3 // 4 + m * hdim // 32 + d * hdim * 3 // 4 + d * hdim // 32 + m * d * 2,
        "tuning": {k: {"config": v["config"], "us": v["us"], "default_us": v["default_us"]} for k, v in tuned.items()},
        "configs": {"fc1": list(cfg1.key()), "fc2": list(cfg2.key())},
        "kernels": {"fc1": kernel_name("fc1", cfg1), "fc2": kernel_name("fc2", cfg2)},
    }


def bench_proj(table, iters: int = 50):
    """The projection-shaped GEMM (4096 x 3072 x 3072): bf16 activations
    quantized inside the call (the call a user makes: quantize + GEMM), and
    the GEMM alone on activations quantized beforehand; bf16 out; weights
    pre-quantized; three rotating buffer sets."""
    w = syn.WORKLOADS["proj"]
    dev = torch.device("cuda:0")
    a_host, w_host = syn.make_a(w), syn.make_w(w)
    a_s = [a_host.to(dev) for _ in range(SETS)]
    aq_s = [mx.mx_quantize(a, "e2m3") for a in a_s]
    w_s = [mx.mx_quantize(w_host.to(dev), "e2m3") for _ in range(SETS)]
    outs = [torch.empty((w.m, w.n), dtype=torch.bfloat16, device=dev) for _ in range(SETS)]
    work = torch.empty(mx.mx_gemm_workspace_size(w.m, w.n, w.k, True, 0), dtype=torch.uint8, device=dev)
    cfg = table.lookup(w.m, w.n, w.k) or mx.mx_gemm_select_config(w.m, w.n, w.k)
    call_fn = lambda i: mx.mx_gemm(a_s[i % SETS], w_s[i % SETS], out_kind="bf16", out=outs[i % SETS],  # noqa: E731
                                   workspace=work, config=cfg)
    kern_fn = lambda i: mx.mx_gemm(aq_s[i % SETS], w_s[i % SETS], out_kind="bf16", out=outs[i % SETS],  # noqa: E731
                                   config=cfg)
    flops = 2.0 * w.m * w.n * w.k
    alg = w.m * w.k * 2 + w.n * w.k * 3 // 4 + w.n * w.k // 32 + w.m * w.n * 2
    c, k = time_batches(call_fn, iters), time_batches(kern_fn, iters)
    return {"workload": "projection 4096x3072x3072, bf16 activations quantized in the call (E2M3), "
                        "E2M3 weights, bf16 out",
            "call_ms": c, "kernel_ms": k, "call_ms_each_bracketed": stats(time_calls(call_fn, iters)),
            "kernel_ms_each_bracketed": stats(time_calls(kern_fn, iters)), "config": list(cfg.key()),
            "tflops": round(flops / c["median"] / 1e9, 1), "frac": round(flops / c["median"] / 1e9 / PEAK_MXFP6_TFLOPS, 4),
            "kernel_tflops": round(flops / k["median"] / 1e9, 1),
            "kernel_frac": round(flops / k["median"] / 1e9 / PEAK_MXFP6_TFLOPS, 4),
            "algorithmic_bytes": alg, "gb_s": round(alg / c["median"] / 1e6, 1)}


def bench_mlp_share(table, m: int = 2560, iters: int = 50):
    """The MLP step on one GPU's share of the 20480 tokens when sequence
    parallelism spreads them over 8 GPUs (2560 tokens: quantize x, fc1 GELU ->
    E2M3, fc2 bf16), with the same weights, three rotating buffer sets and
    the tuning table's configurations (the nearest tuned shapes)."""
    fc1, fc2 = syn.WORKLOADS["fc1"], syn.WORKLOADS["fc2"]
    d, hdim = fc1.k, fc1.n
    dev = torch.device("cuda:0")
    x_host = syn.make_a(fc1, m=m)
    xs = [x_host.to(dev) for _ in range(SETS)]
    w1s = [mx.mx_quantize(syn.make_w(fc1).to(dev), "e2m3") for _ in range(SETS)]
    w2s = [mx.mx_quantize(syn.make_w(fc2).to(dev), "e2m3") for _ in range(SETS)]
    xqs = [mx.MXTensor.empty(m, d, "e2m3", "tiled", dev) for _ in range(SETS)]
    hs = [mx.MXTensor.empty(m, hdim, "e2m3", "tiled", dev) for _ in range(SETS)]
    ys = [torch.empty((m, d), dtype=torch.bfloat16, device=dev) for _ in range(SETS)]
    cfg1 = (table.lookup(m, hdim, d, epilogue="gelu_tanh", out_kind="mx")
            or mx.mx_gemm_select_config(m, hdim, d, epilogue="gelu_tanh", out_kind="mx"))
    cfg2 = table.lookup(m, d, hdim) or mx.mx_gemm_select_config(m, d, hdim)

    def step(i):
        j = i % SETS
        mx.mx_quantize(xs[j], "e2m3", "tiled", out=xqs[j])
        mx.mx_gemm(xqs[j], w1s[j], out_kind="mx", epilogue="gelu_tanh", out=hs[j], config=cfg1)
        mx.mx_gemm(hs[j], w2s[j], out_kind="bf16", out=ys[j], config=cfg2)

    settle(lambda: step(0))
    t = time_batches(step, iters)
    flops = 2 * 2.0 * m * d * hdim
    return {"workload": f"DiT MLP step on {m} tokens (one GPU's share of 20480 over 8 GPUs): quantize x, "
                        f"fc1 {m}x3072x12288 (GELU -> E2M3), fc2 {m}x12288x3072 (bf16 out)",
            "tokens": m, "ms_per_step": t, "tflops": round(flops / t["median"] / 1e9, 1),
            "frac": round(flops / t["median"] / 1e9 / PEAK_MXFP6_TFLOPS, 4),
            "configs": [list(cfg1.key()), list(cfg2.key())]}


def bench_tiny(iters: int = 50):
    """The tiny 256^3 GEMM (E2M3 x E2M3, fp32 out, activations quantized in
    the call): launch-latency bound, reported for completeness."""
    w = syn.WORKLOADS["tiny"]
    dev = torch.device("cuda:0")
    a = syn.make_a(w).to(dev)
    wq = mx.mx_quantize(syn.make_w(w).to(dev), "e2m3")
    out = torch.empty((w.m, w.n), dtype=torch.float32, device=dev)
    work = torch.empty(mx.mx_gemm_workspace_size(w.m, w.n, w.k, True, 0), dtype=torch.uint8, device=dev)
    call = time_batches(lambda i: mx.mx_gemm(a, wq, out_kind="f32", out=out, workspace=work), iters)
    return {"workload": "tiny 256x256x256 E2M3, quantized in the call, fp32 out", "call_ms": call,
            "tflops": round(2.0 * w.m * w.n * w.k / call["median"] / 1e9, 2)}


def bench_swiglu_mlp(table, steps: int, warmup: int):
    """The SwiGLU variant of the MLP step (the activation the Krea 3 post names):
    quantize x, stacked gate/up GEMM 20480 x 3072 x 16384 with SwiGLU -> E2M3
    (8192 features), down projection 20480 x 8192 x 3072 to bf16."""
    w1w, w2w = syn.WORKLOADS["sw_fc1"], syn.WORKLOADS["sw_fc2"]
    m, d, n1 = w1w.m, w1w.k, w1w.n
    hdim = n1 // 2
    dev = torch.device("cuda:0")
    x = syn.make_a(w1w).to(dev)
    w1 = mx.mx_quantize(syn.make_w(w1w).to(dev), "e2m3")
    w2 = mx.mx_quantize(syn.make_w(w2w).to(dev), "e2m3")
    xq = mx.MXTensor.empty(m, d, "e2m3", "tiled", dev)
    h = mx.MXTensor.empty(m, hdim, "e2m3", "tiled", dev)
    y = torch.empty((m, d), dtype=torch.bfloat16, device=dev)
    # launch configurations from the tuning table where it has these shapes
    cfg1 = table.lookup(m, n1, d, epilogue="swiglu", out_kind="mx")
    cfg2 = table.lookup(m, d, hdim, epilogue="none", out_kind="bf16")

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        mx.mx_quantize(x, "e2m3", "tiled", out=xq)
        if ev is not None:
            ev[1].record()
        mx.mx_gemm(xq, w1, out_kind="mx", epilogue="swiglu", out=h, config=cfg1)
        if ev is not None:
            ev[2].record()
        mx.mx_gemm(h, w2, out_kind="bf16", out=y, config=cfg2)
        if ev is not None:
            ev[3].record()

    settle(step, 0.3)
    for _ in range(warmup):
        step()
    evs = [_events(4) for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    f1 = np.array([e[1].elapsed_time(e[2]) for e in evs]).mean()
    f2 = np.array([e[2].elapsed_time(e[3]) for e in evs]).mean()
    fl1, fl2 = 2.0 * m * d * n1, 2.0 * m * hdim * d
    return {"workload": "SwiGLU MLP forward: quantize x, gate/up 20480x3072x16384 (SwiGLU -> E2M3, 8192 "
                        "features), down 20480x8192x3072 (bf16 out)",
            "ms_per_step": round(wall * 1e3 / steps, 4), "tflops": round((fl1 + fl2) / (wall / steps) / 1e12, 1),
            "fc1_ms": round(float(f1), 4), "fc1_tflops": round(fl1 / f1 / 1e9, 1),
            "fc2_ms": round(float(f2), 4), "fc2_tflops": round(fl2 / f2 / 1e9, 1),
            "configs": [list(c.key()) if c is not None else None for c in (cfg1, cfg2)]}


PEAK_BY_FMT = {"e2m3": 10100.0, "e2m1": 10100.0, "e4m3": 5000.0, "e5m2": 5000.0}


def bench_formats(table, iters: int = 20, tune: bool = True):
    """The operand formats of the same scaled matrix instruction on fc1's shape
    (20480 x 3072 x 12288, both operands pre-quantized, bf16 out, no
    epilogue): MXFP6 E2M3, MXFP4 E2M1 and MXFP8 E4M3, each against its own
    dense peak (10.1 PF for FP6 and FP4, 5.0 PF for FP8), each in the launch
    configuration the tuning table picks for it (tuned untimed, first)."""
    w = syn.WORKLOADS["fc1"]
    dev = torch.device("cuda:0")
    a_src = syn.make_a(w).to(dev)
    w_src = syn.make_w(w).to(dev)
    out = torch.empty((w.m, w.n), dtype=torch.bfloat16, device=dev)
    flops = 2.0 * w.m * w.n * w.k
    res = {}
    for fmt in ("e2m3", "e2m1", "e4m3"):
        aq, wq = mx.mx_quantize(a_src, fmt), mx.mx_quantize(w_src, fmt)
        cfg = table.lookup(w.m, w.n, w.k, fmt, fmt, "none", "bf16")
        if tune and cfg is None:
            tuning.tune_gemm(table, aq, wq, out_kind="bf16")
            cfg = table.lookup(w.m, w.n, w.k, fmt, fmt, "none", "bf16")
        elif not tune:
            cfg = None

        def call():
            mx.mx_gemm(aq, wq, out_kind="bf16", out=out, config=cfg)

        settle(call, 0.2)
        e0, e1 = _events(2)
        e0.record()
        for _ in range(iters):
            call()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / iters
        tf = flops / ms / 1e9
        res[fmt] = {"ms": round(ms, 4), "tflops": round(tf, 1), "peak_tflops": PEAK_BY_FMT[fmt],
                    "frac": round(tf / PEAK_BY_FMT[fmt], 4),
                    "config": list(cfg.key()) if cfg is not None else list(mx.mx_gemm_default_config().key())}
        del aq, wq
    return {"workload": "fc1-shaped GEMM 20480x3072x12288, pre-quantized operands, bf16 out", **res}


def bench_producer(iters: int = 50):
    """The quantize-once producer on fc1's input: RMSNorm with a gain, two
    conditionings of 10240 rows (modulation), MX E2M3 into the tiled layout.
    HBM-bound: algorithmic bytes = the bf16 input once + the packed output."""
    w = syn.WORKLOADS["fc1"]
    dev = torch.device("cuda:0")
    x = syn.make_a(w).to(dev)
    g = torch.ones(w.k, dtype=torch.float32, device=dev)
    sh = torch.zeros((2, w.k), dtype=torch.float32, device=dev)
    sc = torch.zeros((2, w.k), dtype=torch.float32, device=dev)
    out = mx.MXTensor.empty(w.m, w.k, "e2m3", "tiled", dev)

    def call():
        mx.mx_rmsnorm_quantize(x, g, sh, sc, 10240, 1e-6, "e2m3", out=out)

    settle(call, 0.2)
    e0, e1 = _events(2)
    e0.record()
    for _ in range(iters):
        call()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / iters
    # the same call with the 256 MB last-level cache flushed first (a 768 MB
    # fill between calls, outside the timed events): x then comes from HBM
    flush = torch.empty(768 << 20, dtype=torch.uint8, device=dev)
    cold = []
    for it in range(iters // 2):
        flush.fill_(it & 0xFF)
        e0, e1 = _events(2)
        e0.record()
        call()
        e1.record()
        torch.cuda.synchronize()
        cold.append(e0.elapsed_time(e1))
    del flush
    ms_cold = float(np.mean(cold[2:]))
    alg = w.m * w.k * 2 + w.m * w.k * 3 // 4 + w.m * w.k // 32
    return {"workload": "RMSNorm + modulation + E2M3 of 20480x3072 bf16 (fc1 input)", "ms": round(ms, 4),
            "algorithmic_bytes": alg, "gb_s": round(alg / ms / 1e6, 1), "hbm_frac": round(alg / ms / 1e6 / PEAK_HBM_GBS, 4),
            "ms_cold_cache": round(ms_cold, 4), "gb_s_cold_cache": round(alg / ms_cold / 1e6, 1)}


def bench_stacked_projection(table, iters: int = 10):
    """Quantize once, then one GEMM for the stacked projections: the producer
    (RMSNorm + modulation + E2M3) on 20480 x 3072 bf16, then one mx_gemm over
    the stacked [Wq; Wk; Wv; Wgate] weights (12288 x 3072, bf16 out), against
    the same four projections as four GEMMs of 3072 x 3072 on the same
    quantized activations."""
    w = syn.WORKLOADS["fc1"]
    dev = torch.device("cuda:0")
    x = syn.make_a(w).to(dev)
    g = torch.ones(w.k, dtype=torch.float32, device=dev)
    sh = torch.zeros((2, w.k), dtype=torch.float32, device=dev)
    sc = torch.zeros((2, w.k), dtype=torch.float32, device=dev)
    a = mx.MXTensor.empty(w.m, w.k, "e2m3", "tiled", dev)
    wsrc = syn.make_w(w).to(dev)  # 12288 = 4 x 3072 rows: q, k, v, gate
    w_stack = mx.mx_quantize(wsrc, "e2m3")
    d = w.k
    w_parts = [mx.mx_quantize(wsrc[i * d:(i + 1) * d].contiguous(), "e2m3") for i in range(4)]
    del wsrc
    out = torch.empty((w.m, w.n), dtype=torch.bfloat16, device=dev)
    outs = [torch.empty((w.m, d), dtype=torch.bfloat16, device=dev) for _ in range(4)]
    cfg = table.lookup(w.m, w.n, w.k, epilogue="none", out_kind="bf16")

    def fused():
        mx.mx_rmsnorm_quantize(x, g, sh, sc, 10240, 1e-6, "e2m3", out=a)
        mx.mx_gemm(a, w_stack, out_kind="bf16", out=out, config=cfg)

    def separate():
        mx.mx_rmsnorm_quantize(x, g, sh, sc, 10240, 1e-6, "e2m3", out=a)
        for wp, o in zip(w_parts, outs):
            mx.mx_gemm(a, wp, out_kind="bf16", out=o)

    res = {"workload": "RMSNorm + modulation + E2M3 of 20480x3072 bf16, then stacked QKV + gate 20480x3072x12288 "
                       "(bf16 out)"}
    flops = 2.0 * w.m * w.n * w.k
    for name, fn in (("one_stacked_gemm", fused), ("four_gemms", separate)):
        settle(fn, 0.2)
        e0, e1 = _events(2)
        e0.record()
        for _ in range(iters):
            fn()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / iters
        res[name] = {"ms": round(ms, 4), "tflops": round(flops / ms / 1e9, 1)}
    res["config"] = list(cfg.key()) if cfg is not None else None
    return res


def bench_skinny(m: int, splits: int, iters: int, copies: int = SETS):
    """Skinny split-K: the call (activations quantized inside it) and the
    split-K kernel alone (activations quantized beforehand), rotating over
    `copies` weight copies (the 170 MB of weights fit in the 256 MB
    last-level cache otherwise); per-call median and min."""
    w = syn.WORKLOADS["skinny"]
    dev = torch.device("cuda:0")
    a = syn.make_a(w, m=m).to(dev)
    wb = syn.make_w(w).to(dev)
    ws = [mx.mx_quantize(wb, w.w_fmt, "tiled") for _ in range(copies)]
    del wb
    out = torch.empty((m, w.n), dtype=torch.bfloat16, device=dev)
    work = torch.empty(mx.mx_gemm_workspace_size(m, w.n, w.k, True, splits), dtype=torch.uint8, device=dev)
    call_fn = lambda i: mx.mx_gemm_splitk(a, ws[i % copies], splits, out=out, workspace=work)  # noqa: E731
    call = time_batches(call_fn, iters)
    call_each = stats(time_calls(call_fn, iters))
    aq = mx.mx_quantize(a, "e2m3", "tiled")
    kern_fn = lambda i: mx.mx_gemm_splitk(aq, ws[i % copies], splits, out=out)  # noqa: E731
    kern = time_batches(kern_fn, iters)
    kern_each = stats(time_calls(kern_fn, iters))
    wbytes = w.n * w.k * 3 // 4 + w.n * w.k // 32
    alg = wbytes + m * w.k * 2 + m * w.n * 2
    kalg = wbytes + m * w.k * 3 // 4 + m * w.k // 32 + m * w.n * 2
    ms, kms = call["median"], kern["median"]
    return {"m": m, "splits": splits, "ms": ms, "call_ms": call, "call_ms_each_bracketed": call_each,
            "algorithmic_bytes": alg, "gb_s": alg / ms / 1e6,
            "hbm_frac": alg / ms / 1e6 / PEAK_HBM_GBS, "hbm_frac_best": alg / call["min"] / 1e6 / PEAK_HBM_GBS,
            "tflops": 2.0 * m * w.n * w.k / ms / 1e9,
            "kernel_ms": kms, "kernel_call_ms": kern, "kernel_ms_each_bracketed": kern_each,
            "kernel_algorithmic_bytes": kalg, "kernel_gb_s": kalg / kms / 1e6,
            "kernel_hbm_frac": kalg / kms / 1e6 / PEAK_HBM_GBS}


def mfma_ceiling():
    """The matrix instruction's rate with nothing else in the loop (the
    measurement probe libmxprobe.so): 6-bit operands, one and two waves per
    SIMD, and 4-bit operands; with the average engine clock it ran at."""
    import ctypes

    from microscaled_precision_gemm_amd import build as B

    if not os.path.exists(B.PROBE_PATH):
        return None
    L = ctypes.CDLL(B.PROBE_PATH)
    f = L.mx_probe_mfma_ceiling
    f.argtypes = [ctypes.c_int] * 4 + [ctypes.POINTER(ctypes.c_double)] * 3
    f.restype = ctypes.c_int
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    res = {}
    for name, fmt, wgs in (("e2m3_1wave", 2, cus), ("e2m3_2waves", 2, 2 * cus), ("e2m1_1wave", 4, cus)):
        ms, tf, ghz = ctypes.c_double(), ctypes.c_double(), ctypes.c_double()
        if f(fmt, wgs, 20000, 3, ctypes.byref(ms), ctypes.byref(tf), ctypes.byref(ghz)) != 0:
            return None
        res[name] = {"tflops": round(tf.value, 1), "frac_of_peak": round(tf.value / PEAK_MXFP6_TFLOPS, 4),
                     "clock_ghz": round(ghz.value, 3), "ms": round(ms.value, 3)}
    return res


def gemm_sources_sha256() -> str:
    h = hashlib.sha256()
    for name in GEMM_SOURCES:
        with open(os.path.join(ROOT, "microscaled_precision_gemm_amd", "csrc", name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


def measured_traffic(gemm: str, kernel: str):
    """HBM bytes per launch of `gemm` ("fc1" / "fc2") from the committed
    rocprofv3 counter summary (FETCH_SIZE + WRITE_SIZE, each scaled by the same
    counter's reading for a copy of known size), or None when the summary is
    missing, was taken of another kernel (tile width) than `kernel`, or the
    GEMM sources changed since it was taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            text = f.read()
    except OSError:
        return None
    m = re.search(r"^kernel_sources_sha256: ([0-9a-f]{64})$", text, re.M)
    t = re.search(rf"^{gemm}_traffic_bytes_per_launch: (\d+)$", text, re.M)
    k = re.search(rf"^{gemm}_kernel: (.+)$", text, re.M)
    if not m or not t or not k or m.group(1) != gemm_sources_sha256() or k.group(1).strip() != kernel:
        return None
    return int(t.group(1))


def copy_calibration(mib: int = 1024, reps: int = 3):
    """A plain device copy of known size, for scaling the FETCH_SIZE /
    WRITE_SIZE counters (each copy reads and writes `mib` MiB once)."""
    src = torch.ones(mib << 20, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    return {"bytes_each_way": mib << 20, "reps": reps}


def _oracle_weights():
    """The fc1 and fc2 weights quantized and dequantized by the oracle (the
    weights are pre-quantized on the GPU side too: untimed)."""
    from oracle import mx_oracle as O

    fc1, fc2 = syn.WORKLOADS["fc1"], syn.WORKLOADS["fc2"]
    w1 = O.dequantize(*O.quantize(syn.as_f64(syn.make_w(fc1)), "e2m3"), "e2m3")
    w2 = O.dequantize(*O.quantize(syn.as_f64(syn.make_w(fc2)), "e2m3"), "e2m3")
    return w1, w2


def cpu_baseline(w1, w2, target_s: float = 15.0):
    """The CPU oracle (as written, untuned) on a bounded sample of the step:
    the same MLP pass for a sample of token rows (weights quantized once,
    untimed, as on the GPU side)."""
    from threadpoolctl import threadpool_info

    from oracle import mx_oracle as O

    fc1 = syn.WORKLOADS["fc1"]
    d, hdim = fc1.k, fc1.n
    x_all = syn.make_a(fc1)

    def run(rows):
        x = syn.as_f64(x_all[:rows])
        t0 = time.perf_counter()
        a = O.dequantize(*O.quantize(x, "e2m3"), "e2m3")
        codes, scales, *_ = O.fc1_gelu_mx_ref(a, w1)
        O.gemm_ref(O.dequantize(codes, scales, "e2m3"), w2)
        return time.perf_counter() - t0

    # size the sample from two probes (the first, on 32 rows, is dominated by
    # fixed costs), then run it
    rows = 32
    for frac in (0.2, 1.0):
        t = run(rows)
        rows = int(min(fc1.m, max(32, rows * frac * target_s / max(t, 1e-3))) // 32 * 32)
    t = run(rows)
    flops = 2 * 2.0 * rows * d * hdim
    threads = sum(p.get("num_threads", 0) for p in threadpool_info() if p.get("user_api") == "blas") or 1
    return {"value": flops / t / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"MLP fc1(GELU->E2M3)+fc2 on {rows} of 20480 token rows, float64 numpy, weights pre-quantized",
            "seconds": t, "host_cpus": len(os.sched_getaffinity(0))}


def oracle_per_config(w1, w2) -> dict:
    """The CPU oracle's time for each workload, from a timed sample scaled to
    the whole workload (the oracle's cost is linear in the sampled rows):
    what the call computes, with the weights quantized beforehand as on the
    GPU side.  ms = estimate for the whole workload."""
    from oracle import mx_oracle as O

    W = syn.WORKLOADS
    res = {}

    def t_ms(fn):
        t0 = time.perf_counter()
        fn()
        return (time.perf_counter() - t0) * 1e3

    deq = lambda x, f: O.dequantize(*O.quantize(x, f), f)  # noqa: E731
    # tiny: the whole GEMM (quantize A, exact product), weights untimed
    w = W["tiny"]
    dw = deq(syn.as_f64(syn.make_w(w)), "e2m3")
    a = syn.as_f64(syn.make_a(w))
    res["tiny"] = {"ms": round(t_ms(lambda: O.gemm_ref(deq(a, "e2m3"), dw)), 2), "sample": "whole GEMM"}
    # proj: 512 of 4096 token rows, quantized in the call
    w = W["proj"]
    dw = deq(syn.as_f64(syn.make_w(w)), "e2m3")
    a = syn.as_f64(syn.make_a(w, m=512))
    res["proj"] = {"ms": round(t_ms(lambda: O.gemm_ref(deq(a, "e2m3"), dw)) * w.m / 512, 1),
                   "sample": "512 of 4096 token rows, scaled"}
    # fc1: 64 of 20480 rows: quantize, GEMM, GELU, E2M3 along N
    w = W["fc1"]
    a = syn.as_f64(syn.make_a(w, m=64))
    res["fc1"] = {"ms": round(t_ms(lambda: O.fc1_gelu_mx_ref(deq(a, "e2m3"), w1)) * w.m / 64, 1),
                  "sample": "64 of 20480 token rows, scaled"}
    # fc2: 64 rows of the E2M3 activations (quantized beforehand, untimed)
    w = W["fc2"]
    da = deq(syn.as_f64(syn.make_a(w, m=64)), "e2m3")
    res["fc2"] = {"ms": round(t_ms(lambda: O.gemm_ref(da, w2)) * w.m / 64, 1),
                  "sample": "64 of 20480 token rows, scaled"}
    # skinny: 16 tokens quantized in the call; the product against 512 of 13312 weight rows, scaled
    w = W["skinny"]
    dw = deq(syn.as_f64(syn.make_w(w, n=512)), w.w_fmt)
    a = syn.as_f64(syn.make_a(w, m=16))
    tq = t_ms(lambda: deq(a, "e2m3"))
    da = deq(a, "e2m3")
    res["skinny_m16"] = {"ms": round(tq + t_ms(lambda: O.gemm_ref(da, dw)) * w.n / 512, 2),
                         "sample": "16 tokens, 512 of 13312 weight rows for the product, scaled"}
    return res


def main():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=100)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--skinny-iters", type=int, default=100)
    p.add_argument("--no-tune", action="store_true", help="use the library's default launch configuration")
    p.add_argument("--tuning-table", default=tuning.SHIPPED_TABLE,
                   help="JSON tuning table to read the GEMM configurations from (default: the table shipped "
                        "with the package); shapes it lacks for this device are tuned here, untimed")
    p.add_argument("--save-tuning", default=None, help="write the resulting tuning table to this path")
    p.add_argument("--copy-calibration", action="store_true",
                   help="also run a 1 GiB device copy (for scaling rocprofv3 byte counters)")
    args = p.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(json.dumps({"error": "bench.py measures one GPU (the sharded path is a design, not a measurement here); --gpus must be 1"}))
        sys.exit(2)
    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(2)

    table = tuning.TuningTable(args.tuning_table if args.tuning_table and os.path.exists(args.tuning_table) else None)
    r = bench_mlp(table, args.steps, args.warmup, tune=not args.no_tune)
    ms_step = r["wall_ms_per_step"]
    value = r["flops_per_step"] / ms_step / 1e9  # TFLOP/s
    # dominant kernel: the slower of the two GEMMs, timed with events on its own stream
    dom = "fc1" if r["fc1_ms"] >= r["fc2_ms"] else "fc2"
    dom_ms = r[f"{dom}_ms"]
    achieved = r["flops_per_gemm"] / dom_ms / 1e9
    ceiling = mfma_ceiling()
    skinny = [bench_skinny(mm, ss, args.skinny_iters) for ss in (16, 8) for mm in (16, 8)]
    proj = bench_proj(table if not args.no_tune else tuning.TuningTable())
    tiny = bench_tiny()
    share = bench_mlp_share(table if not args.no_tune else tuning.TuningTable())
    share["full_step_ms_over_8"] = round(ms_step / 8, 4)
    swiglu = bench_swiglu_mlp(table if not args.no_tune else tuning.TuningTable(), args.steps, args.warmup)
    producer = bench_producer()
    stacked = bench_stacked_projection(table if not args.no_tune else tuning.TuningTable())
    formats = bench_formats(table, tune=not args.no_tune)
    if args.save_tuning and not args.no_tune:
        table.save(args.save_tuning)
    fl = r["flops_per_gemm"]
    tf = lambda ms: round(fl / ms / 1e9, 1)  # noqa: E731
    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "mxfp6_e2m3",
        "data": "synthetic",
        "inputs": {"generator": "numpy default_rng([workload index, stream]); stream 0 = activations, 1 = weights, "
                                "2 = the outlier-channel choice; float32 draws rounded to bfloat16 (RNE)",
                   "seeds": {name: {"activations": [w.index, 0], "weights": [w.index, 1]}
                             for name, w in syn.WORKLOADS.items()},
                   "mlp_step": "x = fc1 activations, W1 = fc1 weights, W2 = fc2 weights; fc2 reads fc1's output"},
        "config": {"workload": "DiT MLP forward: quantize x, fc1 20480x3072x12288 (GELU-tanh -> E2M3), "
                               "fc2 20480x12288x3072 (bf16 out)",
                   "tokens": 20480, "d_model": 3072, "d_hidden": 12288, "buffer_sets": SETS,
                   "frac_of_mxfp6_peak": round(value / PEAK_MXFP6_TFLOPS, 4)},
        "roofline": {"bound": "mfma", "kernel": f"{r['kernels'][dom]} ({dom})", "achieved": round(achieved, 1),
                     "peak": PEAK_MXFP6_TFLOPS, "unit": "TFLOP/s", "frac": round(achieved / PEAK_MXFP6_TFLOPS, 4),
                     "traffic": measured_traffic(dom, r["kernels"][dom]), "traffic_unit": "bytes per launch",
                     "algorithmic_bytes": r[f"{dom}_bytes"], "avg_launch_ms": round(dom_ms, 4),
                     "median_launch_ms": r[dom]["median"], "min_launch_ms": r[dom]["min"]},
        "kernels_ms": {"quantize": r["quantize"], "fc1": r["fc1"], "fc2": r["fc2"],
                       "fc1_tflops": tf(r["fc1"]["median"]), "fc2_tflops": tf(r["fc2"]["median"]),
                       "fc1_tflops_best": tf(r["fc1"]["min"]), "fc2_tflops_best": tf(r["fc2"]["min"]),
                       "quantize_gb_s": round(r["quantize_bytes"] / r["quantize"]["median"] / 1e6, 1)},
        "mfma_only_ceiling": ceiling,
        "tuning": r["tuning"],
        "gemm_configs": r["configs"],
        "gemm_kernels": r["kernels"],
        "producer_fed_step": {"workload": "the same step with RMSNorm + modulation + E2M3 (mx_rmsnorm_quantize) "
                                          "producing fc1's input instead of mx_quantize",
                              **r["producer_step"]},
        "proj": proj,
        "tiny": tiny,
        "share_of_8_gpus": share,
        "skinny_splitk": [{k: (round(v, 4) if isinstance(v, float) else v) for k, v in s_.items()} for s_ in skinny],
        "swiglu_mlp": swiglu,
        "producer": producer,
        "stacked_projection": stacked,
        "operand_formats": formats,
    }
    if ceiling:
        c1 = ceiling["e2m3_1wave"]["tflops"]
        line["mfma_only_ceiling"]["fc1_frac_of_ceiling"] = round(tf(r["fc1"]["median"]) / c1, 4)
        line["mfma_only_ceiling"]["fc2_frac_of_ceiling"] = round(tf(r["fc2"]["median"]) / c1, 4)
    if args.copy_calibration:
        line["copy_calibration"] = copy_calibration()
    if not args.no_cpu_baseline:
        w1, w2 = _oracle_weights()
        line["cpu_baseline"] = {k: (round(v, 6) if isinstance(v, float) else v) for k, v in cpu_baseline(w1, w2).items()}
        orc = oracle_per_config(w1, w2)
        gpu = {"tiny": tiny["call_ms"]["median"], "proj": proj["call_ms"]["median"], "fc1": r["fc1"]["median"],
               "fc2": r["fc2"]["median"], "skinny_m16": skinny[0]["call_ms"]["median"]}
        line["oracle_vs_gpu_ms"] = {k: {"oracle_ms": v["ms"], "gpu_ms": gpu[k], "oracle_sample": v["sample"]}
                                    for k, v in orc.items()}
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
