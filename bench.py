#!/usr/bin/env python3
"""Benchmark of the SmoothQuant W8A8 linear-layer path on one MI355X.

One step = the whole path once, on one batch of synthetic input already in
HBM: calibration absmax over the calibration tokens, smoothing factors,
smoothed per-output-channel INT8 weights, smoothed per-token INT8
activations, INT8 GEMM with the dequant epilogue to bf16.  Inputs rotate over
a pool of independent sets larger than the 256 MB Infinity Cache, so reads
come from HBM.

Prints ONE JSON line with the whole-step throughput, a per-kernel breakdown,
the roofline of the dominant kernel (the GEMM) measured with HIP events on the
stream the library launches on, and a CPU baseline (the oracle timed on a
bounded sample on the host cores).

    python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--config 2] [--no-cpu]
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

HBM_PEAK_GBS = 8000.0      # MI355X HBM3E, GB/s
INT8_PEAK_TOPS = 5000.0    # MI355X dense INT8 MFMA, TOPS (5.0 POP/s)
METRIC = "W8A8 GEMM TOPS (% INT8 MFMA peak); quant-kernel HBM GB/s (% peak)"


def _parse():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--config", type=int, default=2, help="workload: 2 = attention projection 2048x4096x4096")
    p.add_argument("--pool-gb", type=float, default=1.0, help="rotate inputs over at least this many GB")
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baseline")
    p.add_argument("--cpu-seconds", type=float, default=15.0, help="target CPU time of the oracle sample")
    return p.parse_args()


def _cpu_baseline(cfg, target_s: float):
    """Time the oracle (as it stands) on the host cores over a bounded sample
    of the same workload, scaled to whole-step TOPS."""
    import numpy as np

    import oracle
    import synth

    cores = len(os.sched_getaffinity(0))
    M, K, N = cfg.M, cfg.K, cfg.N
    inp = synth.make(cfg, device="cpu")
    x, w, cal = synth.to_numpy(inp.x), synth.to_numpy(inp.w), synth.to_numpy(inp.calib)
    t = {}
    t0 = time.perf_counter()
    amax = oracle.calib_absmax(cal)
    t["calib_absmax"] = time.perf_counter() - t0
    t0 = time.perf_counter()
    aw = oracle.weight_rowmax(w)
    s, inv_s = oracle.smooth_factors(amax, aw, cfg.alphas[0])
    t["smooth_factors"] = time.perf_counter() - t0
    t0 = time.perf_counter()
    wq, ws = oracle.quant_weight(w, s)
    t["quant_weight"] = time.perf_counter() - t0
    t0 = time.perf_counter()
    xq, xs = oracle.quant_act(x, inv_s, oracle.PER_TOKEN)
    t["quant_act"] = time.perf_counter() - t0
    # GEMM: a probe on a few rows sizes the sample so it takes ~target_s.
    probe = max(1, min(M, 8))
    t0 = time.perf_counter()
    oracle.gemm_i8(xq[:probe], wq, nthreads=min(cores, probe))
    per_row = (time.perf_counter() - t0) / probe * min(cores, probe) / cores
    spent = sum(t.values())
    rows = int(max(cores, min(M, (max(target_s - spent, 1.0)) / max(per_row, 1e-9))))
    rows = min(M, (rows + cores - 1) // cores * cores)
    t0 = time.perf_counter()
    acc = oracle.gemm_i8(xq[:rows], wq, nthreads=cores)
    g = time.perf_counter() - t0
    t0 = time.perf_counter()
    oracle.dequant(acc, xs[:rows], oracle.PER_TOKEN, ws)
    d = time.perf_counter() - t0
    t["gemm_w8a8"] = (g + d) * M / rows
    total = sum(t.values())
    ops = 2.0 * M * N * K
    return {
        "value": ops / total / 1e12, "unit": "TOPS", "cores": cores, "kind": "oracle",
        "sample": (f"all five oracle steps on the full {M}x{K}x{N} workload ({cfg.calib_tokens} calibration "
                   f"tokens), except the GEMM + dequant, timed on {rows} of {M} token rows and scaled by "
                   f"{M / rows:.2f}; GEMM on {cores} threads, other steps single-threaded"),
        "seconds_per_step": total, "stage_seconds": {k: round(v, 4) for k, v in t.items()},
        "cpu_model": _cpu_model(),
    }


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def main():
    args = _parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(f"bench.py measures one GPU only: this path runs on a single MI355X and has no multi-GPU mode "
              f"(asked for --gpus {args.gpus}).", file=sys.stderr)
        sys.exit(2)

    import torch

    import post_quantization_act_amd as sq
    import synth
    from post_quantization_act_amd import pipeline

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    cfg = synth.CONFIGS[args.config]
    M, K, N = cfg.M, cfg.K, cfg.N
    alpha = cfg.alphas[0]
    gran = sq.SQ_PER_TENSOR if cfg.gran == "per_tensor" else sq.SQ_PER_TOKEN
    esz = 2 if cfg.x_dtype == "bf16" else 4
    T = cfg.calib_tokens

    set_bytes = (M * K + K * N + T * K) * esz
    pool = max(1, int(-(-args.pool_gb * 1e9 // set_bytes)))
    print(f"# workload {cfg.name}: M={M} K={K} N={N} T={T} alpha={alpha}; pool of {pool} input sets "
          f"({pool * set_bytes / 1e9:.2f} GB)", file=sys.stderr, flush=True)
    sets = [synth.make(cfg, device=dev, variant=v) for v in range(pool)]
    torch.cuda.synchronize()
    b = pipeline.W8A8Buffers.allocate(M, N, K, gran, dev)
    stream = torch.cuda.current_stream(dev)

    stages = ["calib_absmax", "smooth_factors", "quant_weight", "quant_act", "gemm_w8a8"]

    def step(i, ev=None):
        s = sets[i % pool]
        if ev is not None:
            ev[0].record(stream)
        pipeline.calibrate(s.calib, b.amax_x)
        if ev is not None:
            ev[1].record(stream)
        sq.sq_smooth_factors(b.amax_x, s.w, alpha, b.s, b.inv_s, b.amax_w)
        if ev is not None:
            ev[2].record(stream)
        sq.sq_quant_weight(s.w, b.s, b.wq, b.w_scale, b.ws_w)
        if ev is not None:
            ev[3].record(stream)
        sq.sq_quant_act(s.x, b.inv_s, gran, b.xq, b.x_scale, b.ws_a)
        if ev is not None:
            ev[4].record(stream)
        sq.sq_gemm_w8a8(b.xq, b.x_scale, gran, b.wq, b.w_scale, b.y)
        if ev is not None:
            ev[5].record(stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    events = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(args.warmup + i, events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps

    per = {name: [] for name in stages}
    for ev in events:
        for k, name in enumerate(stages):
            per[name].append(ev[k].elapsed_time(ev[k + 1]) * 1e3)  # us
    avg_us = {name: sum(v) / len(v) for name, v in per.items()}

    ops = 2.0 * M * N * K
    bytes_alg = {
        "calib_absmax": T * K * esz + 8 * K,
        "smooth_factors": K * N * esz + 12 * K,
        "quant_weight": K * N * esz + N * K + 4 * N + 4 * K,
        "quant_act": M * K * esz + M * K + 4 * M + 4 * K,
        "gemm_w8a8": M * K + N * K + 2 * M * N + 4 * (M + N),
    }
    kernels = {}
    for name in stages:
        us = avg_us[name]
        gbs = bytes_alg[name] / (us * 1e-6) / 1e9
        kernels[name] = {"us": round(us, 2), "alg_bytes": bytes_alg[name], "GB_s": round(gbs, 1),
                         "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 1)}
    gemm_tops = ops / (avg_us["gemm_w8a8"] * 1e-6) / 1e12
    kernels["gemm_w8a8"].update({"ops": ops, "TOPS": round(gemm_tops, 1),
                                 "pct_int8_peak": round(100 * gemm_tops / INT8_PEAK_TOPS, 1)})

    value = ops / (ms_per_step * 1e-3) / 1e12
    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "TOPS", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "int8", "data": "synthetic",
        "config": {"workload": cfg.name, "M": M, "K": K, "N": N, "calib_tokens": T, "alpha": alpha,
                   "act_granularity": cfg.gran, "weight_granularity": "per_output_channel",
                   "input_dtype": cfg.x_dtype, "output_dtype": "bf16", "input_pool_sets": pool,
                   "value_definition": "2*M*N*K of the GEMM / wall time of one whole five-step pass"},
        "roofline": {"bound": "mfma", "kernel": "k_gemm_w8a8", "achieved": round(gemm_tops, 1),
                     "peak": INT8_PEAK_TOPS, "unit": "TOPS", "frac": round(gemm_tops / INT8_PEAK_TOPS, 4),
                     "traffic": None, "launch_us": round(avg_us["gemm_w8a8"], 2),
                     "alg_ops_per_launch": ops},
        "kernels": kernels,
    }
    if not args.no_cpu:
        out["cpu_baseline"] = _cpu_baseline(cfg, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
