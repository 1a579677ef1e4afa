#!/usr/bin/env python3
"""Benchmark of the SmoothQuant W8A8 linear-layer path on one MI355X.

One step = the whole path once, on one batch of synthetic input already in
HBM: calibration absmax over the calibration tokens, smoothing factors,
smoothed per-output-channel INT8 weights, smoothed per-token INT8
activations, INT8 GEMM with the dequant epilogue to bf16.  The step runs on
the attention-projection workload (M=2048 tokens, K=4096, N=4096, 8192
calibration tokens, alpha=0.5, per-token); inputs rotate over a pool of
independent sets larger than the 256 MB Infinity Cache, so reads come from
HBM.

The JSON line carries, besides the whole-step throughput:
  roofline      the GEMM of the step (its dominant kernel) against the INT8
                MFMA peak, timed with HIP events on the library's stream;
  kernels       every stage of the step (HIP events around each call);
  large         the HBM-bound kernels at the large workload's sizes
                (M=8192, K=12288, N=49152, 262144 calibration tokens), the
                GEMM at the MLP (4096x4096x14336) and large shapes, and the
                decode GEMM's weight-stream rate (16x8192x28672);
  alpha_sweep   relative Frobenius error of the smoothed and unsmoothed W8A8
                output (fp32) against X W (fp64) for the large workload's
                alphas, on a 256-token sample;
  llm_int8_comparator
                the LLM.int8()-style mixed-precision route (outlier channels
                above 6 in bf16, the rest INT8) against SmoothQuant on the
                attention-projection workload: runtime per call, GEMMs alone,
                and fp32 output error against X W (fp64);
  cpu_baseline  the CPU oracle as it stands, on the host cores, over the same
                step workload (the GEMM on a row sample when needed).

    python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--no-cpu] [--no-large]
"""
from __future__ import annotations

import argparse
import hashlib
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
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemm_w8a8_attn_proj_2048x4096x4096_traffic.json")
GEMM_SOURCES = [os.path.join(ROOT, "post_quantization_act_amd", "csrc", f) for f in ("sq_gemm.hip", "sq_device.h")]


def _parse():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--config", default="attn_proj_2048x4096x4096_bf16",
                   help="workload of the step, by name (the attention projection by default)")
    p.add_argument("--pool-gb", type=float, default=1.0, help="rotate inputs over at least this many GB")
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baseline")
    p.add_argument("--no-large", action="store_true", help="skip the large-shape kernel table and alpha sweep")
    p.add_argument("--cpu-seconds", type=float, default=15.0, help="target CPU time of the oracle sample")
    p.add_argument("--launch", choices=("graph", "eager"), default="eager",
                   help="graph: each pass replays a HIP graph of the five calls (one per input set); "
                        "eager: the five calls are launched one by one")
    p.add_argument("--copy-probe-mb", type=int, default=0,
                   help="after timing, run one device copy of this size (for counter calibration)")
    return p.parse_args()


def gemm_source_hash() -> str:
    h = hashlib.sha256()
    for f in GEMM_SOURCES:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def _traffic():
    """HBM bytes per GEMM launch from the committed counter summary, or None
    when it is missing or was taken on a different GEMM source."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("gemm_source_sha256_16") != gemm_source_hash():
        return None
    return t.get("bytes_per_launch")


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _cpu_baseline(cfg, target_s: float):
    """The oracle (as it stands) on the host cores over the step workload,
    scaled to whole-step TOPS; the GEMM runs on a row sample if the full one
    would exceed the time budget."""
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
                   f"tokens); the GEMM + dequant timed on {rows} of {M} token rows and scaled by {M / rows:.2f}; "
                   f"GEMM on {cores} threads, other steps single-threaded"),
        "seconds_per_step": total, "stage_seconds": {k: round(v, 4) for k, v in t.items()},
        "cpu_model": _cpu_model(),
    }


class _Timer:
    """Average duration of a call, from HIP events on the current stream."""

    def __init__(self, torch):
        self.torch = torch

    def __call__(self, fn, reps=5, warm=1):
        torch = self.torch
        for i in range(warm):
            fn(i)
        torch.cuda.synchronize()
        s = torch.cuda.current_stream()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for i, (a, b) in enumerate(evs):
            a.record(s)
            fn(warm + i)
            b.record(s)
        torch.cuda.synchronize()
        return sum(a.elapsed_time(b) for a, b in evs) / reps * 1e3  # us


def _large(torch, sq, synth, pipeline, dev):
    """HBM-bound kernels at the large workload's sizes, GEMMs at the MLP and
    large shapes, the decode weight stream, and the alpha sweep."""
    tm = _Timer(torch)
    out = {}
    cfg = synth.CONFIGS[synth.LARGE]
    M, K, N, T = cfg.M, cfg.K, cfg.N, cfg.calib_tokens
    print(f"# large: drawing {cfg.name} ({T} calibration tokens)", file=sys.stderr, flush=True)
    inp = synth.make(cfg, device=dev)
    b = pipeline.W8A8Buffers.allocate(M, N, K, sq.SQ_PER_TOKEN, dev)
    torch.cuda.synchronize()

    def rate(us, byts):
        gbs = byts / (us * 1e-6) / 1e9
        return {"us": round(us, 1), "alg_bytes": int(byts), "GB_s": round(gbs, 1),
                "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 1)}

    def calib(i):
        b.amax_x.zero_()
        sq.sq_calib_absmax(inp.calib, b.amax_x)

    us_zero = tm(lambda i: b.amax_x.zero_(), reps=5)
    us = tm(calib, reps=3) - us_zero
    out["calib_absmax"] = rate(us, 2 * T * K + 8 * K)
    out["smooth_factors"] = rate(tm(lambda i: sq.sq_smooth_factors(b.amax_x, inp.w, 0.5, b.s, b.inv_s, b.amax_w),
                                    reps=3), 2 * K * N + 12 * K)
    out["quant_weight_call"] = rate(tm(lambda i: sq.sq_quant_weight(inp.w, b.s, b.wq, b.w_scale, b.ws_w), reps=3),
                                    3 * K * N + 4 * N + 4 * K)
    out["quant_weight_call"]["note"] = ("algorithmic 3 B/element; the call moves 5 (column-max pass reads W, the "
                                        "coding pass reads W and writes the codes)")
    out["prepare_weights_call"] = rate(tm(lambda i: sq.sq_prepare_weights(b.amax_x, inp.w, 0.5, b.s, b.inv_s,
                                                                          b.amax_w, b.wq, b.w_scale, b.ws_p),
                                          reps=3), 5 * K * N + 4 * N + 16 * K)
    out["prepare_weights_call"]["note"] = ("steps 2 + 3 in one call: algorithmic 2 + 3 B/element (row maxima; "
                                           "codes), realised as one read of W for the row and column maxima and "
                                           "one read + write for the codes")
    out["quant_act"] = rate(tm(lambda i: sq.sq_quant_act(inp.x, b.inv_s, sq.SQ_PER_TOKEN, b.xq, b.x_scale), reps=5),
                            3 * M * K + 4 * M + 4 * K)
    # per-tensor activation scales: dynamic (a max pass, then codes) and static (calibrated max, one pass)
    xs1 = torch.empty(1, dtype=torch.float32, device=dev)
    ws_t = torch.empty(sq.sq_workspace_size(sq.SQ_OP_QUANT_ACT, M, N, K, sq.SQ_PER_TENSOR), dtype=torch.uint8,
                       device=dev)
    a_st = torch.empty(1, dtype=torch.float32, device=dev)
    sq.sq_static_act_max(b.amax_x, b.inv_s, a_st)
    out["quant_act_per_tensor_dynamic"] = rate(tm(lambda i: sq.sq_quant_act(inp.x, b.inv_s, sq.SQ_PER_TENSOR, b.xq,
                                                                            xs1, ws_t), reps=5),
                                               3 * M * K + 4 * K)
    out["quant_act_per_tensor_static"] = rate(tm(lambda i: sq.sq_quant_act_static(inp.x, b.inv_s, a_st, b.xq, xs1),
                                                 reps=5), 3 * M * K + 4 * K)
    # LayerNorm fold: the runtime LayerNorm + per-token codes with 1/s folded into gamma and beta
    gam = torch.ones(K, dtype=torch.float32, device=dev)
    bet = torch.zeros(K, dtype=torch.float32, device=dev)
    sq.sq_fold_layernorm(gam, bet, b.inv_s, gam, bet)
    out["layernorm_quant"] = rate(tm(lambda i: sq.sq_layernorm_quant(inp.x, gam, bet, 1e-5, b.xq, b.x_scale),
                                     reps=5), 3 * M * K + 4 * M + 8 * K)
    us = tm(lambda i: sq.sq_gemm_w8a8(b.xq, b.x_scale, sq.SQ_PER_TOKEN, b.wq, b.w_scale, b.y), reps=3)
    ops = 2.0 * M * N * K
    out["gemm_8192x12288x49152"] = {"us": round(us, 1), "TOPS": round(ops / us / 1e6, 1),
                                    "pct_int8_peak": round(100 * ops / us / 1e6 / INT8_PEAK_TOPS, 1),
                                    "kernel": sq.sq_gemm_kernel_name(M, N, K)}

    # alpha sweep on a 256-token sample, fp32 output, error against fp64 X W
    rows = torch.arange(0, M, M // 256, device=dev)[:256]
    xs_ = inp.x[rows].contiguous()
    y_ref = xs_.double() @ inp.w.double()
    ref_norm = float(torch.linalg.norm(y_ref))
    bs = pipeline.W8A8Buffers.allocate(256, N, K, sq.SQ_PER_TOKEN, dev, y_dtype=torch.float32)
    bs.amax_x.copy_(b.amax_x)
    sweep = {}
    for a in cfg.alphas:
        sq.sq_smooth_factors(bs.amax_x, None, a, bs.s, bs.inv_s, b.amax_w)
        sq.sq_quant_weight(inp.w, bs.s, bs.wq, bs.w_scale, bs.ws_w)
        pipeline.forward(xs_, sq.SQ_PER_TOKEN, bs, smoothed=True)
        err = float(torch.linalg.norm(bs.y.double() - y_ref)) / ref_norm
        sweep[str(a)] = round(err, 6)
    sq.sq_quant_weight(inp.w, None, bs.wq, bs.w_scale, bs.ws_w)
    pipeline.forward(xs_, sq.SQ_PER_TOKEN, bs, smoothed=False)
    base_tok = float(torch.linalg.norm(bs.y.double() - y_ref)) / ref_norm
    bt = pipeline.W8A8Buffers.allocate(256, N, K, sq.SQ_PER_TENSOR, dev, y_dtype=torch.float32)
    sq.sq_quant_weight(inp.w, None, bt.wq, bt.w_scale, bt.ws_w)
    pipeline.forward(xs_, sq.SQ_PER_TENSOR, bt, smoothed=False)
    base_ten = float(torch.linalg.norm(bt.y.double() - y_ref)) / ref_norm
    grid = [round(0.05 * i, 2) for i in range(21)]
    t0 = time.perf_counter()
    best, errs = pipeline.search_alpha(xs_, inp.w, b.amax_x, grid)
    torch.cuda.synchronize()
    search = {"grid": "0.00 .. 1.00 step 0.05", "best_alpha": best, "best_error": round(errs[best], 6),
              "seconds": round(time.perf_counter() - t0, 3),
              "errors": {f"{a:.2f}": round(e, 6) for a, e in errs.items()}}
    out_sweep = {"workload": cfg.name, "sample_tokens": 256, "output": "fp32", "reference": "X W in fp64",
                 "search": search,
                 "metric": "relative Frobenius error", "smoothed_per_token": sweep,
                 "unsmoothed_per_token": round(base_tok, 6), "unsmoothed_per_tensor": round(base_ten, 6)}
    del inp, b, bs, bt, y_ref
    torch.cuda.empty_cache()

    # MLP shape GEMM (operands rotate over 3 sets: 3 x 75 MB)
    M3, K3, N3 = 4096, 4096, 14336
    g = torch.Generator(device=dev)
    g.manual_seed(3)
    xq3 = [torch.randint(-127, 128, (M3, K3), dtype=torch.int8, device=dev, generator=g) for _ in range(3)]
    wq3 = [torch.randint(-127, 128, (N3, K3), dtype=torch.int8, device=dev, generator=g) for _ in range(3)]
    xs3 = torch.rand(M3, device=dev, generator=g) * 0.01
    ws3 = torch.rand(N3, device=dev, generator=g) * 0.01
    y3 = torch.empty(M3, N3, dtype=torch.bfloat16, device=dev)
    us = tm(lambda i: sq.sq_gemm_w8a8(xq3[i % 3], xs3, sq.SQ_PER_TOKEN, wq3[i % 3], ws3, y3), reps=6)
    ops = 2.0 * M3 * N3 * K3
    out["gemm_4096x4096x14336"] = {"us": round(us, 1), "TOPS": round(ops / us / 1e6, 1),
                                   "pct_int8_peak": round(100 * ops / us / 1e6 / INT8_PEAK_TOPS, 1),
                                   "kernel": sq.sq_gemm_kernel_name(M3, N3, K3)}
    del xq3, wq3, y3
    # decode GEMM: the weight stream (235 MB) rotates over 2 copies (> MALL)
    M4, K4, N4 = 16, 8192, 28672
    xq4 = torch.randint(-127, 128, (M4, K4), dtype=torch.int8, device=dev, generator=g)
    wq4 = [torch.randint(-127, 128, (N4, K4), dtype=torch.int8, device=dev, generator=g) for _ in range(2)]
    xs4 = torch.rand(M4, device=dev, generator=g) * 0.01
    ws4 = torch.rand(N4, device=dev, generator=g) * 0.01
    y4 = torch.empty(M4, N4, dtype=torch.bfloat16, device=dev)
    us = tm(lambda i: sq.sq_gemm_w8a8(xq4, xs4, sq.SQ_PER_TOKEN, wq4[i % 2], ws4, y4), reps=10)
    out["gemm_decode_16x8192x28672"] = rate(us, N4 * K4 + M4 * K4 + 2 * M4 * N4 + 4 * (M4 + N4))
    out["gemm_decode_16x8192x28672"]["note"] = "weight-stream bound: 235 MB of int8 weights per launch"
    out["gemm_decode_16x8192x28672"]["kernel"] = sq.sq_gemm_kernel_name(M4, N4, K4)
    del xq4, wq4, y4
    torch.cuda.empty_cache()
    return out, out_sweep


def _comparator(torch, sq, synth, pipeline, dev):
    """SmoothQuant against the LLM.int8()-style mixed-precision route on the
    attention-projection workload (2048 x 4096 x 4096, 41 outlier channels):
    runtime time of each per call (inputs rotating over sets larger than the
    Infinity Cache), the two GEMMs alone, and the output error of each against
    X W in fp64 on a 256-token sample."""
    tm = _Timer(torch)
    cfg = synth.CONFIGS[synth.ATTN_PROJ]
    M, K, N = cfg.M, cfg.K, cfg.N
    nsets = 6  # 6 x (16.8 MB x + 33.5 MB w + 16.8 MB codes) > 256 MB
    print(f"# comparator: drawing {nsets} sets of {cfg.name}", file=sys.stderr, flush=True)
    sets = [synth.make(cfg, device=dev, variant=v) for v in range(nsets)]
    sqb = [pipeline.W8A8Buffers.allocate(M, N, K, sq.SQ_PER_TOKEN, dev) for _ in range(nsets)]
    lb = [pipeline.LlmInt8Buffers.allocate(M, N, K, dev) for _ in range(nsets)]
    for inp, b, l in zip(sets, sqb, lb):
        pipeline.calibrate(inp.calib, b.amax_x)
        pipeline.prepare_weights(inp.w, 0.5, b)
        pipeline.llm_int8_prepare(inp.w, l)
        pipeline.llm_int8_forward(inp.x, inp.w, 6.0, l)
    torch.cuda.synchronize()
    n_out = [int(l.count.item()) for l in lb]

    def sq_run(i):
        k = i % nsets
        pipeline.forward(sets[k].x, sq.SQ_PER_TOKEN, sqb[k], smoothed=True)

    def l8_run(i):
        k = i % nsets
        pipeline.llm_int8_forward(sets[k].x, sets[k].w, 6.0, lb[k])

    def sq_gemm(i):
        b = sqb[i % nsets]
        sq.sq_gemm_w8a8(b.xq, b.x_scale, sq.SQ_PER_TOKEN, b.wq, b.w_scale, b.y)

    def l8_gemm(i):
        l = lb[i % nsets]
        sq.sq_gemm_w8a8_outlier(l.xq, l.x_scale, l.wq, l.w_scale, l.x_o, l.w_ot, l.count, l.y)

    reps = 4 * nsets
    t_sq, t_l8 = tm(sq_run, reps=reps, warm=nsets), tm(l8_run, reps=reps, warm=nsets)
    g_sq, g_l8 = tm(sq_gemm, reps=reps, warm=nsets), tm(l8_gemm, reps=reps, warm=nsets)
    ops = 2.0 * M * N * K

    # errors of the fp32 outputs on set 0 against X W in fp64 (256 sampled tokens)
    inp = sets[0]
    rows = torch.arange(0, M, M // 256, device=dev)[:256]
    y_ref = inp.x[rows].double() @ inp.w.double()
    nrm = float(torch.linalg.norm(y_ref))

    def err(y):
        return round(float(torch.linalg.norm(y[rows].double() - y_ref)) / nrm, 6)

    b32 = pipeline.W8A8Buffers.allocate(M, N, K, sq.SQ_PER_TOKEN, dev, y_dtype=torch.float32)
    b32.amax_x.copy_(sqb[0].amax_x)
    pipeline.prepare_weights(inp.w, 0.5, b32)
    pipeline.forward(inp.x, sq.SQ_PER_TOKEN, b32, smoothed=True)
    e_sq = err(b32.y)
    pipeline.prepare_weights(inp.w, None, b32)
    pipeline.forward(inp.x, sq.SQ_PER_TOKEN, b32, smoothed=False)
    e_plain = err(b32.y)
    l32 = pipeline.LlmInt8Buffers.allocate(M, N, K, dev, y_dtype=torch.float32)
    pipeline.llm_int8_prepare(inp.w, l32)
    pipeline.llm_int8_forward(inp.x, inp.w, 6.0, l32)
    e_l8 = err(l32.y)
    torch.cuda.synchronize()
    out = {
        "workload": cfg.name, "threshold": 6.0, "outlier_channels": n_out[0],
        "outlier_channels_all_sets": n_out,
        "smoothquant_runtime_us": round(t_sq, 1),
        "llm_int8_runtime_us": round(t_l8, 1),
        "runtime_ratio_llm_int8_over_smoothquant": round(t_l8 / t_sq, 3),
        "smoothquant_gemm_us": round(g_sq, 1),
        "llm_int8_gemm_us": round(g_l8, 1),
        "smoothquant_gemm_pct_int8_peak": round(100 * ops / g_sq / 1e6 / INT8_PEAK_TOPS, 1),
        "llm_int8_gemm_kernel": sq.sq_gemm_outlier_kernel_name(M, N, K),
        "error_rel_fro_fp32": {"smoothquant_alpha_0.5_per_token": e_sq, "llm_int8": e_l8,
                               "unsmoothed_per_token": e_plain},
        "runtime_steps": {"smoothquant": "quant_act (smoothing fused) + gemm_w8a8",
                          "llm_int8": "absmax of x + outlier_columns + quant_act (keep mask) + gather_outliers "
                                      "+ gemm_w8a8_outlier"},
    }
    del sets, sqb, lb, b32, l32, y_ref
    torch.cuda.empty_cache()
    return out


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

    stages = ["calib_absmax", "prepare_and_quant_act", "gemm_w8a8"]

    def step(i, ev=None):
        s = sets[i % pool]
        if ev is not None:
            ev[0].record(stream)
        pipeline.calibrate(s.calib, b.amax_x)
        if ev is not None:
            ev[1].record(stream)
        sq.sq_prepare_and_quant_act(b.amax_x, s.w, alpha, b.s, b.inv_s, b.amax_w, b.wq, b.w_scale, s.x, gran, b.xq,
                                    b.x_scale, b.ws_pa)
        if ev is not None:
            ev[2].record(stream)
        sq.sq_gemm_w8a8(b.xq, b.x_scale, gran, b.wq, b.w_scale, b.y)
        if ev is not None:
            ev[3].record(stream)

    if args.launch == "graph":
        graphs = [pipeline.CapturedPass(st.x, st.w, st.calib, alpha, gran, b) for st in sets]
        torch.cuda.synchronize()

        def run(i):
            graphs[i % pool].replay()
    else:
        def run(i):
            step(i)

    for i in range(args.warmup):
        run(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        run(args.warmup + i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps
    print(f"# timed {args.steps} steps ({args.launch}): {ms_per_step:.4f} ms/step", file=sys.stderr, flush=True)

    # per-call breakdown: separate eager passes with HIP events between the calls
    # (not part of the timed region above)
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(len(stages) + 1)] for _ in range(args.steps)]
    for i in range(args.steps):
        step(i, events[i])
    torch.cuda.synchronize()
    per = {name: [] for name in stages}
    for ev in events:
        for k, name in enumerate(stages):
            per[name].append(ev[k].elapsed_time(ev[k + 1]) * 1e3)  # us
    avg_us = {name: sum(v) / len(v) for name, v in per.items()}

    ops = 2.0 * M * N * K
    bytes_alg = {
        "calib_absmax": T * K * esz + 8 * K,
        "prepare_and_quant_act": (2 * K * N * esz + N * K + 4 * N + 16 * K) + (M * K * esz + M * K + 4 * M + 4 * K),
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
    kernels["note"] = ("HIP-event intervals per call from separate eager passes (not the timed ones): calib_absmax "
                       "includes zeroing the running max; prepare_and_quant_act is steps 2-4 (one read of W for row "
                       "and column maxima, a reduction of per-block maxima, then the weight codes and the activation "
                       "codes in one launch); algorithmic bytes are those of steps 2 + 3 (2 B per W element read, "
                       "1 written) plus step 4 (2 B per X element read, 1 written)")

    if args.copy_probe_mb > 0:
        # a plain copy of known size whose source is not cache resident: 1 GiB
        # is written between filling the source and copying it
        nb = args.copy_probe_mb << 20
        src = torch.empty(nb, dtype=torch.uint8, device=dev)
        dst = torch.empty(nb, dtype=torch.uint8, device=dev)
        flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        src.fill_(1)
        flush.fill_(2)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst, flush

    value = ops / (ms_per_step * 1e-3) / 1e12
    traffic = _traffic()
    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "TOPS", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "int8", "data": "synthetic",
        "config": {"workload": cfg.name, "M": M, "K": K, "N": N, "calib_tokens": T, "alpha": alpha,
                   "act_granularity": cfg.gran, "weight_granularity": "per_output_channel",
                   "input_dtype": cfg.x_dtype, "output_dtype": "bf16", "input_pool_sets": pool,
                   "value_definition": "2*M*N*K of the GEMM / wall time of one whole five-step pass",
                   "launch": args.launch},
        "roofline": {"bound": "mfma", "kernel": sq.sq_gemm_kernel_name(M, N, K), "achieved": round(gemm_tops, 1),
                     "peak": INT8_PEAK_TOPS, "unit": "TOPS", "frac": round(gemm_tops / INT8_PEAK_TOPS, 4),
                     "traffic": traffic, "launch_us": round(avg_us["gemm_w8a8"], 2), "alg_ops_per_launch": ops,
                     "gemm_source_sha256_16": gemm_source_hash()},
        "kernels": kernels,
    }
    if not args.no_large:
        del sets
        torch.cuda.empty_cache()
        out["large"], out["alpha_sweep"] = _large(torch, sq, synth, pipeline, dev)
        out["llm_int8_comparator"] = _comparator(torch, sq, synth, pipeline, dev)
    if not args.no_cpu:
        print("# CPU oracle baseline", file=sys.stderr, flush=True)
        out["cpu_baseline"] = _cpu_baseline(cfg, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
