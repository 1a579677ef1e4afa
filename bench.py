#!/usr/bin/env python3
"""Benchmark of the SmoothQuant W8A8 linear-layer path on one MI355X.

One step = the whole path once over one batch of synthetic input already in
HBM, on the large workload (M = 8192 tokens, K = 12288, N = 49152, Student-t
body with 61 outlier channels x200, 512 x 512 calibration tokens) with its
alpha sweep: the calibration absmax over the 262144 calibration tokens
(6.44 GB), then for each alpha in (0.4, 0.5, 0.6, 0.75) the smoothing factors,
the smoothed per-output-channel INT8 weights, the smoothed per-token INT8
activations (sq_prepare_and_quant_act, steps 2-4) and the INT8 GEMM with the
dequant epilogue to bf16 (sq_gemm_w8a8).  The runtime batch rotates over a
pool of 5 independent x (1 GB); the calibration set and W are each larger
than the 256 MB Infinity Cache.

value = 4 GEMMs x 2 M N K / wall time of one step (the whole five-step pass,
calibration and weight preparation included) in TOPS.  The GEMM alone is the
roofline object: its launches inside the timed steps are bracketed by HIP
events on the library's stream.

Besides the headline line, the JSON carries:
  kernels       the step's calls, averaged over the timed steps;
  workloads     every kernel of the per-workload set as a median of >= 50 HIP-event
                timed calls over input pools of >= 1 GB (or single inputs
                larger than that): calibration absmax, weight row max +
                factors, weight codes, activation codes (per token, per
                tensor dynamic and static, LayerNorm + codes) and the GEMM on
                the large workload; the weight calls and activation codes on
                the MLP-up (4096x4096x14336) and decode (16x8192x28672)
                workloads; the GEMMs on the attention-projection
                (2048x4096x4096) and MLP-up shapes; the decode weight stream
                alone and with its activation codes;
  attn_proj_step  the five-step pass on the attention-projection workload;
  alpha_sweep   relative Frobenius error of the smoothed and unsmoothed W8A8
                output (fp32) against X W (fp64) per alpha on a 256-token sample;
  llm_int8_comparator   the LLM.int8()-style mixed-precision route against
                SmoothQuant on the attention-projection workload;
  hbm_probe     torch's bf16 -> int8 conversion, bf16 copy and bf16 max on
                1 GB pools: what generic kernels reach on this GPU for the
                quantizers' read + write pattern and for a read stream;
  cpu_baseline  the CPU oracle as it stands, on the host cores, over bounded
                samples of the step's stages, scaled to the whole step;
  tile_sweep    (only when asked for) the 256 x 256 GEMM at 4096 tokens over
                2-6 tiles per CU and K = 2048-8192, with the time of one tile
                and the launch's fixed part fitted per K.

    python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--no-cpu]
                    [--sections step,workloads,attn_proj,alpha,comparator,probe[,tile_sweep]]
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import ctypes
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0      # MI355X HBM3E, GB/s
INT8_PEAK_TOPS = 5000.0    # MI355X dense INT8 MFMA, TOPS (5.0 POP/s)
METRIC = "W8A8 GEMM TOPS (% INT8 MFMA peak); quant-kernel HBM GB/s (% peak)"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemm_w8a8_large_8192x12288x49152_traffic.json")
MFMA_FILE = os.path.join(ROOT, "profiles", "gemm_mfma_large_8192x12288x49152.json")
GEMM_SOURCES = [os.path.join(ROOT, "post_quantization_act_amd", "csrc", f) for f in ("sq_gemm.hip", "sq_device.h")]
SECTIONS = ("step", "workloads", "attn_proj", "alpha", "comparator", "probe")
EXTRA_SECTIONS = ("tile_sweep",)  # run only when asked for
RUNS = 50          # HIP-event timed calls per workload row (median reported)
POOL_BYTES = 1e9   # rotate inputs over at least this many bytes
CPU_THREADS_MAX = 16


def _parse():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baseline")
    p.add_argument("--sections", default=",".join(SECTIONS),
                   help="comma list of parts to run besides the headline step (default " + ",".join(SECTIONS) +
                        "; also " + ",".join(EXTRA_SECTIONS) + ")")
    p.add_argument("--runs", type=int, default=RUNS, help="timed calls per workload row")
    p.add_argument("--cpu-seconds", type=float, default=20.0, help="target CPU time of the oracle samples")
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


def _mfma_counters():
    """Sustained shader clock and matrix-core busy share of the large GEMM from
    the committed counter summary, or None when it is missing or was taken on
    a different GEMM source."""
    try:
        with open(MFMA_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("gemm_source_sha256_16") != gemm_source_hash():
        return None
    return {"shader_clock_ghz": t.get("shader_clock_ghz"), "mfma_busy_pct": t.get("mfma_busy_pct"),
            "source": "profiles/gemm_mfma_large_8192x12288x49152.json (rocprofv3 --pmc, under the profiler)"}


def _cpu_model():
    """The host's model name with its family / model / stepping numbers (some
    hosts report only a short name) and the count of online logical CPUs."""
    fields = {}
    try:
        for line in open("/proc/cpuinfo"):
            if ":" in line:
                k, v = (p.strip() for p in line.split(":", 1))
                if k in ("model name", "cpu family", "model", "stepping") and k not in fields:
                    fields[k] = v
            elif fields:
                break
    except OSError:
        return "unknown"
    name = fields.get("model name", "unknown")
    ids = ", ".join(f"{k} {fields[k]}" for k in ("cpu family", "model", "stepping") if k in fields)
    return f"{name} ({ids}; {os.cpu_count()} logical CPUs online)" if ids else name


def _say(msg):
    print(f"# {msg}", file=sys.stderr, flush=True)


def _rate(us, alg_bytes, **extra):
    gbs = alg_bytes / (us * 1e-6) / 1e9
    r = {"us": round(us, 2), "alg_bytes": int(alg_bytes), "GB_s": round(gbs, 1),
         "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 1)}
    r.update(extra)
    return r


def _tops(us, ops, **extra):
    t = ops / (us * 1e-6) / 1e12
    r = {"us": round(us, 2), "ops": ops, "TOPS": round(t, 1), "pct_int8_peak": round(100 * t / INT8_PEAK_TOPS, 1)}
    r.update(extra)
    return r


class _Timer:
    """Per-call durations from HIP events recorded on the current stream (the
    stream the library launches on); returns the median in microseconds.

    The timed calls are enqueued behind a spin kernel of about 20 ms, so the
    host has queued them all before the GPU reaches them: each event interval
    is then the call's device time (its kernels and the gaps between them),
    not the host's launch overhead, which exceeds the device time of the short
    calls."""

    SPIN_CYCLES = 40_000_000

    def __init__(self, torch, runs):
        self.torch = torch
        self.runs = runs

    def __call__(self, fn, warm=5, runs=None):
        torch = self.torch
        runs = self.runs if runs is None else runs
        for i in range(warm):
            fn(i)
        torch.cuda.synchronize()
        s = torch.cuda.current_stream()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(runs)]
        torch.cuda._sleep(self.SPIN_CYCLES)
        for i, (a, b) in enumerate(evs):
            a.record(s)
            fn(warm + i)
            b.record(s)
        torch.cuda.synchronize()
        return statistics.median(a.elapsed_time(b) * 1e3 for a, b in evs)


def _pool(t, min_bytes=POOL_BYTES):
    """Independent copies of tensor t (distinct addresses) totalling at least
    min_bytes, so that calls cycling through them read HBM, not cache."""
    n = max(1, int(-(-min_bytes // (t.numel() * t.element_size()))))
    return [t] + [t.clone() for _ in range(n - 1)]


# ---- headline step -------------------------------------------------------------------

def _step(torch, sq, synth, pipeline, dev, args):
    cfg = synth.CONFIGS[synth.LARGE]
    M, K, N, T = cfg.M, cfg.K, cfg.N, cfg.calib_tokens
    alphas = cfg.alphas
    _say(f"workload {cfg.name}: M={M} K={K} N={N} T={T} alphas={alphas}")
    inp = synth.make(cfg, device=dev)
    nx = max(1, int(-(-POOL_BYTES // (M * K * 2))))
    xs = [inp.x] + [synth.make_x(cfg, device=dev, variant=v) for v in range(1, nx)]
    b = pipeline.W8A8Buffers.allocate(M, N, K, sq.SQ_PER_TOKEN, dev)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    na = len(alphas)
    n_ev = 2 + 2 * na

    def step(i, ev=None):
        x = xs[i % nx]
        if ev is not None:
            ev[0].record(stream)
        pipeline.calibrate(inp.calib, b.amax_x)
        if ev is not None:
            ev[1].record(stream)
        for k, a in enumerate(alphas):
            sq.sq_prepare_and_quant_act(b.amax_x, inp.w, a, b.s, b.inv_s, b.amax_w, b.wq, b.w_scale, x,
                                        sq.SQ_PER_TOKEN, b.xq, b.x_scale, b.ws_pa)
            if ev is not None:
                ev[2 + 2 * k].record(stream)
            sq.sq_gemm_w8a8(b.xq, b.x_scale, sq.SQ_PER_TOKEN, b.wq, b.w_scale, b.y)
            if ev is not None:
                ev[3 + 2 * k].record(stream)

    events = [[torch.cuda.Event(enable_timing=True) for _ in range(n_ev)] for _ in range(args.steps)]
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(args.warmup + i, events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps
    _say(f"timed {args.steps} steps: {ms_per_step:.3f} ms/step")

    def iv(ev, a, c):
        return ev[a].elapsed_time(ev[c]) * 1e3  # us

    calib_us = [iv(ev, 0, 1) for ev in events]
    prep_us = {a: [iv(ev, 1 + 2 * k, 2 + 2 * k) for ev in events] for k, a in enumerate(alphas)}
    gemm_us = {a: [iv(ev, 2 + 2 * k, 3 + 2 * k) for ev in events] for k, a in enumerate(alphas)}
    ops = 2.0 * M * N * K
    all_gemm = [u for a in alphas for u in gemm_us[a]]
    gemm_avg = sum(all_gemm) / len(all_gemm)
    gemm_tops = ops / (gemm_avg * 1e-6) / 1e12
    kernels = {
        "calib_absmax": _rate(sum(calib_us) / len(calib_us), 2 * T * K + 8 * K,
                              note="sq_calib_reset + sq_calib_absmax over the 262144 x 12288 calibration set"),
        "prepare_and_quant_act": {
            f"{a}": _rate(sum(prep_us[a]) / len(prep_us[a]), 2 * K * N + (2 * K * N + N * K) + 3 * M * K + 4 * (M + N),
                          note="steps 2-4 (sq_prepare_and_quant_act): W read for the row maxima, W read and codes "
                               "written, x read and codes written (algorithmic 2 + 3 B per W element, 3 B per x "
                               "element)") for a in alphas},
        "gemm_w8a8": {f"{a}": _tops(sum(gemm_us[a]) / len(gemm_us[a]), ops,
                                    median_us=round(statistics.median(gemm_us[a]), 2)) for a in alphas},
        "note": "HIP-event intervals recorded on the library's stream inside the timed steps (averages over the "
                "timed steps)",
    }
    if args.copy_probe_mb > 0:
        # a plain copy of known size whose source is not cache resident (1 GiB is
        # written in between), to scale the traffic counters
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

    n_alpha_ops = na * ops
    head = {
        "metric": METRIC, "value": round(n_alpha_ops / (ms_per_step * 1e-3) / 1e12, 2), "unit": "TOPS",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "int8", "data": "synthetic",
        "config": {"workload": cfg.name, "M": M, "K": K, "N": N, "calib_tokens": T, "alphas": list(alphas),
                   "x_body": "Student-t nu=4", "outlier_channels": cfg.n_out, "outlier_factor": cfg.out_hi,
                   "act_granularity": "per_token", "weight_granularity": "per_output_channel",
                   "input_dtype": "bf16", "output_dtype": "bf16", "x_pool": nx,
                   "value_definition": (f"{na} x 2*M*N*K (one GEMM per alpha) / wall time of one whole step: "
                                        "calibration absmax over the 262144 calibration tokens, then per alpha "
                                        "steps 2-4 and the GEMM; whole-path throughput, not the GEMM alone "
                                        "(the GEMM alone is roofline.achieved)")},
        "roofline": {"bound": "mfma", "kernel": sq.sq_gemm_kernel_name(M, N, K), "achieved": round(gemm_tops, 1),
                     "peak": INT8_PEAK_TOPS, "unit": "TOPS", "frac": round(gemm_tops / INT8_PEAK_TOPS, 4),
                     "traffic": _traffic(), "counters": _mfma_counters(), "launch_us": round(gemm_avg, 2),
                     "alg_ops_per_launch": ops,
                     "launches_timed": len(all_gemm), "gemm_source_sha256_16": gemm_source_hash()},
        "kernels": kernels,
    }
    state = dict(cfg=cfg, inp=inp, xs=xs, b=b)
    return head, state


def _vendor_gemm(torch, tm, operands, ops):
    """The same INT8 product through the vendor BLAS for comparison: torch._int_mm
    (hipBLASLt on ROCm) on the same codes, Xq [M, K] times a column-major view
    of Wq^T, int32 output (no dequantization epilogue, so it writes twice the
    bytes of the library's bf16 y)."""
    n = len(operands)
    try:
        t = tm(lambda i: torch._int_mm(operands[i % n][0], operands[i % n][1].t()))
    except RuntimeError as e:  # an unsupported shape or build: recorded, not fatal
        return {"error": str(e)[:200]}
    return _tops(t, ops, kernel="torch._int_mm (hipBLASLt)", note="comparison only: int32 output, same codes")


def _tile_sweep(torch, sq, dev, tm):
    """Where the 256 x 256 GEMM's time goes: 4096 tokens, 2 to 6 tiles per CU
    (N = 8192 .. 24576) and 16 to 64 stages of 128 k-bytes per tile (K = 2048
    .. 8192), operands rotated over >= 1 GB; per K, a least-squares line
    through the medians over the tiles per CU.  The codes are
    clamp(round(N(0, 28^2)), -127, 127), shaped like real ones."""
    import numpy as np
    M = 4096
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    g = torch.Generator(device=dev)
    g.manual_seed(4096)

    def codes(r, c):
        return torch.clamp(torch.round(torch.randn(r, c, device=dev, generator=g) * 28.0), -127, 127).to(torch.int8)

    rows, per_k = [], {}
    for K in (2048, 4096, 8192):
        tiles_l, times = [], []
        for N in (8192, 12288, 16384, 24576):
            n = max(1, int(-(-POOL_BYTES // (M * K + N * K))))
            ops = [(codes(M, K), codes(N, K)) for _ in range(n)]
            xs = torch.rand(M, device=dev, generator=g) * 1e-3
            ws = torch.rand(N, device=dev, generator=g) * 1e-3
            y = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
            us = tm(lambda i: sq.sq_gemm_w8a8(ops[i % n][0], xs, sq.SQ_PER_TOKEN, ops[i % n][1], ws, y))
            tiles = M * N / (256 * 256) / cus
            rows.append({"M": M, "N": N, "K": K, "tiles_per_cu": tiles, "stages_per_tile": K // 128,
                         **_tops(us, 2.0 * M * N * K), "kernel": sq.sq_gemm_kernel_name(M, N, K)[:30]})
            tiles_l.append(tiles)
            times.append(us)
            del ops, y
            torch.cuda.empty_cache()
        slope, icpt = np.polyfit(tiles_l, times, 1)
        per_k[str(K)] = {"stages_per_tile": K // 128, "us_per_tile": round(float(slope), 2),
                         "intercept_us": round(float(icpt), 2)}
    return {"shapes": rows, "per_k_fit": per_k,
            "note": "median HIP-event times; per K a straight line over tiles per CU: the slope is one tile's "
                    "time (its stages and the change to the next tile), the intercept the launch's fixed part; "
                    "the clock falls as runs get longer, so the per-stage time differs between the K"}


# ---- the per-workload kernel set -----------------------------------------------------------

def _workload_large(torch, sq, pipeline, dev, tm, st):
    cfg, inp, xs, b = st["cfg"], st["inp"], st["xs"], st["b"]
    M, K, N, T = cfg.M, cfg.K, cfg.N, cfg.calib_tokens
    nx = len(xs)
    out = {}
    _say("workloads: large")
    out["calib_absmax"] = _rate(tm(lambda i: (sq.sq_calib_reset(b.amax_x),
                                              sq.sq_calib_absmax(inp.calib, b.amax_x))), 2 * T * K + 8 * K,
                                input_bytes=2 * T * K, note="sq_calib_reset + sq_calib_absmax, 6.44 GB per call")
    out["smooth_factors"] = _rate(tm(lambda i: sq.sq_smooth_factors(b.amax_x, inp.w, 0.5, b.s, b.inv_s, b.amax_w)),
                                  2 * K * N + 12 * K, input_bytes=2 * K * N, note="W row maxima + factors (K2a, K2b)")
    out["quant_weight_call"] = _rate(tm(lambda i: sq.sq_quant_weight(inp.w, b.s, b.wq, b.w_scale, b.ws_w)),
                                     3 * K * N + 4 * N + 4 * K,
                                     note="algorithmic 3 B/element; the call's two passes move 5 (column maxima "
                                          "of diag(s) W, then codes)")
    out["prepare_weights_call"] = _rate(tm(lambda i: sq.sq_prepare_weights(b.amax_x, inp.w, 0.5, b.s, b.inv_s,
                                                                          b.amax_w, b.wq, b.w_scale, b.ws_p)),
                                        5 * K * N + 4 * N + 16 * K,
                                        note="steps 2 + 3: algorithmic 2 + 3 B/element, realised as one read of W "
                                             "for row and column maxima and one read + write for the codes")
    pool = f"{nx} x of {M * K * 2 / 1e6:.0f} MB"
    out["quant_act_per_token"] = _rate(tm(lambda i: sq.sq_quant_act(xs[i % nx], b.inv_s, sq.SQ_PER_TOKEN, b.xq,
                                                                    b.x_scale)), 3 * M * K + 4 * M + 4 * K, pool=pool)
    xs1 = torch.empty(1, dtype=torch.float32, device=dev)
    ws_t = torch.empty(sq.sq_workspace_size(sq.SQ_OP_QUANT_ACT, M, N, K, sq.SQ_PER_TENSOR), dtype=torch.uint8,
                       device=dev)
    a_st = torch.empty(1, dtype=torch.float32, device=dev)
    sq.sq_static_act_max(b.amax_x, b.inv_s, a_st)
    out["quant_act_per_tensor_dynamic"] = _rate(tm(lambda i: sq.sq_quant_act(xs[i % nx], b.inv_s, sq.SQ_PER_TENSOR,
                                                                             b.xq, xs1, ws_t)), 3 * M * K + 4 * K,
                                                pool=pool, note="two passes over x: the tensor maximum, then codes")
    out["quant_act_per_tensor_static"] = _rate(tm(lambda i: sq.sq_quant_act_static(xs[i % nx], b.inv_s, a_st, b.xq,
                                                                                   xs1)), 3 * M * K + 4 * K, pool=pool)
    gam = torch.ones(K, dtype=torch.float32, device=dev)
    bet = torch.zeros(K, dtype=torch.float32, device=dev)
    sq.sq_fold_layernorm(gam, bet, b.inv_s, gam, bet)
    out["layernorm_quant"] = _rate(tm(lambda i: sq.sq_layernorm_quant(xs[i % nx], gam, bet, 1e-5, b.xq, b.x_scale)),
                                   3 * M * K + 4 * M + 8 * K, pool=pool)
    pipeline.prepare_and_quantize(xs[0], inp.w, 0.5, sq.SQ_PER_TOKEN, b)
    out["gemm"] = _tops(tm(lambda i: sq.sq_gemm_w8a8(b.xq, b.x_scale, sq.SQ_PER_TOKEN, b.wq, b.w_scale, b.y)),
                        2.0 * M * N * K, kernel=sq.sq_gemm_kernel_name(M, N, K),
                        note="operands 704 MB per call (Wq 604 MB + Xq 101 MB)")
    out["gemm_vendor"] = _vendor_gemm(torch, tm, [(b.xq, b.wq)], 2.0 * M * N * K)
    torch.cuda.empty_cache()
    return out


def _workload_mlp_up(torch, sq, synth, pipeline, dev, tm):
    cfg = synth.CONFIGS[synth.MLP_UP]
    M, K, N = cfg.M, cfg.K, cfg.N
    _say(f"workloads: {cfg.name}")
    inp = synth.make(cfg, device=dev)
    b = pipeline.W8A8Buffers.allocate(M, N, K, sq.SQ_PER_TOKEN, dev)
    pipeline.calibrate(inp.calib, b.amax_x)
    ws, xp = _pool(inp.w), _pool(inp.x)
    out = {}
    nw, nx = len(ws), len(xp)
    out["smooth_factors"] = _rate(tm(lambda i: sq.sq_smooth_factors(b.amax_x, ws[i % nw], 0.5, b.s, b.inv_s,
                                                                    b.amax_w)), 2 * K * N + 12 * K,
                                  pool=f"{nw} W of {K * N * 2 / 1e6:.0f} MB")
    out["quant_weight_call"] = _rate(tm(lambda i: sq.sq_quant_weight(ws[i % nw], b.s, b.wq, b.w_scale, b.ws_w)),
                                     3 * K * N + 4 * N + 4 * K, pool=f"{nw} W")
    out["prepare_weights_call"] = _rate(tm(lambda i: sq.sq_prepare_weights(b.amax_x, ws[i % nw], 0.5, b.s, b.inv_s,
                                                                          b.amax_w, b.wq, b.w_scale, b.ws_p)),
                                        5 * K * N + 4 * N + 16 * K, pool=f"{nw} W")
    out["quant_act_per_token"] = _rate(tm(lambda i: sq.sq_quant_act(xp[i % nx], b.inv_s, sq.SQ_PER_TOKEN, b.xq,
                                                                    b.x_scale)), 3 * M * K + 4 * M + 4 * K,
                                       pool=f"{nx} x of {M * K * 2 / 1e6:.1f} MB")
    del ws, xp
    # GEMM on the workload's own codes, rotated over > 1 GB of operand copies
    pipeline.prepare_and_quantize(inp.x, inp.w, 0.5, sq.SQ_PER_TOKEN, b)
    ops = [(b.xq, b.wq)] + [(b.xq.clone(), b.wq.clone())
                            for _ in range(int(-(-POOL_BYTES // (M * K + N * K))) - 1)]
    n = len(ops)
    out["gemm"] = _tops(tm(lambda i: sq.sq_gemm_w8a8(ops[i % n][0], b.x_scale, sq.SQ_PER_TOKEN, ops[i % n][1],
                                                     b.w_scale, b.y)), 2.0 * M * N * K,
                        kernel=sq.sq_gemm_kernel_name(M, N, K), pool=f"{n} operand sets of {(M * K + N * K) / 1e6:.0f} MB")
    out["gemm_vendor"] = _vendor_gemm(torch, tm, ops, 2.0 * M * N * K)
    del ops, inp, b
    torch.cuda.empty_cache()
    return out


def _workload_decode(torch, sq, synth, pipeline, dev, tm):
    cfg = synth.CONFIGS[synth.DECODE]
    M, K, N = cfg.M, cfg.K, cfg.N
    _say(f"workloads: {cfg.name}")
    inp = synth.make(cfg, device=dev)
    b = pipeline.W8A8Buffers.allocate(M, N, K, sq.SQ_PER_TOKEN, dev)
    pipeline.calibrate(inp.calib, b.amax_x)
    out = {}
    ws = _pool(inp.w)
    nw = len(ws)
    out["smooth_factors"] = _rate(tm(lambda i: sq.sq_smooth_factors(b.amax_x, ws[i % nw], 0.5, b.s, b.inv_s,
                                                                    b.amax_w)), 2 * K * N + 12 * K,
                                  pool=f"{nw} W of {K * N * 2 / 1e6:.0f} MB")
    out["quant_weight_call"] = _rate(tm(lambda i: sq.sq_quant_weight(ws[i % nw], b.s, b.wq, b.w_scale, b.ws_w)),
                                     3 * K * N + 4 * N + 4 * K, pool=f"{nw} W")
    out["prepare_weights_call"] = _rate(tm(lambda i: sq.sq_prepare_weights(b.amax_x, ws[i % nw], 0.5, b.s, b.inv_s,
                                                                          b.amax_w, b.wq, b.w_scale, b.ws_p)),
                                        5 * K * N + 4 * N + 16 * K, pool=f"{nw} W")
    del ws
    # the runtime: activation codes of the 16 tokens (latency-bound, reported) and the weight stream
    out["quant_act_per_token"] = _rate(tm(lambda i: sq.sq_quant_act(inp.x, b.inv_s, sq.SQ_PER_TOKEN, b.xq,
                                                                    b.x_scale)), 3 * M * K + 4 * M + 4 * K,
                                       note="reported only: 0.39 MB, launch-latency bound")
    wqs = _pool(b.wq)
    n = len(wqs)
    stream_bytes = N * K + M * K + 2 * M * N + 4 * (M + N)
    out["gemm_weight_stream"] = _rate(tm(lambda i: sq.sq_gemm_w8a8(b.xq, b.x_scale, sq.SQ_PER_TOKEN, wqs[i % n],
                                                                   b.w_scale, b.y)), stream_bytes,
                                      kernel=sq.sq_gemm_kernel_name(M, N, K),
                                      pool=f"{n} Wq of {N * K / 1e6:.0f} MB",
                                      note="weight-stream bound: 235 MB of int8 weights per call")

    def both(i):
        sq.sq_quant_act(inp.x, b.inv_s, sq.SQ_PER_TOKEN, b.xq, b.x_scale)
        sq.sq_gemm_w8a8(b.xq, b.x_scale, sq.SQ_PER_TOKEN, wqs[i % n], b.w_scale, b.y)

    out["quant_act_then_gemm"] = _rate(tm(both), stream_bytes + 2 * M * K + 4 * K,
                                       note="steps 4 + 5 of one decode token batch as two calls (sq_quant_act, "
                                            "sq_gemm_w8a8), the weight-stream rate of the pair")
    del wqs, inp, b
    torch.cuda.empty_cache()
    return out


def _workload_attn_gemm(torch, sq, synth, pipeline, dev, tm):
    cfg = synth.CONFIGS[synth.ATTN_PROJ]
    M, K, N = cfg.M, cfg.K, cfg.N
    inp = synth.make(cfg, device=dev)
    b = pipeline.W8A8Buffers.allocate(M, N, K, sq.SQ_PER_TOKEN, dev)
    pipeline.calibrate(inp.calib, b.amax_x)
    pipeline.prepare_and_quantize(inp.x, inp.w, 0.5, sq.SQ_PER_TOKEN, b)
    ops = [(b.xq, b.wq)] + [(b.xq.clone(), b.wq.clone())
                            for _ in range(int(-(-POOL_BYTES // (M * K + N * K))) - 1)]
    n = len(ops)
    r = _tops(tm(lambda i: sq.sq_gemm_w8a8(ops[i % n][0], b.x_scale, sq.SQ_PER_TOKEN, ops[i % n][1], b.w_scale,
                                           b.y)), 2.0 * M * N * K, kernel=sq.sq_gemm_kernel_name(M, N, K),
              pool=f"{n} operand sets of {(M * K + N * K) / 1e6:.0f} MB")
    r = {"gemm": r, "gemm_vendor": _vendor_gemm(torch, tm, ops, 2.0 * M * N * K)}
    del ops, inp, b
    torch.cuda.empty_cache()
    return r


def _attn_proj_step(torch, sq, synth, pipeline, dev, tm):
    """The five-step pass on the attention-projection workload (the earlier
    headline), inputs rotating over >= 1 GB of sets."""
    cfg = synth.CONFIGS[synth.ATTN_PROJ]
    M, K, N, T = cfg.M, cfg.K, cfg.N, cfg.calib_tokens
    set_bytes = (M * K + K * N + T * K) * 2
    pool = max(1, int(-(-POOL_BYTES // set_bytes)))
    _say(f"attention-projection step: {pool} input sets")
    sets = [synth.make(cfg, device=dev, variant=v) for v in range(pool)]
    b = pipeline.W8A8Buffers.allocate(M, N, K, sq.SQ_PER_TOKEN, dev)

    def step(i):
        s = sets[i % pool]
        pipeline.calibrate(s.calib, b.amax_x)
        sq.sq_prepare_and_quant_act(b.amax_x, s.w, 0.5, b.s, b.inv_s, b.amax_w, b.wq, b.w_scale, s.x,
                                    sq.SQ_PER_TOKEN, b.xq, b.x_scale, b.ws_pa)
        sq.sq_gemm_w8a8(b.xq, b.x_scale, sq.SQ_PER_TOKEN, b.wq, b.w_scale, b.y)

    us = tm(step)
    ops = 2.0 * M * N * K
    r = {"workload": cfg.name, "us_median": round(us, 2), "TOPS_whole_pass": round(ops / (us * 1e-6) / 1e12, 1),
         "pool_sets": pool, "calls": "sq_calib_reset, sq_calib_absmax, sq_prepare_and_quant_act, sq_gemm_w8a8"}
    del sets, b
    torch.cuda.empty_cache()
    return r


def _rel_error(torch, sq, dev, y_ref):
    """||y - y_ref||_F / ||y_ref||_F of an fp32 y against an fp64 y_ref, by the library."""
    ws = torch.empty(sq.sq_workspace_size(sq.SQ_OP_REL_ERROR, *y_ref.shape, 0), dtype=torch.uint8, device=dev)
    err = torch.empty(1, dtype=torch.float64, device=dev)

    def rel(y):
        sq.sq_rel_error(y, y_ref, err, ws)
        return float(err.item())
    return rel


def _alpha_sweep(torch, sq, pipeline, dev, st):
    cfg, inp, b = st["cfg"], st["inp"], st["b"]
    M, K, N = cfg.M, cfg.K, cfg.N
    _say("alpha sweep errors")
    pipeline.calibrate(inp.calib, b.amax_x)
    rows = torch.arange(0, M, M // 256, device=dev)[:256]
    xs_ = inp.x[rows].contiguous()
    y_ref = torch.empty(256, N, dtype=torch.float64, device=dev)
    sq.sq_matmul_f64(xs_, inp.w, y_ref)  # warm-up
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    sq.sq_matmul_f64(xs_, inp.w, y_ref)
    e1.record()
    torch.cuda.synchronize()
    ref_us = e0.elapsed_time(e1) * 1e3
    rel = _rel_error(torch, sq, dev, y_ref)
    bs = pipeline.W8A8Buffers.allocate(256, N, K, sq.SQ_PER_TOKEN, dev, y_dtype=torch.float32)
    bs.amax_x.copy_(b.amax_x)
    sweep = {}
    sq.sq_smooth_factors(bs.amax_x, inp.w, 0.5, bs.s, bs.inv_s, bs.amax_w)
    for a in cfg.alphas:
        sq.sq_smooth_factors(bs.amax_x, None, a, bs.s, bs.inv_s, bs.amax_w)
        sq.sq_quant_weight(inp.w, bs.s, bs.wq, bs.w_scale, bs.ws_w)
        pipeline.forward(xs_, sq.SQ_PER_TOKEN, bs, smoothed=True)
        sweep[str(a)] = round(rel(bs.y), 6)
    sq.sq_quant_weight(inp.w, None, bs.wq, bs.w_scale, bs.ws_w)
    pipeline.forward(xs_, sq.SQ_PER_TOKEN, bs, smoothed=False)
    base_tok = rel(bs.y)
    bt = pipeline.W8A8Buffers.allocate(256, N, K, sq.SQ_PER_TENSOR, dev, y_dtype=torch.float32)
    sq.sq_quant_weight(inp.w, None, bt.wq, bt.w_scale, bt.ws_w)
    pipeline.forward(xs_, sq.SQ_PER_TENSOR, bt, smoothed=False)
    base_ten = rel(bt.y)
    grid = [round(0.05 * i, 2) for i in range(21)]
    t0 = time.perf_counter()
    best, errs = pipeline.search_alpha(xs_, inp.w, b.amax_x, grid)
    torch.cuda.synchronize()
    search = {"grid": "0.00 .. 1.00 step 0.05", "best_alpha": best, "best_error": round(errs[best], 6),
              "seconds": round(time.perf_counter() - t0, 3),
              "errors": {f"{a:.2f}": round(e, 6) for a, e in errs.items()}}
    r = {"workload": cfg.name, "sample_tokens": 256, "output": "fp32", "reference": "X W in fp64",
         "search": search, "metric": "relative Frobenius error", "smoothed_per_token": sweep,
         "reference_product": {"us": round(ref_us, 1),
                               "fp64_TFLOPs": round(2.0 * 256 * N * K / (ref_us * 1e-6) / 1e12, 2)},
         "unsmoothed_per_token": round(base_tok, 6), "unsmoothed_per_tensor": round(base_ten, 6)}
    del bs, bt, y_ref
    torch.cuda.empty_cache()
    return r


def _comparator(torch, sq, synth, pipeline, dev, tm):
    """SmoothQuant against the LLM.int8()-style mixed-precision route on the
    attention-projection workload (2048 x 4096 x 4096, 41 outlier channels):
    runtime time of each per call (inputs rotating over sets larger than the
    Infinity Cache), the two GEMMs alone, and the output error of each against
    X W in fp64 on a 256-token sample."""
    cfg = synth.CONFIGS[synth.ATTN_PROJ]
    M, K, N = cfg.M, cfg.K, cfg.N
    nsets = 6  # 6 x (16.8 MB x + 33.5 MB w + 16.8 MB codes) > 256 MB
    _say(f"comparator: {nsets} sets of {cfg.name}")
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
    t_sq = tm(lambda i: pipeline.forward(sets[i % nsets].x, sq.SQ_PER_TOKEN, sqb[i % nsets], smoothed=True))
    t_l8 = tm(lambda i: pipeline.llm_int8_forward(sets[i % nsets].x, sets[i % nsets].w, 6.0, lb[i % nsets]))
    g_sq = tm(lambda i: sq.sq_gemm_w8a8(sqb[i % nsets].xq, sqb[i % nsets].x_scale, sq.SQ_PER_TOKEN,
                                        sqb[i % nsets].wq, sqb[i % nsets].w_scale, sqb[i % nsets].y))
    g_l8 = tm(lambda i: sq.sq_gemm_w8a8_outlier(lb[i % nsets].xq, lb[i % nsets].x_scale, lb[i % nsets].wq,
                                                lb[i % nsets].w_scale, lb[i % nsets].x_o, lb[i % nsets].w_ot,
                                                lb[i % nsets].count, lb[i % nsets].y))
    ops = 2.0 * M * N * K
    inp = sets[0]
    rows = torch.arange(0, M, M // 256, device=dev)[:256]
    y_ref = torch.empty(256, N, dtype=torch.float64, device=dev)
    sq.sq_matmul_f64(inp.x[rows].contiguous(), inp.w, y_ref)
    rel = _rel_error(torch, sq, dev, y_ref)

    def err(y):
        return round(rel(y[rows].contiguous()), 6)

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
        "workload": cfg.name, "threshold": 6.0, "outlier_channels": n_out[0], "outlier_channels_all_sets": n_out,
        "smoothquant_runtime_us": round(t_sq, 1), "llm_int8_runtime_us": round(t_l8, 1),
        "runtime_ratio_llm_int8_over_smoothquant": round(t_l8 / t_sq, 3),
        "smoothquant_gemm_us": round(g_sq, 1), "llm_int8_gemm_us": round(g_l8, 1),
        "smoothquant_gemm_pct_int8_peak": round(100 * ops / g_sq / 1e6 / INT8_PEAK_TOPS, 1),
        "llm_int8_gemm_kernel": sq.sq_gemm_outlier_kernel_name(M, N, K),
        "error_rel_fro_fp32": {"smoothquant_alpha_0.5_per_token": e_sq, "llm_int8": e_l8,
                               "unsmoothed_per_token": e_plain},
        "runtime_steps": {"smoothquant": "quant_act (smoothing fused) + gemm_w8a8",
                          "llm_int8": "absmax of x + outlier_columns + quant_act (keep mask) + gather_outliers "
                                      "+ gemm_w8a8_outlier"},
        "timing": "medians of HIP-event timed calls",
    }
    del sets, sqb, lb, b32, l32, y_ref
    torch.cuda.empty_cache()
    return out


def _hbm_probe(torch, dev, tm):
    """Reference points for the quantizers' access pattern on this GPU, from
    torch's own kernels over rotating 1 GB pools: a bf16 -> int8 conversion
    (reads 2 B and writes 1 B per element, the pattern of every code kernel
    here), a bf16 copy (2 + 2 B) and a bf16 max reduction (a read stream)."""
    n = 1 << 27  # 128 Mi elements: 256 MB of bf16
    src = [torch.empty(n, dtype=torch.bfloat16, device=dev).normal_() for _ in range(4)]
    dst8 = [torch.empty(n, dtype=torch.int8, device=dev) for _ in range(4)]
    dst16 = [torch.empty(n, dtype=torch.bfloat16, device=dev) for _ in range(4)]
    out = {
        "bf16_to_int8_copy": _rate(tm(lambda i: dst8[i % 4].copy_(src[i % 4])), 3 * n,
                                   note="torch elementwise conversion: read 2 B, write 1 B per element"),
        "bf16_copy": _rate(tm(lambda i: dst16[i % 4].copy_(src[i % 4])), 4 * n,
                           note="torch copy: read 2 B, write 2 B per element"),
        "bf16_amax": _rate(tm(lambda i: torch.amax(src[i % 4])), 2 * n,
                           note="torch max reduction: read 2 B per element"),
        "elements": n,
    }
    del src, dst8, dst16
    torch.cuda.empty_cache()
    return out


# ---- CPU baseline ----------------------------------------------------------------------------

def _cpu_baseline(target_s: float):
    """The oracle as it stands on the host cores, over bounded samples of the
    step's stages (large workload, alpha = 0.5), each scaled to its full size;
    the step's time is the calibration plus four times the per-alpha stages.
    The oracle's functions are single-threaded except its GEMM; samples split
    into independent row or column blocks run on a thread pool (the C calls
    release the interpreter lock), so every stage uses all the cores."""
    import numpy as np

    import oracle
    import synth

    cores = max(1, min(len(os.sched_getaffinity(0)), CPU_THREADS_MAX))
    cfg = synth.CONFIGS[synth.LARGE]
    M, K, N, T = cfg.M, cfg.K, cfg.N, cfg.calib_tokens
    L = oracle.lib()
    pool = cf.ThreadPoolExecutor(max_workers=cores)

    def blocks(n, parts):
        step = -(-n // parts)
        return [(i, min(n, i + step)) for i in range(0, n, step)]

    def p(a):
        return a.ctypes.data_as(ctypes.c_void_p)

    _say("CPU oracle baseline: drawing samples")
    tc, rw, cw, rx = 16384, 2048, 4096, 2048
    calib = synth.to_numpy(synth.make_x(cfg, "cpu", variant=101, rows=tc))
    x = synth.to_numpy(synth.make_x(cfg, "cpu", variant=102, rows=rx))
    w_rows = synth.to_numpy(synth.make(cfg, "cpu", M=1, K=rw, N=N, calib_chunks=0, variant=103).w)
    w_cols = synth.to_numpy(synth.make(cfg, "cpu", M=1, K=K, N=cw, calib_chunks=0, variant=104).w)
    t, alg = {}, {}

    # step 1: calibration absmax over tc tokens, in token blocks, maxima combined
    t0 = time.perf_counter()
    parts = list(pool.map(lambda r: oracle.calib_absmax(calib[r[0]:r[1]]), blocks(tc, cores)))
    amax = np.maximum.reduce(parts)
    t["calib_absmax"] = (time.perf_counter() - t0) * T / tc
    alg["calib_absmax"] = 2 * T * K
    # step 2: W row maxima on rw rows (row blocks), then the factors
    t0 = time.perf_counter()
    aw = np.concatenate(list(pool.map(lambda r: oracle.weight_rowmax(w_rows[r[0]:r[1]]), blocks(rw, cores))))
    t_rows = (time.perf_counter() - t0) * K / rw
    aw_full = np.resize(aw, K).astype(np.float32)
    t0 = time.perf_counter()
    s, inv_s = oracle.smooth_factors(amax, aw_full, 0.5)
    t["smooth_factors"] = t_rows + time.perf_counter() - t0
    alg["smooth_factors"] = 2 * K * N
    # step 3: weight codes of cw output columns over all K rows (column blocks of W, row stride cw)
    wq = np.empty((cw, K), np.int8)
    wsc = np.empty(cw, np.float32)

    def qw(r):
        rc = L.sqo_quant_weight(p(w_cols[:, r[0]:]), oracle.BF16, K, r[1] - r[0], cw, p(s), p(wq[r[0]:]), K,
                                p(wsc[r[0]:]))
        if rc != 0:
            raise RuntimeError("oracle quant_weight failed")

    t0 = time.perf_counter()
    list(pool.map(qw, blocks(cw, cores)))
    t["quant_weight"] = (time.perf_counter() - t0) * N / cw
    alg["quant_weight"] = 3 * K * N
    # step 4: per-token codes of rx tokens (row blocks)
    t0 = time.perf_counter()
    res = list(pool.map(lambda r: oracle.quant_act(x[r[0]:r[1]], inv_s, oracle.PER_TOKEN), blocks(rx, cores)))
    t["quant_act"] = (time.perf_counter() - t0) * M / rx
    alg["quant_act"] = 3 * M * K
    xq = np.concatenate([r[0] for r in res])
    xsc = np.concatenate([r[1] for r in res])
    # step 5: the GEMM + dequant on a row sample against the full N output channels; the weight codes of the
    # sample columns are tiled to N rows (the same codes, the full-size operand)
    wq_full = np.ascontiguousarray(np.tile(wq, (N // cw, 1)))
    ws_full = np.tile(wsc, N // cw)
    probe = cores
    t0 = time.perf_counter()
    oracle.gemm_i8(xq[:probe], wq_full, nthreads=cores)
    per_row = (time.perf_counter() - t0) / probe
    spent = sum(t.values()) * (tc / T)
    rows = int(max(cores, min(M, max(target_s - spent, 2.0) / max(per_row, 1e-9))))
    rows = min(rx, (rows + cores - 1) // cores * cores)
    t0 = time.perf_counter()
    acc = oracle.gemm_i8(xq[:rows], wq_full, nthreads=cores)
    oracle.dequant(acc, xsc[:rows], oracle.PER_TOKEN, ws_full)
    t["gemm_w8a8"] = (time.perf_counter() - t0) * M / rows
    pool.shutdown()
    na = len(cfg.alphas)
    per_alpha = t["smooth_factors"] + t["quant_weight"] + t["quant_act"] + t["gemm_w8a8"]
    total = t["calib_absmax"] + na * per_alpha
    ops = na * 2.0 * M * N * K
    stages = {}
    for k, v in t.items():
        if k == "gemm_w8a8":
            stages[k] = {"seconds_full": round(v, 3), "GOPS": round(2.0 * M * N * K / v / 1e9, 2)}
        else:
            stages[k] = {"seconds_full": round(v, 4), "GB_s": round(alg[k] / v / 1e9, 2)}
    return {
        "value": ops / total / 1e12, "unit": "TOPS", "cores": cores, "kind": "oracle",
        "sample": (f"large workload, alpha 0.5 stages timed on samples and scaled to full size: calibration absmax "
                   f"on {tc} of {T} tokens, W row maxima on {rw} of {K} rows, weight codes on {cw} of {N} output "
                   f"columns (all {K} rows), activation codes on {rx} of {M} tokens, GEMM + dequant on {rows} of "
                   f"{M} tokens against all {N} channels; step = calibration + {na} x (factors, weight codes, "
                   f"activation codes, GEMM); every stage on {cores} threads (sample blocks on a thread pool; the "
                   f"GEMM on the oracle's own threads)"),
        "seconds_per_step_extrapolated": round(total, 2), "stages": stages, "cpu_model": _cpu_model(),
    }


def main():
    args = _parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(f"bench.py measures one GPU only: this path runs on a single MI355X and has no multi-GPU mode "
              f"(asked for --gpus {args.gpus}).", file=sys.stderr)
        sys.exit(2)
    sections = [s for s in args.sections.split(",") if s]
    for s in sections:
        if s not in SECTIONS + EXTRA_SECTIONS:
            print(f"unknown section {s!r}; choose from {','.join(SECTIONS + EXTRA_SECTIONS)}", file=sys.stderr)
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
    tm = _Timer(torch, args.runs)

    out, st = _step(torch, sq, synth, pipeline, dev, args)
    if "workloads" in sections:
        rows = {"timing": f"median of {args.runs} HIP-event timed calls after 5 warm-up calls; inputs rotate over "
                            f">= {POOL_BYTES / 1e9:.0f} GB of independent copies unless one input is larger"}
        rows["large_8192x12288x49152"] = _workload_large(torch, sq, pipeline, dev, tm, st)
    if "alpha" in sections:
        out["alpha_sweep"] = _alpha_sweep(torch, sq, pipeline, dev, st)
    del st
    torch.cuda.empty_cache()
    if "workloads" in sections:
        rows["mlp_up_4096x4096x14336"] = _workload_mlp_up(torch, sq, synth, pipeline, dev, tm)
        rows["decode_16x8192x28672"] = _workload_decode(torch, sq, synth, pipeline, dev, tm)
        rows["attn_proj_2048x4096x4096"] = _workload_attn_gemm(torch, sq, synth, pipeline, dev, tm)
        out["workloads"] = rows
    if "attn_proj" in sections:
        out["attn_proj_step"] = _attn_proj_step(torch, sq, synth, pipeline, dev, tm)
    if "comparator" in sections:
        out["llm_int8_comparator"] = _comparator(torch, sq, synth, pipeline, dev, tm)
    if "probe" in sections:
        out["hbm_probe"] = _hbm_probe(torch, dev, tm)
    if "tile_sweep" in sections:
        out["tile_sweep"] = _tile_sweep(torch, sq, dev, tm)
    if not args.no_cpu:
        out["cpu_baseline"] = _cpu_baseline(args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
