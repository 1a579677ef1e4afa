"""The five calls in order, over device buffers allocated once.

This is orchestration only: it allocates output tensors with torch and calls
the C entry points; every step of the computation runs in the HIP kernels.
"""
from __future__ import annotations

from dataclasses import dataclass

import torch

from . import (SQ_OP_PREPARE_AND_QUANT_ACT, SQ_OP_PREPARE_WEIGHTS, SQ_OP_QUANT_ACT, SQ_OP_QUANT_WEIGHT, SQ_OP_REL_ERROR,
               SQ_PER_TENSOR, SQ_PER_TOKEN, sq_calib_absmax, sq_gather_outliers, sq_gemm_w8a8, sq_gemm_w8a8_outlier,
               sq_matmul_f64, sq_outlier_columns, sq_prepare_and_quant_act, sq_prepare_weights, sq_quant_act,
               sq_quant_weight, sq_calib_reset, sq_rel_error, sq_smooth_factors, sq_workspace_size)


@dataclass
class W8A8Buffers:
    amax_x: torch.Tensor
    amax_w: torch.Tensor
    s: torch.Tensor
    inv_s: torch.Tensor
    wq: torch.Tensor
    w_scale: torch.Tensor
    xq: torch.Tensor
    x_scale: torch.Tensor
    y: torch.Tensor
    acc: torch.Tensor | None
    ws_w: torch.Tensor | None
    ws_a: torch.Tensor | None
    ws_p: torch.Tensor | None
    ws_pa: torch.Tensor | None

    @classmethod
    def allocate(cls, M: int, N: int, K: int, gran: int, device, y_dtype=torch.bfloat16, with_acc=False):
        f32 = dict(dtype=torch.float32, device=device)

        def ws(nbytes):
            return torch.empty(max(nbytes, 16), dtype=torch.uint8, device=device) if nbytes else None

        return cls(
            amax_x=torch.zeros(K, **f32), amax_w=torch.empty(K, **f32), s=torch.empty(K, **f32),
            inv_s=torch.empty(K, **f32), wq=torch.empty(N, K, dtype=torch.int8, device=device),
            w_scale=torch.empty(N, **f32), xq=torch.empty(M, K, dtype=torch.int8, device=device),
            x_scale=torch.empty(1 if gran == SQ_PER_TENSOR else M, **f32),
            y=torch.empty(M, N, dtype=y_dtype, device=device),
            acc=torch.empty(M, N, dtype=torch.int32, device=device) if with_acc else None,
            ws_w=ws(sq_workspace_size(SQ_OP_QUANT_WEIGHT, M, N, K, gran)),
            ws_a=ws(sq_workspace_size(SQ_OP_QUANT_ACT, M, N, K, gran)),
            ws_p=ws(sq_workspace_size(SQ_OP_PREPARE_WEIGHTS, M, N, K, gran)),
            ws_pa=ws(sq_workspace_size(SQ_OP_PREPARE_AND_QUANT_ACT, M, N, K, gran)),
        )


def calibrate(calib, amax_x: torch.Tensor, reset: bool = True, stream=None) -> None:
    """Step 1 over one [T, K] tensor or a sequence of chunks."""
    if reset:
        sq_calib_reset(amax_x, stream=stream)
    chunks = calib if isinstance(calib, (list, tuple)) else [calib]
    for c in chunks:
        sq_calib_absmax(c, amax_x, stream=stream)


def prepare_weights(w: torch.Tensor, alpha: float | None, b: W8A8Buffers, stream=None, fused: bool = True) -> None:
    """Steps 2-3 (alpha=None: unsmoothed weights).  fused: one sq_prepare_weights call; otherwise
    sq_smooth_factors then sq_quant_weight (same results)."""
    if alpha is None:
        sq_quant_weight(w, None, b.wq, b.w_scale, b.ws_w, stream=stream)
        return
    if fused:
        sq_prepare_weights(b.amax_x, w, alpha, b.s, b.inv_s, b.amax_w, b.wq, b.w_scale, b.ws_p, stream=stream)
        return
    sq_smooth_factors(b.amax_x, w, alpha, b.s, b.inv_s, b.amax_w, stream=stream)
    sq_quant_weight(w, b.s, b.wq, b.w_scale, b.ws_w, stream=stream)


def forward(x: torch.Tensor, gran: int, b: W8A8Buffers, smoothed: bool = True, stream=None) -> torch.Tensor:
    """Steps 4-5 on activations x [M, K]."""
    sq_quant_act(x, b.inv_s if smoothed else None, gran, b.xq, b.x_scale, b.ws_a, stream=stream)
    sq_gemm_w8a8(b.xq, b.x_scale, gran, b.wq, b.w_scale, b.y, b.acc, stream=stream)
    return b.y


def prepare_and_quantize(x: torch.Tensor, w: torch.Tensor, alpha: float, gran: int, b: W8A8Buffers,
                         stream=None) -> None:
    """Steps 2-4 in one call (the weight codes and the activation codes may share a launch)."""
    sq_prepare_and_quant_act(b.amax_x, w, alpha, b.s, b.inv_s, b.amax_w, b.wq, b.w_scale, x, gran, b.xq, b.x_scale,
                             b.ws_pa, stream=stream)


def smoothquant_w8a8(x, w, calib, alpha: float | None, gran: int, b: W8A8Buffers, stream=None,
                     fused: bool = True) -> torch.Tensor:
    """All five steps.  alpha=None runs the unsmoothed W8A8 baseline (no calibration).  fused: steps 2-4
    through sq_prepare_and_quant_act; otherwise sq_smooth_factors, sq_quant_weight, sq_quant_act."""
    if alpha is None:
        prepare_weights(w, None, b, stream=stream)
        return forward(x, gran, b, smoothed=False, stream=stream)
    calibrate(calib, b.amax_x, stream=stream)
    if fused:
        prepare_and_quantize(x, w, alpha, gran, b, stream=stream)
        sq_gemm_w8a8(b.xq, b.x_scale, gran, b.wq, b.w_scale, b.y, b.acc, stream=stream)
        return b.y
    prepare_weights(w, alpha, b, stream=stream, fused=False)
    return forward(x, gran, b, smoothed=True, stream=stream)


class CapturedPass:
    """All five calls recorded once into a HIP graph over fixed tensors (x, w,
    calib and the buffers in b), then replayed with a single launch.

    The library enqueues only kernels (its buffer clears, the clear of the
    running maximum included, are fill kernels), so the recorded graph holds no
    memset nodes.  Inputs are read where they lie at replay time: write new
    data into the same tensors between replays."""

    def __init__(self, x, w, calib, alpha: float | None, gran: int, b: W8A8Buffers, warmup: int = 1):
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for _ in range(warmup):
                smoothquant_w8a8(x, w, calib, alpha, gran, b)
        torch.cuda.current_stream().wait_stream(side)
        self.graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.graph):
            smoothquant_w8a8(x, w, calib, alpha, gran, b)
        self.b = b

    def replay(self) -> torch.Tensor:
        self.graph.replay()
        return self.b.y


def search_alpha(x_sample: torch.Tensor, w: torch.Tensor, amax_x: torch.Tensor, alphas, gran: int = 0):
    """Offline migration-strength search: for each alpha of the grid, quantize W
    and the token sample x_sample with the library and compare the W8A8 output
    (fp32, before the bf16 rounding) with X W in fp64, by relative Frobenius
    error.  amax_x: the calibration maxima (step 1).  Returns (best alpha,
    {alpha: error}); ties go to the first alpha of the grid.

    Every step runs in the library: the quantization, the INT8 GEMM, the fp64
    reference product (sq_matmul_f64) and the error (sq_rel_error); Python only
    picks the smallest of the returned errors."""
    M, K = x_sample.shape
    N = w.shape[1]
    dev = x_sample.device
    b = W8A8Buffers.allocate(M, N, K, gran, dev, y_dtype=torch.float32)
    b.amax_x.copy_(amax_x)
    y_ref = torch.empty(M, N, dtype=torch.float64, device=dev)
    sq_matmul_f64(x_sample, w, y_ref)
    ws = torch.empty(sq_workspace_size(SQ_OP_REL_ERROR, M, N, 0), dtype=torch.uint8, device=dev)
    err = torch.empty(len(alphas), dtype=torch.float64, device=dev)
    for i, a in enumerate(alphas):
        if i == 0:
            sq_smooth_factors(b.amax_x, w, float(a), b.s, b.inv_s, b.amax_w)  # row maxima of W once
        else:
            sq_smooth_factors(b.amax_x, None, float(a), b.s, b.inv_s, b.amax_w)
        sq_quant_weight(w, b.s, b.wq, b.w_scale, b.ws_w)
        forward(x_sample, gran, b, smoothed=True)
        sq_rel_error(b.y, y_ref, err[i:i + 1], ws)
    errs = dict(zip((float(a) for a in alphas), err.tolist()))
    best = min(errs, key=lambda a: (errs[a], list(errs).index(a)))
    return best, errs


# ---- LLM.int8()-style comparator -------------------------------------------------------

@dataclass
class LlmInt8Buffers:
    """Device buffers of the mixed-precision comparator: offline weight codes
    of W itself, and the per-call outlier set, INT8 activations and compact
    16-bit outlier operands (kp = K rounded up to 16, room for every channel)."""
    wq: torch.Tensor
    w_scale: torch.Tensor
    amax_x: torch.Tensor
    idx: torch.Tensor
    count: torch.Tensor
    keep: torch.Tensor
    xq: torch.Tensor
    x_scale: torch.Tensor
    x_o: torch.Tensor
    w_ot: torch.Tensor
    y: torch.Tensor
    ws_w: torch.Tensor | None

    @classmethod
    def allocate(cls, M: int, N: int, K: int, device, y_dtype=torch.bfloat16):
        kp = (K + 15) // 16 * 16
        nb = sq_workspace_size(SQ_OP_QUANT_WEIGHT, 0, N, K)
        return cls(
            wq=torch.empty(N, K, dtype=torch.int8, device=device),
            w_scale=torch.empty(N, dtype=torch.float32, device=device),
            amax_x=torch.empty(K, dtype=torch.float32, device=device),
            idx=torch.empty(K, dtype=torch.int32, device=device),
            count=torch.empty(1, dtype=torch.int32, device=device),
            keep=torch.empty(K, dtype=torch.float32, device=device),
            xq=torch.empty(M, K, dtype=torch.int8, device=device),
            x_scale=torch.empty(M, dtype=torch.float32, device=device),
            x_o=torch.empty(M, kp, dtype=torch.bfloat16, device=device),
            w_ot=torch.empty(N, kp, dtype=torch.bfloat16, device=device),
            y=torch.empty(M, N, dtype=y_dtype, device=device),
            ws_w=torch.empty(max(nb, 16), dtype=torch.uint8, device=device) if nb else None,
        )


def llm_int8_prepare(w: torch.Tensor, b: LlmInt8Buffers, stream=None) -> None:
    """Offline: per-output-channel INT8 codes of W itself (no smoothing)."""
    sq_quant_weight(w, None, b.wq, b.w_scale, b.ws_w, stream=stream)


def llm_int8_forward(x: torch.Tensor, w: torch.Tensor, threshold: float, b: LlmInt8Buffers,
                     stream=None) -> torch.Tensor:
    """Runtime pass: outlier channels of this x (max |x| > threshold) in 16 bits,
    the rest per-token INT8, summed (five library calls, no host sync)."""
    b.amax_x.zero_()
    sq_calib_absmax(x, b.amax_x, stream=stream)
    sq_outlier_columns(b.amax_x, threshold, b.idx, b.count, b.keep, stream=stream)
    sq_quant_act(x, b.keep, SQ_PER_TOKEN, b.xq, b.x_scale, stream=stream)
    sq_gather_outliers(x, w, b.idx, b.count, b.x_o, b.w_ot, stream=stream)
    sq_gemm_w8a8_outlier(b.xq, b.x_scale, b.wq, b.w_scale, b.x_o, b.w_ot, b.count, b.y, stream=stream)
    return b.y
