"""SmoothQuant W8A8 linear layer on AMD Instinct MI355X (gfx950).

Thin ctypes binding over ``libsq.so`` (the C ABI declared in include/sq.h).
Each function has the name of the C entry point, takes torch tensors that
live on the GPU, passes their device pointers, strides and the current HIP
stream, and raises ``SqError`` with the library's message when the call is
rejected.  No computation happens in Python: every step runs in the HIP
kernels, and the module refuses to work without the built library.

Build the library first: ``python -m post_quantization_act_amd.build``.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "SqError", "SQ_F32", "SQ_BF16", "SQ_PER_TOKEN", "SQ_PER_TENSOR",
    "SQ_OP_CALIB_ABSMAX", "SQ_OP_SMOOTH_FACTORS", "SQ_OP_QUANT_WEIGHT", "SQ_OP_QUANT_ACT", "SQ_OP_GEMM_W8A8",
    "lib", "lib_path", "sq_calib_absmax", "sq_calib_reset", "sq_smooth_factors", "sq_quant_weight",
    "sq_quant_weight_noalloc", "sq_quant_act",
    "sq_gemm_w8a8", "sq_prepare_weights", "sq_prepare_and_quant_act", "SQ_OP_PREPARE_WEIGHTS",
    "SQ_OP_PREPARE_AND_QUANT_ACT", "sq_static_act_max", "sq_quant_act_static", "sq_fold_layernorm",
    "sq_layernorm_quant", "sq_outlier_columns", "sq_gather_outliers", "sq_gemm_w8a8_outlier",
    "sq_gemm_outlier_kernel_name", "sq_matmul_f64", "sq_rel_error", "SQ_OP_REL_ERROR", "sq_workspace_size",
    "sq_status_str", "sq_last_error", "sq_version", "sq_gemm_kernel_name", "EXPORTED_SYMBOLS",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libsq.so")

SQ_F32, SQ_BF16 = 0, 1
SQ_PER_TOKEN, SQ_PER_TENSOR = 0, 1
(SQ_OP_CALIB_ABSMAX, SQ_OP_SMOOTH_FACTORS, SQ_OP_QUANT_WEIGHT, SQ_OP_QUANT_ACT, SQ_OP_GEMM_W8A8, SQ_OP_PREPARE_WEIGHTS,
 SQ_OP_PREPARE_AND_QUANT_ACT, SQ_OP_REL_ERROR) = range(8)

EXPORTED_SYMBOLS = (
    "sq_calib_absmax", "sq_calib_reset", "sq_smooth_factors", "sq_quant_weight", "sq_quant_weight_noalloc",
    "sq_quant_act", "sq_gemm_w8a8", "sq_prepare_weights", "sq_prepare_and_quant_act", "sq_static_act_max", "sq_quant_act_static", "sq_fold_layernorm", "sq_layernorm_quant", "sq_outlier_columns",
    "sq_gather_outliers", "sq_gemm_w8a8_outlier", "sq_matmul_f64", "sq_rel_error", "sq_workspace_size", "sq_status_str", "sq_last_error",
    "sq_version", "sq_gemm_kernel_name", "sq_gemm_outlier_kernel_name",
)


class SqError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{sq_status_str(status)}: {message}")
        self.status = status


_lib = None


def lib_path() -> str:
    return _LIB_PATH


def lib() -> ctypes.CDLL:
    """Load libsq.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(f"{_LIB_PATH} is missing: build it with `python -m post_quantization_act_amd.build`")
    L = ctypes.CDLL(_LIB_PATH)
    vp, i64, i32, f32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float
    sz = ctypes.c_size_t
    L.sq_calib_absmax.argtypes = [vp, i32, i64, i64, i64, vp, vp]
    L.sq_calib_reset.argtypes = [vp, i64, vp]
    L.sq_smooth_factors.argtypes = [vp, vp, i32, i64, i64, i64, f32, vp, vp, vp, vp]
    L.sq_quant_weight.argtypes = [vp, i32, i64, i64, i64, vp, vp, vp, vp, sz, vp]
    L.sq_quant_weight_noalloc.argtypes = [vp, i32, i64, i64, i64, vp, vp, vp, vp]
    L.sq_quant_act.argtypes = [vp, i32, i64, i64, i64, vp, i32, vp, vp, vp, sz, vp]
    L.sq_gemm_w8a8.argtypes = [vp, vp, i32, vp, vp, i64, i64, i64, vp, i32, vp, vp, sz, vp]
    L.sq_prepare_weights.argtypes = [vp, vp, i32, i64, i64, i64, f32, vp, vp, vp, vp, vp, vp, sz, vp]
    L.sq_prepare_and_quant_act.argtypes = [vp, vp, i32, i64, i64, i64, f32, vp, vp, vp, vp, vp, vp, i32, i64, i64,
                                           i32, vp, vp, vp, sz, vp]
    L.sq_static_act_max.argtypes = [vp, vp, i64, vp, vp]
    L.sq_quant_act_static.argtypes = [vp, i32, i64, i64, i64, vp, vp, vp, vp, vp]
    L.sq_fold_layernorm.argtypes = [vp, vp, vp, i64, vp, vp, vp]
    L.sq_layernorm_quant.argtypes = [vp, i32, i64, i64, i64, vp, vp, f32, vp, vp, vp]
    L.sq_outlier_columns.argtypes = [vp, i64, f32, vp, vp, vp, vp]
    L.sq_gather_outliers.argtypes = [vp, i32, i64, i64, i64, vp, i32, i64, i64, vp, vp, i64, vp, vp, vp]
    L.sq_gemm_w8a8_outlier.argtypes = [vp, vp, vp, vp, i64, i64, i64, vp, vp, i64, vp, vp, i32, vp]
    L.sq_matmul_f64.argtypes = [vp, i32, i64, i64, i64, vp, i32, i64, i64, vp, vp]
    L.sq_rel_error.argtypes = [vp, vp, i64, i64, vp, vp, sz, vp]
    for f in ("sq_calib_absmax", "sq_smooth_factors", "sq_quant_weight", "sq_quant_weight_noalloc", "sq_quant_act",
              "sq_gemm_w8a8",
              "sq_prepare_weights", "sq_static_act_max", "sq_quant_act_static", "sq_fold_layernorm",
              "sq_layernorm_quant", "sq_outlier_columns", "sq_gather_outliers", "sq_gemm_w8a8_outlier",
              "sq_matmul_f64", "sq_rel_error"):
        getattr(L, f).restype = ctypes.c_int
    L.sq_workspace_size.argtypes = [i32, i64, i64, i64, i32]
    L.sq_workspace_size.restype = sz
    L.sq_status_str.argtypes = [i32]
    L.sq_status_str.restype = ctypes.c_char_p
    L.sq_last_error.argtypes = []
    L.sq_last_error.restype = ctypes.c_char_p
    L.sq_version.argtypes = []
    L.sq_version.restype = ctypes.c_char_p
    L.sq_gemm_kernel_name.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int64]
    L.sq_gemm_kernel_name.restype = ctypes.c_char_p
    L.sq_gemm_outlier_kernel_name.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int64]
    L.sq_gemm_outlier_kernel_name.restype = ctypes.c_char_p
    _lib = L
    return L


def sq_status_str(status: int) -> str:
    return lib().sq_status_str(int(status)).decode()


def sq_last_error() -> str:
    return lib().sq_last_error().decode()


def sq_version() -> str:
    return lib().sq_version().decode()


def sq_gemm_kernel_name(M: int, N: int, K: int) -> str:
    """Which GEMM kernel sq_gemm_w8a8 launches for an M x N x K product."""
    return lib().sq_gemm_kernel_name(int(M), int(N), int(K)).decode()


def sq_gemm_outlier_kernel_name(M: int, N: int, K: int) -> str:
    """Which GEMM kernel sq_gemm_w8a8_outlier launches for an M x N x K product."""
    return lib().sq_gemm_outlier_kernel_name(int(M), int(N), int(K)).decode()


def sq_workspace_size(op: int, M: int, N: int, K: int, gran: int = SQ_PER_TOKEN) -> int:
    return int(lib().sq_workspace_size(int(op), int(M), int(N), int(K), int(gran)))


# ---- marshalling helpers -----------------------------------------------------------

def _ptr(t):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"expected a torch.Tensor, got {type(t)}")
    if t.numel() > 0 and t.device.type != "cuda":
        raise ValueError("libsq takes device tensors; got a tensor on " + str(t.device))
    return ctypes.c_void_p(t.data_ptr()) if t.numel() > 0 else ctypes.c_void_p(t.data_ptr() or None)


def _dtype(t) -> int:
    if t.dtype == torch.bfloat16:
        return SQ_BF16
    if t.dtype == torch.float32:
        return SQ_F32
    raise TypeError(f"unsupported dtype {t.dtype}: use torch.bfloat16 or torch.float32")


def _stream(device, stream):
    if stream is not None:
        return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))
    if device is None or device.type != "cuda":
        return ctypes.c_void_p(None)
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _rows(t):
    """(rows, cols, row stride) of a 2-D tensor whose last axis is contiguous."""
    if t.dim() != 2:
        raise ValueError(f"expected a 2-D tensor, got shape {tuple(t.shape)}")
    if t.shape[1] > 1 and t.stride(1) != 1:
        raise ValueError("the last axis must be contiguous")
    return t.shape[0], t.shape[1], (t.stride(0) if t.shape[0] > 1 else t.shape[1])


def _dense(t, name, shape, dtype):
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _check(rc: int):
    if rc != 0:
        raise SqError(rc, sq_last_error())


def _dev(*ts):
    for t in ts:
        if isinstance(t, torch.Tensor):
            return t.device
    return None


# ---- the five entry points ---------------------------------------------------------

def sq_calib_absmax(x: torch.Tensor, amax: torch.Tensor, stream=None) -> None:
    """amax[j] = max(amax[j], max_t |x[t, j]|) for x [T, K] (bf16 or fp32)."""
    T, K, ld = _rows(x)
    _dense(amax, "amax", (K,), torch.float32)
    _check(lib().sq_calib_absmax(_ptr(x), _dtype(x), T, K, ld, _ptr(amax), _stream(_dev(x, amax), stream)))


def sq_calib_reset(amax: torch.Tensor, stream=None) -> None:
    """amax[:] = 0, the start of a calibration (a library kernel, safe to record in a HIP graph)."""
    K = amax.shape[0]
    _dense(amax, "amax", (K,), torch.float32)
    _check(lib().sq_calib_reset(_ptr(amax), K, _stream(_dev(amax), stream)))


def sq_smooth_factors(amax_x: torch.Tensor, w: torch.Tensor | None, alpha: float, s: torch.Tensor,
                      inv_s: torch.Tensor, amax_w: torch.Tensor | None = None, stream=None) -> None:
    """s, inv_s [K] from amax_x [K] and W [K, N] (or a precomputed amax_w when w is None)."""
    K = amax_x.shape[0]
    _dense(amax_x, "amax_x", (K,), torch.float32)
    _dense(s, "s", (K,), torch.float32)
    _dense(inv_s, "inv_s", (K,), torch.float32)
    if amax_w is not None:
        _dense(amax_w, "amax_w", (K,), torch.float32)
    if w is not None:
        Kw, N, ld = _rows(w)
        if Kw != K:
            raise ValueError(f"w has {Kw} rows, amax_x has {K} entries")
        wt = _dtype(w)
    else:
        N, ld, wt = 0, 0, SQ_BF16
    _check(lib().sq_smooth_factors(_ptr(amax_x), _ptr(w), wt, K, N, ld, ctypes.c_float(alpha), _ptr(s),
                                   _ptr(inv_s), _ptr(amax_w), _stream(_dev(amax_x), stream)))


def sq_quant_weight(w: torch.Tensor, s: torch.Tensor | None, wq: torch.Tensor, w_scale: torch.Tensor,
                    ws: torch.Tensor | None, stream=None) -> None:
    """wq [N, K] int8 and w_scale [N] from W [K, N] smoothed by s [K] (None: unsmoothed)."""
    K, N, ld = _rows(w)
    _dense(wq, "wq", (N, K), torch.int8)
    _dense(w_scale, "w_scale", (N,), torch.float32)
    if s is not None:
        _dense(s, "s", (K,), torch.float32)
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().sq_quant_weight(_ptr(w), _dtype(w), K, N, ld, _ptr(s), _ptr(wq), _ptr(w_scale), _ptr(ws), nbytes,
                                 _stream(_dev(w), stream)))


def sq_quant_weight_noalloc(w: torch.Tensor, s: torch.Tensor | None, wq: torch.Tensor, w_scale: torch.Tensor,
                            stream=None) -> None:
    """sq_quant_weight with the library's static scratch instead of a workspace (N <= 65536; calls on one
    device must not overlap)."""
    K, N, ld = _rows(w)
    _dense(wq, "wq", (N, K), torch.int8)
    _dense(w_scale, "w_scale", (N,), torch.float32)
    if s is not None:
        _dense(s, "s", (K,), torch.float32)
    _check(lib().sq_quant_weight_noalloc(_ptr(w), _dtype(w), K, N, ld, _ptr(s), _ptr(wq), _ptr(w_scale),
                                         _stream(_dev(w), stream)))


def sq_prepare_weights(amax_x: torch.Tensor, w: torch.Tensor, alpha: float, s: torch.Tensor, inv_s: torch.Tensor,
                       amax_w: torch.Tensor | None, wq: torch.Tensor, w_scale: torch.Tensor, ws: torch.Tensor | None,
                       stream=None) -> None:
    """Steps 2 and 3 in one call: s, inv_s [K] (and amax_w) from amax_x and W [K, N], then wq [N, K] and
    w_scale [N] of diag(s) W."""
    K, N, ld = _rows(w)
    _dense(amax_x, "amax_x", (K,), torch.float32)
    _dense(s, "s", (K,), torch.float32)
    _dense(inv_s, "inv_s", (K,), torch.float32)
    if amax_w is not None:
        _dense(amax_w, "amax_w", (K,), torch.float32)
    _dense(wq, "wq", (N, K), torch.int8)
    _dense(w_scale, "w_scale", (N,), torch.float32)
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().sq_prepare_weights(_ptr(amax_x), _ptr(w), _dtype(w), K, N, ld, ctypes.c_float(alpha), _ptr(s),
                                    _ptr(inv_s), _ptr(amax_w), _ptr(wq), _ptr(w_scale), _ptr(ws), nbytes,
                                    _stream(_dev(w, amax_x), stream)))


def sq_prepare_and_quant_act(amax_x: torch.Tensor, w: torch.Tensor, alpha: float, s: torch.Tensor,
                             inv_s: torch.Tensor, amax_w: torch.Tensor | None, wq: torch.Tensor, w_scale: torch.Tensor,
                             x: torch.Tensor, gran: int, xq: torch.Tensor, x_scale: torch.Tensor,
                             ws: torch.Tensor | None, stream=None) -> None:
    """Steps 2, 3 and 4 in one call: sq_prepare_weights(amax_x, w, alpha, ...) then
    sq_quant_act(x, inv_s, gran, xq, x_scale, ...), with the same results."""
    K, N, ldw = _rows(w)
    M, Kx, ldx = _rows(x)
    if Kx != K:
        raise ValueError(f"x has {Kx} channels, w has {K}")
    _dense(amax_x, "amax_x", (K,), torch.float32)
    _dense(s, "s", (K,), torch.float32)
    _dense(inv_s, "inv_s", (K,), torch.float32)
    if amax_w is not None:
        _dense(amax_w, "amax_w", (K,), torch.float32)
    _dense(wq, "wq", (N, K), torch.int8)
    _dense(w_scale, "w_scale", (N,), torch.float32)
    _dense(xq, "xq", (M, K), torch.int8)
    _dense(x_scale, "x_scale", (1,) if gran == SQ_PER_TENSOR else (M,), torch.float32)
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().sq_prepare_and_quant_act(_ptr(amax_x), _ptr(w), _dtype(w), K, N, ldw, ctypes.c_float(alpha), _ptr(s),
                                          _ptr(inv_s), _ptr(amax_w), _ptr(wq), _ptr(w_scale), _ptr(x), _dtype(x), M,
                                          ldx, int(gran), _ptr(xq), _ptr(x_scale), _ptr(ws), nbytes,
                                          _stream(_dev(w, x), stream)))


def sq_fold_layernorm(gamma: torch.Tensor, beta: torch.Tensor | None, inv_s: torch.Tensor, gamma_out: torch.Tensor,
                      beta_out: torch.Tensor | None = None, stream=None) -> None:
    """gamma_out = gamma * inv_s, beta_out = beta * inv_s (fp32, [K]): the smoothing folded into a LayerNorm."""
    K = gamma.shape[0]
    for t, n in ((gamma, "gamma"), (inv_s, "inv_s"), (gamma_out, "gamma_out")):
        _dense(t, n, (K,), torch.float32)
    if beta is not None:
        _dense(beta, "beta", (K,), torch.float32)
        _dense(beta_out, "beta_out", (K,), torch.float32)
    _check(lib().sq_fold_layernorm(_ptr(gamma), _ptr(beta), _ptr(inv_s), K, _ptr(gamma_out), _ptr(beta_out),
                                   _stream(_dev(gamma), stream)))


def sq_layernorm_quant(x: torch.Tensor, gamma: torch.Tensor, beta: torch.Tensor | None, eps: float,
                       xq: torch.Tensor, x_scale: torch.Tensor, stream=None) -> None:
    """LayerNorm of bf16 rows x [M, K] with (folded) gamma/beta, then per-token INT8 codes and scales."""
    M, K, ld = _rows(x)
    _dense(gamma, "gamma", (K,), torch.float32)
    if beta is not None:
        _dense(beta, "beta", (K,), torch.float32)
    _dense(xq, "xq", (M, K), torch.int8)
    _dense(x_scale, "x_scale", (M,), torch.float32)
    _check(lib().sq_layernorm_quant(_ptr(x), _dtype(x), M, K, ld, _ptr(gamma), _ptr(beta), ctypes.c_float(eps),
                                    _ptr(xq), _ptr(x_scale), _stream(_dev(x), stream)))


def sq_static_act_max(amax_x: torch.Tensor, inv_s: torch.Tensor | None, a_static: torch.Tensor,
                      stream=None) -> None:
    """a_static[0] = max_j fl(amax_x[j] * inv_s[j]): the calibrated per-tensor maximum of X'."""
    K = amax_x.shape[0]
    _dense(amax_x, "amax_x", (K,), torch.float32)
    if inv_s is not None:
        _dense(inv_s, "inv_s", (K,), torch.float32)
    _dense(a_static, "a_static", (1,), torch.float32)
    _check(lib().sq_static_act_max(_ptr(amax_x), _ptr(inv_s), K, _ptr(a_static), _stream(_dev(amax_x), stream)))


def sq_quant_act_static(x: torch.Tensor, inv_s: torch.Tensor | None, a_static: torch.Tensor, xq: torch.Tensor,
                        x_scale: torch.Tensor, stream=None) -> None:
    """Step 4 with the fixed per-tensor maximum a_static[0] (values beyond it saturate)."""
    M, K, ld = _rows(x)
    _dense(xq, "xq", (M, K), torch.int8)
    _dense(x_scale, "x_scale", (1,), torch.float32)
    _dense(a_static, "a_static", (1,), torch.float32)
    if inv_s is not None:
        _dense(inv_s, "inv_s", (K,), torch.float32)
    _check(lib().sq_quant_act_static(_ptr(x), _dtype(x), M, K, ld, _ptr(inv_s), _ptr(a_static), _ptr(xq),
                                     _ptr(x_scale), _stream(_dev(x), stream)))


def sq_quant_act(x: torch.Tensor, inv_s: torch.Tensor | None, gran: int, xq: torch.Tensor,
                 x_scale: torch.Tensor, ws: torch.Tensor | None = None, stream=None) -> None:
    """xq [M, K] int8 and x_scale ([M] per token, [1] per tensor) from X [M, K] smoothed by inv_s."""
    M, K, ld = _rows(x)
    _dense(xq, "xq", (M, K), torch.int8)
    _dense(x_scale, "x_scale", (1,) if gran == SQ_PER_TENSOR else (M,), torch.float32)
    if inv_s is not None:
        _dense(inv_s, "inv_s", (K,), torch.float32)
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().sq_quant_act(_ptr(x), _dtype(x), M, K, ld, _ptr(inv_s), int(gran), _ptr(xq), _ptr(x_scale),
                              _ptr(ws), nbytes, _stream(_dev(x), stream)))


def sq_gemm_w8a8(xq: torch.Tensor, x_scale: torch.Tensor, gran: int, wq: torch.Tensor, w_scale: torch.Tensor,
                 y: torch.Tensor, acc_out: torch.Tensor | None = None, ws: torch.Tensor | None = None,
                 stream=None) -> None:
    """y [M, N] (bf16 or fp32) = dequant(Xq [M, K] . Wq [N, K]^T); acc_out [M, N] int32 optional."""
    M, K = xq.shape
    N = wq.shape[0]
    _dense(xq, "xq", (M, K), torch.int8)
    _dense(wq, "wq", (N, K), torch.int8)
    _dense(x_scale, "x_scale", (1,) if gran == SQ_PER_TENSOR else (M,), torch.float32)
    _dense(w_scale, "w_scale", (N,), torch.float32)
    if y.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("y must be bfloat16 or float32")
    _dense(y, "y", (M, N), y.dtype)
    if acc_out is not None:
        _dense(acc_out, "acc_out", (M, N), torch.int32)
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().sq_gemm_w8a8(_ptr(xq), _ptr(x_scale), int(gran), _ptr(wq), _ptr(w_scale), M, N, K, _ptr(y),
                              _dtype(y), _ptr(acc_out), _ptr(ws), nbytes, _stream(_dev(xq), stream)))


# ---- LLM.int8()-style comparator ---------------------------------------------------

def sq_outlier_columns(amax_x: torch.Tensor, threshold: float, idx: torch.Tensor, count: torch.Tensor,
                       keep: torch.Tensor, stream=None) -> None:
    """idx[0:count] = the channels with amax_x > threshold (ascending); keep = 0 there, 1 elsewhere."""
    K = amax_x.shape[0]
    _dense(amax_x, "amax_x", (K,), torch.float32)
    _dense(idx, "idx", (K,), torch.int32)
    _dense(count, "count", (1,), torch.int32)
    _dense(keep, "keep", (K,), torch.float32)
    _check(lib().sq_outlier_columns(_ptr(amax_x), K, float(threshold), _ptr(idx), _ptr(count), _ptr(keep),
                                    _stream(_dev(amax_x), stream)))


def sq_gather_outliers(x: torch.Tensor, w: torch.Tensor, idx: torch.Tensor, count: torch.Tensor,
                       x_o: torch.Tensor, w_ot: torch.Tensor, stream=None) -> None:
    """x_o [M, kp] = outlier columns of x [M, K]; w_ot [N, kp] = outlier rows of w [K, N], transposed
    (bf16, zero-padded to a multiple of 16 channels)."""
    M, K, ldx = _rows(x)
    K2, N, ldw = _rows(w)
    if K2 != K:
        raise ValueError("x and w disagree on K")
    kp = x_o.shape[1] if x_o.dim() == 2 else 0
    _dense(x_o, "x_o", (M, kp), torch.bfloat16)
    _dense(w_ot, "w_ot", (N, kp), torch.bfloat16)
    _dense(idx, "idx", (K,), torch.int32)
    _dense(count, "count", (1,), torch.int32)
    _check(lib().sq_gather_outliers(_ptr(x), _dtype(x), M, K, ldx, _ptr(w), _dtype(w), N, ldw, _ptr(idx),
                                    _ptr(count), kp, _ptr(x_o), _ptr(w_ot), _stream(_dev(x), stream)))


def sq_gemm_w8a8_outlier(xq: torch.Tensor, x_scale: torch.Tensor, wq: torch.Tensor, w_scale: torch.Tensor,
                         x_o: torch.Tensor, w_ot: torch.Tensor, count: torch.Tensor, y: torch.Tensor,
                         stream=None) -> None:
    """y [M, N] = dequant(Xq . Wq^T) (per-token x_scale) + x_o . w_ot^T over the count outlier channels."""
    M, K = xq.shape
    N = wq.shape[0]
    kp = x_o.shape[1]
    _dense(xq, "xq", (M, K), torch.int8)
    _dense(wq, "wq", (N, K), torch.int8)
    _dense(x_scale, "x_scale", (M,), torch.float32)
    _dense(w_scale, "w_scale", (N,), torch.float32)
    _dense(x_o, "x_o", (M, kp), torch.bfloat16)
    _dense(w_ot, "w_ot", (N, kp), torch.bfloat16)
    _dense(count, "count", (1,), torch.int32)
    if y.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError("y must be bfloat16 or float32")
    _dense(y, "y", (M, N), y.dtype)
    _check(lib().sq_gemm_w8a8_outlier(_ptr(xq), _ptr(x_scale), _ptr(wq), _ptr(w_scale), M, N, K, _ptr(x_o),
                                      _ptr(w_ot), kp, _ptr(count), _ptr(y), _dtype(y), _stream(_dev(xq), stream)))


# ---- alpha-search criterion ---------------------------------------------------------

def sq_matmul_f64(x: torch.Tensor, w: torch.Tensor, y_ref: torch.Tensor, stream=None) -> None:
    """y_ref [M, N] fp64 = x [M, K] . w [K, N] with every product and sum in fp64."""
    M, K, ldx = _rows(x)
    K2, N, ldw = _rows(w)
    if K2 != K:
        raise ValueError("x and w disagree on K")
    _dense(y_ref, "y_ref", (M, N), torch.float64)
    _check(lib().sq_matmul_f64(_ptr(x), _dtype(x), M, K, ldx, _ptr(w), _dtype(w), N, ldw, _ptr(y_ref),
                               _stream(_dev(x), stream)))


def sq_rel_error(y: torch.Tensor, y_ref: torch.Tensor, err: torch.Tensor, ws: torch.Tensor, stream=None) -> None:
    """err[0] = ||y - y_ref||_F / ||y_ref||_F in fp64 (y fp32 [M, N], y_ref fp64 [M, N])."""
    if y.dim() != 2:
        raise ValueError("y must be 2-D")
    M, N = y.shape
    _dense(y, "y", (M, N), torch.float32)
    _dense(y_ref, "y_ref", (M, N), torch.float64)
    _dense(err, "err", (1,), torch.float64)
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().sq_rel_error(_ptr(y), _ptr(y_ref), M, N, _ptr(err), _ptr(ws), nbytes, _stream(_dev(y), stream)))
