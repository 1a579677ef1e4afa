"""CPU oracle for the SmoothQuant W8A8 linear layer.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import this
package: only the tests, the smoke check and the benchmark's CPU-baseline leg
use it.  It shares no code with the HIP library.

Two halves:

* ``sq_oracle.c`` -- the five steps in fp32 with a fixed operation order
  (see the header of that file for the passages each step follows), wrapped
  here with ctypes over numpy arrays;
* fp64 helpers written here in numpy: the ideal smoothed product used for the
  equivalence identity (page "大模型训练、适配与推理" section 3.5 and page
  "4.2 W8A8 量化与 SmoothQuant" section 3: X diag(s)^-1 diag(s) W = X W in exact
  arithmetic) and the relative Frobenius error that reproduces the errors of
  the worked example on page "量化：只压权重，与训练后量化（PTQ）".

bf16 arrays are carried as ``numpy.uint16`` bit patterns.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "sq_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

F32, BF16 = 0, 1
PER_TOKEN, PER_TENSOR = 0, 1

CFLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared", "-pthread"]


def build() -> str:
    """Compile the C oracle (always recompiles)."""
    tmp = _LIB + ".tmp"
    cmd = ["gcc"] + CFLAGS + [_SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        L = ctypes.CDLL(_LIB)
        vp, i64, f32p = ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p
        L.sqo_calib_absmax.argtypes = [vp, ctypes.c_int, i64, i64, i64, f32p]
        L.sqo_weight_rowmax.argtypes = [vp, ctypes.c_int, i64, i64, i64, f32p]
        L.sqo_smooth_factors.argtypes = [f32p, f32p, i64, ctypes.c_float, f32p, f32p]
        L.sqo_quant_weight.argtypes = [vp, ctypes.c_int, i64, i64, i64, vp, vp, i64, f32p]
        L.sqo_quant_act.argtypes = [vp, ctypes.c_int, i64, i64, i64, vp, ctypes.c_int, vp, i64, f32p]
        L.sqo_static_act_max.argtypes = [vp, ctypes.c_int, i64, i64, i64, vp]
        L.sqo_static_act_max.restype = ctypes.c_float
        L.sqo_quant_act_static.argtypes = [vp, ctypes.c_int, i64, i64, i64, vp, ctypes.c_float, vp, i64, f32p]
        L.sqo_fold_layernorm.argtypes = [vp, vp, vp, i64, vp, vp]
        L.sqo_layernorm_quant.argtypes = [vp, i64, i64, i64, vp, vp, ctypes.c_float, vp, i64, f32p]
        L.sqo_gemm_i8.argtypes = [vp, i64, vp, i64, i64, i64, i64, vp, i64, ctypes.c_int]
        L.sqo_dequant.argtypes = [vp, i64, f32p, ctypes.c_int, f32p, i64, i64, vp, vp, i64]
        L.sqo_quant_sym.argtypes = [f32p, i64, ctypes.c_int, vp, f32p]
        L.sqo_outlier_columns.argtypes = [f32p, i64, ctypes.c_float, vp, vp]
        L.sqo_llm_int8.argtypes = [vp, i64, i64, i64, vp, i64, i64, vp, f32p, vp, i64, vp, f32p, vp, vp, vp]
        L.sqo_float_to_bf16.argtypes = [ctypes.c_float]
        L.sqo_float_to_bf16.restype = ctypes.c_uint16
        L.sqo_floats_to_bf16.argtypes = [vp, i64, vp]
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _dtype_code(a):
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:
        return BF16
    raise TypeError(f"oracle inputs are float32 or bf16 bit patterns (uint16), got {a.dtype}")


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"oracle {what} rejected its arguments (rc={rc})")


# ---- conversions ------------------------------------------------------------

def bf16_to_f32(h: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float32 (exact: the pattern is the top half)."""
    return (np.ascontiguousarray(h, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def f32_to_bf16(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns, round to nearest even (oracle's C routine)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    lib().sqo_floats_to_bf16(_p(x), x.size, _p(out))
    return out


def as_f32(x: np.ndarray) -> np.ndarray:
    return bf16_to_f32(x) if x.dtype == np.uint16 else np.asarray(x, dtype=np.float32)


# ---- the five steps ----------------------------------------------------------

def calib_absmax(x: np.ndarray, amax: np.ndarray | None = None) -> np.ndarray:
    """Step 1: running per-channel max|X| over the rows (tokens) of x[T, K]."""
    x = np.ascontiguousarray(x)
    T, K = x.shape
    out = np.zeros(K, np.float32) if amax is None else np.array(amax, dtype=np.float32, copy=True)
    _check(lib().sqo_calib_absmax(_p(x), _dtype_code(x), T, K, K, _p(out)), "calib_absmax")
    return out


def weight_rowmax(w: np.ndarray) -> np.ndarray:
    """Step 2a: amax_w[j] = max_k |W[j, k]| of w[K, N]."""
    w = np.ascontiguousarray(w)
    K, N = w.shape
    out = np.empty(K, np.float32)
    _check(lib().sqo_weight_rowmax(_p(w), _dtype_code(w), K, N, N, _p(out)), "weight_rowmax")
    return out


def smooth_factors(amax_x: np.ndarray, amax_w: np.ndarray, alpha: float):
    """Step 2b: (s, inv_s) in fp32 from the two channel maxima."""
    ax = np.ascontiguousarray(amax_x, dtype=np.float32)
    aw = np.ascontiguousarray(amax_w, dtype=np.float32)
    K = ax.size
    s = np.empty(K, np.float32)
    inv_s = np.empty(K, np.float32)
    _check(lib().sqo_smooth_factors(_p(ax), _p(aw), K, ctypes.c_float(alpha), _p(s), _p(inv_s)),
           "smooth_factors")
    return s, inv_s


def quant_weight(w: np.ndarray, s: np.ndarray | None):
    """Step 3: (wq[N, K] int8, w_scale[N] fp32) from w[K, N] and s[K] (or None)."""
    w = np.ascontiguousarray(w)
    K, N = w.shape
    sp = None if s is None else np.ascontiguousarray(s, dtype=np.float32)
    wq = np.empty((N, K), np.int8)
    ws = np.empty(N, np.float32)
    _check(lib().sqo_quant_weight(_p(w), _dtype_code(w), K, N, N, _p(sp), _p(wq), K, _p(ws)),
           "quant_weight")
    return wq, ws


def quant_act(x: np.ndarray, inv_s: np.ndarray | None, gran: int = PER_TOKEN):
    """Step 4: (xq[M, K] int8, x_scale[M] or [1] fp32) from x[M, K] and inv_s[K] (or None)."""
    x = np.ascontiguousarray(x)
    M, K = x.shape
    ip = None if inv_s is None else np.ascontiguousarray(inv_s, dtype=np.float32)
    xq = np.empty((M, K), np.int8)
    xs = np.empty(1 if gran == PER_TENSOR else M, np.float32)
    _check(lib().sqo_quant_act(_p(x), _dtype_code(x), M, K, K, _p(ip), gran, _p(xq), K, _p(xs)),
           "quant_act")
    return xq, xs


def static_act_max(calib: np.ndarray, inv_s: np.ndarray | None) -> np.float32:
    """Calibrated per-tensor maximum: max over the calibration tokens of |X'| (fp32)."""
    calib = np.ascontiguousarray(calib)
    T, K = calib.shape
    ip = None if inv_s is None else np.ascontiguousarray(inv_s, dtype=np.float32)
    return np.float32(lib().sqo_static_act_max(_p(calib), _dtype_code(calib), T, K, K, _p(ip)))


def quant_act_static(x: np.ndarray, inv_s: np.ndarray | None, a: float):
    """Per-tensor codes of X' with the fixed (calibrated) maximum a: (xq[M, K], x_scale[1])."""
    x = np.ascontiguousarray(x)
    M, K = x.shape
    ip = None if inv_s is None else np.ascontiguousarray(inv_s, dtype=np.float32)
    xq = np.empty((M, K), np.int8)
    xs = np.empty(1, np.float32)
    _check(lib().sqo_quant_act_static(_p(x), _dtype_code(x), M, K, K, _p(ip), ctypes.c_float(float(a)), _p(xq),
                                      K, _p(xs)), "quant_act_static")
    return xq, xs


def fold_layernorm(gamma: np.ndarray, beta: np.ndarray | None, inv_s: np.ndarray):
    """(gamma', beta') = (fl(gamma * inv_s), fl(beta * inv_s)); beta' is None without a bias."""
    g = np.ascontiguousarray(gamma, dtype=np.float32)
    b = None if beta is None else np.ascontiguousarray(beta, dtype=np.float32)
    i = np.ascontiguousarray(inv_s, dtype=np.float32)
    K = g.size
    go = np.empty(K, np.float32)
    bo = None if b is None else np.empty(K, np.float32)
    _check(lib().sqo_fold_layernorm(_p(g), _p(b), _p(i), K, _p(go), _p(bo)), "fold_layernorm")
    return go, bo


def layernorm_quant(x_bf16: np.ndarray, gamma: np.ndarray, beta: np.ndarray | None, eps: float):
    """The library's arithmetic contract for LayerNorm + per-token INT8: the row
    statistics on a fixed-point grid (order-free exact sums), then fp32
    normalisation (see sqo_layernorm_quant in sq_oracle.c).  It is the bit-exact
    reference of the kernel; layernorm_quant_plain is the definition it is
    held to.  Returns (xq[M, K], x_scale[M])."""
    x = np.ascontiguousarray(x_bf16)
    if x.dtype != np.uint16:
        raise TypeError("layernorm_quant takes bf16 bit patterns (uint16)")
    M, K = x.shape
    g = np.ascontiguousarray(gamma, dtype=np.float32)
    b = None if beta is None else np.ascontiguousarray(beta, dtype=np.float32)
    xq = np.empty((M, K), np.int8)
    xs = np.empty(M, np.float32)
    _check(lib().sqo_layernorm_quant(_p(x), M, K, K, _p(g), _p(b), ctypes.c_float(eps), _p(xq), K, _p(xs)),
           "layernorm_quant")
    return xq, xs


def layernorm_quant_plain(x_bf16: np.ndarray, gamma: np.ndarray, beta: np.ndarray | None, eps: float):
    """LayerNorm of each bf16 row, then per-token symmetric INT8, straight from
    the definition in fp64 with no fp32 rounding anywhere (page "4.2 W8A8 量化与
    SmoothQuant" section 6: LN(x)_j / s_j = (x_j - mu) / sigma * gamma_j / s_j +
    beta_j / s_j; gamma and beta here are the folded gamma / s and beta / s):

      mu = (sum_j x_j) / K,   var = (sum_j (x_j - mu)^2) / K   (biased),
      sigma = sqrt(var + eps),  z_j = (x_j - mu) / sigma * gamma_j + beta_j,
      m = max_j |z_j|,  scale = m / 127,  q_j = z_j * 127 / m,
      code_j = clip(round_half_even(q_j), -127, 127)   (all 0 when m = 0).

    The sums are taken with math.fsum (correctly rounded), so mu is the fp64
    rounding of the exact mean.  eps enters as the fp64 value of the fp32 eps
    the library takes.  Returns a dict: codes int8 [M, K], scale, mu, var, m
    (fp64 [M]) and z, q (fp64 [M, K], the values before rounding)."""
    import math

    x = np.ascontiguousarray(x_bf16)
    if x.dtype != np.uint16:
        raise TypeError("layernorm_quant_plain takes bf16 bit patterns (uint16)")
    M, K = x.shape
    xf = bf16_to_f32(x).astype(np.float64)
    g = np.asarray(gamma, dtype=np.float32).astype(np.float64)
    b = None if beta is None else np.asarray(beta, dtype=np.float32).astype(np.float64)
    e = float(np.float32(eps))
    mu = np.empty(M)
    var = np.empty(M)
    for i in range(M):
        mu[i] = math.fsum(xf[i].tolist()) / K
        d = xf[i] - mu[i]
        var[i] = math.fsum((d * d).tolist()) / K
    z = (xf - mu[:, None]) / np.sqrt(var + e)[:, None] * g[None, :]
    if b is not None:
        z = z + b[None, :]
    m = np.abs(z).max(axis=1)
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.where(m[:, None] > 0, z * (127.0 / np.where(m > 0, m, 1.0))[:, None], 0.0)
    codes = np.clip(np.rint(q), -127, 127).astype(np.int8)
    return dict(codes=codes, scale=m / 127.0, mu=mu, var=var, m=m, z=z, q=q)


def gemm_i8(xq: np.ndarray, wq: np.ndarray, nthreads: int = 1) -> np.ndarray:
    """Step 5a: acc[M, N] = Xq[M, K] . Wq[N, K]^T in int32."""
    xq = np.ascontiguousarray(xq, dtype=np.int8)
    wq = np.ascontiguousarray(wq, dtype=np.int8)
    M, K = xq.shape
    N, K2 = wq.shape
    if K != K2:
        raise ValueError("reduction sizes differ")
    acc = np.empty((M, N), np.int32)
    _check(lib().sqo_gemm_i8(_p(xq), K, _p(wq), K, M, N, K, _p(acc), N, int(nthreads)), "gemm_i8")
    return acc


def dequant(acc: np.ndarray, x_scale: np.ndarray, gran: int, w_scale: np.ndarray):
    """Step 5b: (y fp32[M, N], y bf16 bits[M, N]) = acc * x_scale_i * w_scale_k."""
    acc = np.ascontiguousarray(acc, dtype=np.int32)
    M, N = acc.shape
    xs = np.ascontiguousarray(x_scale, dtype=np.float32)
    ws = np.ascontiguousarray(w_scale, dtype=np.float32)
    y32 = np.empty((M, N), np.float32)
    ybf = np.empty((M, N), np.uint16)
    _check(lib().sqo_dequant(_p(acc), N, _p(xs), gran, _p(ws), M, N, _p(y32), _p(ybf), N), "dequant")
    return y32, ybf


def quant_sym(x: np.ndarray, bits: int):
    """Generic symmetric quantizer of one group: (codes int8, scale fp32)."""
    x = np.ascontiguousarray(x, dtype=np.float32).reshape(-1)
    codes = np.empty(x.size, np.int8)
    scale = np.zeros(1, np.float32)
    _check(lib().sqo_quant_sym(_p(x), x.size, bits, _p(codes), _p(scale)), "quant_sym")
    return codes, float(scale[0])


def w8a8_linear(x, w, alpha: float | None, gran: int = PER_TOKEN, calib=None, nthreads: int = 1):
    """All five steps in order.  alpha=None runs the unsmoothed baseline.

    Returns a dict with every intermediate (amax_x, amax_w, s, inv_s, wq, w_scale,
    xq, x_scale, acc, y32, ybf16)."""
    out = {}
    if alpha is not None:
        calib_src = x if calib is None else calib
        if isinstance(calib_src, (list, tuple)):
            amax = None
            for chunk in calib_src:
                amax = calib_absmax(chunk, amax)
        else:
            amax = calib_absmax(calib_src)
        aw = weight_rowmax(w)
        s, inv_s = smooth_factors(amax, aw, alpha)
        out.update(amax_x=amax, amax_w=aw, s=s, inv_s=inv_s)
    else:
        s = inv_s = None
    wq, ws = quant_weight(w, s)
    xq, xs = quant_act(x, inv_s, gran)
    acc = gemm_i8(xq, wq, nthreads)
    y32, ybf = dequant(acc, xs, gran, ws)
    out.update(wq=wq, w_scale=ws, xq=xq, x_scale=xs, acc=acc, y32=y32, ybf16=ybf)
    return out


def search_alpha(x, w, calib, alphas, gran: int = PER_TOKEN, nthreads: int = 8):
    """Offline migration-strength search (page "4.2 W8A8 量化与 SmoothQuant" 5.2: a
    grid search over alpha on calibration data): for each alpha the W8A8 output
    (fp32, before the bf16 rounding) of the sample x against X W in fp64, by
    relative Frobenius error.  Returns (best alpha, {alpha: error}); ties go to
    the first alpha of the grid."""
    y = matmul_f64(x, w)
    errs = {}
    for a in alphas:
        errs[float(a)] = rel_fro(w8a8_linear(x, w, float(a), gran, calib=calib, nthreads=nthreads)["y32"], y)
    best = min(errs, key=lambda a: (errs[a], list(errs).index(a)))
    return best, errs


# ---- LLM.int8()-style decomposition (comparator) -------------------------------

def outlier_columns(amax_x: np.ndarray, threshold: float):
    """Outlier input channels (page "4.2 W8A8 量化与 SmoothQuant" section 2; page
    "量化：只压权重，与训练后量化（PTQ）", SmoothQuant W8A8 results): the channels whose
    max |x| strictly exceeds the threshold.  Returns (idx int32 ascending,
    keep float32 with 0 on outlier channels and 1 elsewhere)."""
    a = np.ascontiguousarray(amax_x, dtype=np.float32)
    K = a.size
    idx = np.empty(max(K, 1), np.int32)
    keep = np.empty(K, np.float32)
    n = lib().sqo_outlier_columns(_p(a), K, ctypes.c_float(threshold), _p(idx), _p(keep))
    if n < 0:
        raise ValueError("oracle outlier_columns rejected its arguments")
    return idx[:n].copy(), keep


def llm_int8(x_bf16: np.ndarray, w_bf16: np.ndarray, wq: np.ndarray, w_scale: np.ndarray, threshold: float,
             amax_x: np.ndarray | None = None, rows=None):
    """The mixed-precision product of the bf16 activation x[M, K] and weight
    w[K, N]: outlier channels (from amax_x, the channel maxima of the whole x,
    computed here when None) in 16 bits, the rest in INT8 per token with the
    offline weight codes wq[N, K] / w_scale[N] of W itself.  rows selects the
    token rows to evaluate (all when None).  Returns a dict with idx, xq,
    x_scale, y32, ybf16 and bound (sum of |x w| over the outlier channels)."""
    x = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    w = np.ascontiguousarray(w_bf16, dtype=np.uint16)
    M, K = x.shape
    K2, N = w.shape
    if K != K2:
        raise ValueError("reduction sizes differ")
    if amax_x is None:
        amax_x = calib_absmax(x)
    idx, keep = outlier_columns(amax_x, threshold)
    xr = x if rows is None else np.ascontiguousarray(x[np.asarray(rows)])
    R = xr.shape[0]
    wq = np.ascontiguousarray(wq, dtype=np.int8)
    ws = np.ascontiguousarray(w_scale, dtype=np.float32)
    xq = np.empty((R, K), np.int8)
    xs = np.empty(R, np.float32)
    y32 = np.empty((R, N), np.float32)
    ybf = np.empty((R, N), np.uint16)
    bound = np.empty((R, N), np.float64)
    _check(lib().sqo_llm_int8(_p(xr), R, K, K, _p(w), N, N, _p(wq), _p(ws), _p(idx), idx.size, _p(xq), _p(xs),
                              _p(y32), _p(ybf), _p(bound)), "llm_int8")
    return dict(idx=idx, keep=keep, xq=xq, x_scale=xs, y32=y32, ybf16=ybf, bound=bound)


# ---- fp64 ideal path -----------------------------------------------------------

def matmul_f64(x, w) -> np.ndarray:
    """Y_ref = X W accumulated in fp64 from the same (fp32 / bf16) inputs."""
    return as_f32(x).astype(np.float64) @ as_f32(w).astype(np.float64)


def smoothed_product_f64(x, w, s) -> np.ndarray:
    """(X diag(s)^-1)(diag(s) W) in fp64, with no fp32 rounding anywhere."""
    s64 = np.asarray(s, dtype=np.float64)
    xs = as_f32(x).astype(np.float64) / s64[None, :]
    ws = s64[:, None] * as_f32(w).astype(np.float64)
    return xs @ ws


def smooth_factors_f64(amax_x, amax_w, alpha: float) -> np.ndarray:
    """s_j = max|X_j|^alpha / max|W_j|^(1-alpha) in fp64 (no floor, no rounding)."""
    ax = np.asarray(amax_x, dtype=np.float64)
    aw = np.asarray(amax_w, dtype=np.float64)
    return ax ** alpha / aw ** (1.0 - alpha)


def rel_fro(y_hat, y_ref) -> float:
    """Relative Frobenius error ||Y_hat - Y_ref||_F / ||Y_ref||_F (in fp64)."""
    d = np.asarray(y_hat, dtype=np.float64) - np.asarray(y_ref, dtype=np.float64)
    return float(np.linalg.norm(d) / np.linalg.norm(np.asarray(y_ref, dtype=np.float64)))
