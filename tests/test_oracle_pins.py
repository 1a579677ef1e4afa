"""Pins of the CPU oracle to facts outside itself.

Each test checks the oracle against something the pages print, a closed form,
an invariant, a library routine or brute force -- never against a retyped copy
of its own formula.  Together they are chosen so that a dropped term, a wrong
sign, a wrong axis or a transposed operand anywhere in the five steps fails at
least one of them.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def _round_sig(x, sig):
    return float(f"{x:.{sig}g}")


# ---- the worked example on page "量化：只压权重，与训练后量化（PTQ）" -------------

@pytest.fixture(scope="module")
def worked():
    g = _gold("worked_example.json")
    X = np.array(g["X"], np.float32)
    W = np.array(g["W"], np.float32)
    return g, X, W


def test_worked_example_maxima_and_s(worked):
    g, X, W = worked
    ax = oracle.calib_absmax(X)
    aw = oracle.weight_rowmax(W)
    np.testing.assert_array_equal(ax, np.array(g["amax_x"], np.float32))
    np.testing.assert_array_equal(aw, np.array(g["amax_w"], np.float32))
    s, inv_s = oracle.smooth_factors(ax, aw, g["alpha"])
    got = [_round_sig(v, g["s"]["sig_digits"]) for v in s]
    assert got == g["s"]["values"]
    # After smoothing, channel j of X' and row j of W' share the max sqrt(ax*aw).
    xp = X * inv_s[None, :]
    wp = s[:, None] * W
    xmax = np.abs(xp).max(axis=0)
    wmax = np.abs(wp).max(axis=1)
    d = g["smoothed_channel_max"]["decimals"]
    assert [round(float(v), d) for v in xmax] == g["smoothed_channel_max"]["values"]
    assert [round(float(v), d) for v in wmax] == g["smoothed_channel_max"]["values"]


def test_worked_example_steps_and_codes(worked):
    g, X, W = worked
    xq0, xs0 = oracle.quant_act(X, None, oracle.PER_TENSOR)
    ax = oracle.calib_absmax(X)
    s, inv_s = oracle.smooth_factors(ax, oracle.weight_rowmax(W), g["alpha"])
    xq1, xs1 = oracle.quant_act(X, inv_s, oracle.PER_TENSOR)
    st = g["per_tensor_step"]
    assert round(float(xs0[0]), st["before_decimals"]) == st["before"]
    assert round(float(xs1[0]), st["after_decimals"]) == st["after"]
    assert xq0[:, 0].tolist() == g["channel1_codes"]["before"]
    assert xq1[:, 0].tolist() == g["channel1_codes"]["after"]


@pytest.mark.parametrize("gran,key", [(oracle.PER_TENSOR, "per_tensor_act_per_channel_w"),
                                      (oracle.PER_TOKEN, "per_token_act_per_channel_w")])
def test_worked_example_relative_errors(worked, gran, key):
    """The four printed errors pin: per-output-channel weight scales, the
    activation granularity, the smoothing direction, the dequant epilogue and
    the relative Frobenius metric all at once (other readings give other
    numbers)."""
    g, X, W = worked
    e = g["relative_error_percent"][key]
    Y = oracle.matmul_f64(X, W)
    base = oracle.w8a8_linear(X, W, None, gran)
    smooth = oracle.w8a8_linear(X, W, g["alpha"], gran)
    assert round(100 * oracle.rel_fro(base["y32"], Y), e["before_decimals"]) == e["before"]
    assert round(100 * oracle.rel_fro(smooth["y32"], Y), e["after_decimals"]) == e["after"]


# ---- printed constants ---------------------------------------------------------

def test_per_tensor_outlier_step_and_levels():
    """Page "4.2 W8A8 量化与 SmoothQuant" section 1.2: one channel at 100, the
    others within 1 -> step 100/127 ~ 0.79 and only 2-3 usable levels
    (2^8 * m_i / m ~ 2.56) for the small channels."""
    c = _gold("printed_constants.json")["per_tensor_outlier_step"]
    rng = np.random.default_rng(7)
    X = rng.uniform(-1, 1, size=(256, 8)).astype(np.float32)
    X[:, 3] = rng.uniform(-c["channel_max"], c["channel_max"], size=256).astype(np.float32)
    X[0, 3] = c["channel_max"]
    X[1, 0], X[2, 0] = 1.0, -1.0
    xq, xs = oracle.quant_act(X, None, oracle.PER_TENSOR)
    assert round(float(xs[0]), c["step_decimals"]) == c["step"]
    levels = 2 ** 8 * c["other_channel_max"] / c["channel_max"]
    assert 2 <= levels <= 3
    small = np.delete(xq, 3, axis=1)
    distinct = np.unique(small)
    assert set(distinct.tolist()) <= {-1, 0, 1}
    assert len(distinct) == 3  # three codes: 2-3 levels as printed
    assert xq[0, 3] == 127


def test_int4_outlier_row():
    """Page "GBDQ权重与平滑激活量化": 4-bit symmetric scale of the printed row
    is 89.4/7 ~ 12.8 and every small value codes to 0."""
    c = _gold("printed_constants.json")["int4_outlier_row"]
    codes, scale = oracle.quant_sym(np.array(c["row"], np.float32), c["bits"])
    assert round(scale, c["scale_decimals"]) == c["scale"]
    big = int(np.argmax(np.abs(c["row"])))
    assert codes[big] == c["qmax"]
    assert all(v == c["codes_small_values"] for i, v in enumerate(codes) if i != big)


# ---- closed forms of the smoothing factor ----------------------------------------

def _maxima(K, seed):
    rng = np.random.default_rng(seed)
    ax = rng.uniform(0.05, 200.0, K).astype(np.float32)
    aw = rng.uniform(0.001, 0.2, K).astype(np.float32)
    return ax, aw


def test_alpha_zero_closed_form():
    """alpha = 0: s_j = 1 / max|W_j| (page "4.2 ..." section 4), and then every
    smoothed weight row has max 1 (up to one fp32 rounding)."""
    ax, aw = _maxima(513, 1)
    s, inv_s = oracle.smooth_factors(ax, aw, 0.0)
    expect = np.array([float(Fraction(1) / Fraction(float(b))) for b in aw], np.float64).astype(np.float32)
    np.testing.assert_array_equal(s, expect)
    W = np.random.default_rng(2).normal(0, 0.05, (513, 33)).astype(np.float32)
    aw2 = oracle.weight_rowmax(W)
    s2, _ = oracle.smooth_factors(ax, aw2, 0.0)
    rowmax = np.abs(s2[:, None] * W).max(axis=1)
    np.testing.assert_allclose(rowmax, 1.0, rtol=2 ** -23, atol=0)


def test_alpha_one_closed_form():
    """alpha = 1: s_j = max|X_j| (page "4.2 ..." section 4), and then every
    smoothed activation channel has max 1 (reciprocal form: within 1 ulp)."""
    ax, aw = _maxima(513, 3)
    s, inv_s = oracle.smooth_factors(ax, aw, 1.0)
    np.testing.assert_array_equal(s, ax)
    X = np.random.default_rng(4).normal(0, 3, (64, 513)).astype(np.float32)
    ax2 = oracle.calib_absmax(X)
    _, inv2 = oracle.smooth_factors(ax2, aw, 1.0)
    colmax = np.abs(X * inv2[None, :]).max(axis=0)
    np.testing.assert_allclose(colmax, 1.0, rtol=2.5 * 2 ** -23, atol=0)


def test_alpha_half_is_sqrt_ratio():
    """alpha = 0.5 is the square root of the ratio of the maxima (page
    "SmoothQuant大模型平滑量化技术", scale derivation): compare with the exactly
    rounded sqrt of the exact rational ratio."""
    ax, aw = _maxima(257, 5)
    s, _ = oracle.smooth_factors(ax, aw, 0.5)
    ratio = ax.astype(np.float64) / aw.astype(np.float64)
    np.testing.assert_allclose(s, np.sqrt(ratio), rtol=2 ** -23)


@pytest.mark.parametrize("alpha", [0.25, 0.4, 0.5, 0.6, 0.75, 0.9])
def test_general_alpha_balance_invariant(alpha):
    """Derived from the scale formula: after smoothing, channel j of X' has max
    (ax_j aw_j)^(1-alpha) and row j of W' has max (ax_j aw_j)^alpha."""
    rng = np.random.default_rng(11)
    X = rng.normal(0, 1, (128, 96)).astype(np.float32)
    X[:, [5, 40]] *= 80.0
    W = rng.normal(0, 0.02, (96, 48)).astype(np.float32)
    ax, aw = oracle.calib_absmax(X), oracle.weight_rowmax(W)
    s, inv_s = oracle.smooth_factors(ax, aw, alpha)
    xmax = np.abs(X * inv_s[None, :]).max(axis=0).astype(np.float64)
    wmax = np.abs(s[:, None] * W).max(axis=1).astype(np.float64)
    p = ax.astype(np.float64) * aw.astype(np.float64)
    np.testing.assert_allclose(xmax, p ** (1 - alpha), rtol=4e-7)
    np.testing.assert_allclose(wmax, p ** alpha, rtol=4e-7)
    np.testing.assert_allclose(s, oracle.smooth_factors_f64(ax, aw, alpha), rtol=2 ** -23)


def test_floor_on_dead_channels():
    ax = np.array([0.0, 1.0, 0.0], np.float32)
    aw = np.array([0.5, 0.0, 0.0], np.float32)
    s, inv_s = oracle.smooth_factors(ax, aw, 0.5)
    assert np.all(np.isfinite(s)) and np.all(np.isfinite(inv_s)) and np.all(s > 0)


# ---- exact identity (fp64) --------------------------------------------------------

@pytest.mark.parametrize("cfg", synth.ALL)
def test_equivalence_identity_fp64(cfg):
    """X diag(s)^-1 diag(s) W = X W (page "大模型训练、适配与推理" section 3.5):
    in fp64 the two products agree to rounding, rel err <= 1e-12, on each
    configuration's recipe (reduced sizes)."""
    inp = synth.make(cfg, M=48, K=192, N=40, calib_chunks=2 if synth.CONFIGS[cfg].calib_chunks else 0,
                     chunk_tokens=64)
    x, w = synth.to_numpy(inp.x), synth.to_numpy(inp.w)
    ax = oracle.calib_absmax(synth.to_numpy(inp.calib))
    for a in synth.CONFIGS[cfg].alphas:
        s, _ = oracle.smooth_factors(ax, oracle.weight_rowmax(w), a)
        y = oracle.matmul_f64(x, w)
        ys = oracle.smoothed_product_f64(x, w, s)
        assert oracle.rel_fro(ys, y) <= 1e-12


# ---- quantizer properties -----------------------------------------------------------

def test_round_half_to_even():
    """Ties go to the even code (numpy rounding in the demo of page
    "SmoothQuant大模型平滑量化技术"); with row max 127 the multiplier is exactly 1."""
    X = np.array([[127.0, 2.5, 3.5, -2.5, 0.5, 1.5, -0.5, 126.5, 4.5, 0.0, 0.0, 0.0]], np.float32)
    xq, xs = oracle.quant_act(X, None, oracle.PER_TOKEN)
    assert xs[0] == np.float32(1.0)
    assert xq[0].tolist() == [127, 2, 4, -2, 0, 2, 0, 126, 4, 0, 0, 0]


def test_quantizer_properties():
    rng = np.random.default_rng(3)
    X = (rng.standard_t(4, (37, 200)) * rng.uniform(0.01, 50, (37, 1))).astype(np.float32)
    X[5] = 0.0
    xq, xs = oracle.quant_act(X, None, oracle.PER_TOKEN)
    xqn, xsn = oracle.quant_act(-X, None, oracle.PER_TOKEN)
    np.testing.assert_array_equal(xqn, -xq)        # odd symmetry
    np.testing.assert_array_equal(xsn, xs)
    assert xs[5] == 0 and not xq[5].any()            # all-zero token
    nz = np.arange(37) != 5
    assert (np.abs(xq[nz]).max(axis=1) == 127).all()  # row max maps to +-127
    assert xq.min() >= -127
    # reconstruction error at most half a step (plus fp32 rounding slack)
    err = np.abs(xq.astype(np.float64) * xs[:, None] - X)
    assert (err <= 0.5 * xs[:, None].astype(np.float64) * (1 + 1e-5) + 1e-30).all()


def test_reciprocal_vs_division_rarely_differ():
    """The fp32 reciprocal-multiply realisation of x / scale agrees with the
    exact rounding of x * 127 / a except at rare rounding boundaries."""
    rng = np.random.default_rng(9)
    X = rng.normal(0, 1, (512, 1024)).astype(np.float32)
    xq, xs = oracle.quant_act(X, None, oracle.PER_TOKEN)
    a = np.abs(X).max(axis=1).astype(np.float64)
    exact = np.clip(np.rint(X.astype(np.float64) * 127.0 / a[:, None]), -127, 127)
    frac = float((exact != xq).mean())
    assert frac < 1e-4
    assert np.abs(exact - xq).max() <= 1


def test_weight_codes_are_per_output_channel_and_transposed():
    rng = np.random.default_rng(5)
    W = rng.normal(0, 0.02, (64, 24)).astype(np.float32)
    W[:, 7] *= 30.0           # one loud output column
    s = rng.uniform(0.5, 2.0, 64).astype(np.float32)
    wq, ws = oracle.quant_weight(W, s)
    assert wq.shape == (24, 64)
    wp = s[:, None] * W
    np.testing.assert_allclose(ws, np.abs(wp).max(axis=0) / 127.0, rtol=2 ** -23)
    assert (np.abs(wq).max(axis=1) == 127).all()
    # dequantized weights reproduce W' to half a step per output channel
    err = np.abs(wq.T.astype(np.float64) * ws[None, :] - wp)
    assert (err <= 0.5 * ws[None, :] * (1 + 1e-5)).all()


# ---- integer GEMM by brute force -------------------------------------------------

@pytest.mark.parametrize("M,N,K", [(1, 1, 1), (5, 7, 37), (9, 3, 64), (4, 6, 130)])
def test_gemm_brute_force(M, N, K):
    rng = np.random.default_rng(M * 100 + N * 10 + K)
    xq = rng.integers(-127, 128, (M, K), dtype=np.int64).astype(np.int8)
    wq = rng.integers(-127, 128, (N, K), dtype=np.int64).astype(np.int8)
    xq[0, :] = 127
    wq[0, :] = -127
    acc = oracle.gemm_i8(xq, wq, nthreads=3)
    X = xq.tolist()
    Wl = wq.tolist()
    for i in range(M):
        for k in range(N):
            assert acc[i, k] == sum(X[i][j] * Wl[k][j] for j in range(K))


def test_gemm_extreme_accumulator():
    K = 12288
    xq = np.full((2, K), 127, np.int8)
    wq = np.full((3, K), -127, np.int8)
    xq[1] = -127
    acc = oracle.gemm_i8(xq, wq, nthreads=2)
    assert acc[0, 0] == -K * 127 * 127 and acc[1, 2] == K * 127 * 127


# ---- dequant and bf16 --------------------------------------------------------------

def test_dequant_indices_exact():
    """With power-of-two scales every product is exact, so y[i, k] must equal
    acc[i, k] * 2^-i * 2^-2k exactly: pins which scale goes with which axis."""
    M, N = 6, 5
    rng = np.random.default_rng(1)
    acc = rng.integers(-(2 ** 20), 2 ** 20, (M, N)).astype(np.int32)
    xs = np.array([2.0 ** -i for i in range(M)], np.float32)
    ws = np.array([2.0 ** (-2 * k) for k in range(N)], np.float32)
    y32, ybf = oracle.dequant(acc, xs, oracle.PER_TOKEN, ws)
    for i in range(M):
        for k in range(N):
            assert Fraction(float(y32[i, k])) == Fraction(int(acc[i, k])) * Fraction(1, 2 ** (i + 2 * k))
    y32t, _ = oracle.dequant(acc, xs[:1], oracle.PER_TENSOR, ws)
    np.testing.assert_array_equal(y32t[0], y32[0])


def test_bf16_rounding_matches_torch():
    """fp32 -> bf16 round to nearest even agrees with torch's conversion on
    ties, near-ties, subnormals and large values."""
    rng = np.random.default_rng(0)
    base = rng.normal(0, 1, 4000).astype(np.float32)
    u = base.view(np.uint32)
    ties = ((u & 0xFFFF0000) | 0x8000).view(np.float32)
    near = ((u & 0xFFFF0000) | 0x7FFF).view(np.float32)
    odd_ties = ((u | 0x00010000) & 0xFFFF0000 | 0x8000).view(np.float32)
    special = np.array([0.0, -0.0, 1e-40, -3e-39, 3.0e38, 1.0, 1.00390625, 1.01171875], np.float32)
    x = np.concatenate([base, ties, near, odd_ties, special])
    ours = oracle.f32_to_bf16(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)


# ---- calibration resume and the direction of the effect ----------------------------

def test_calibration_chunked_equals_single_pass():
    inp = synth.make(synth.ATTN_PROJ, M=16, K=256, N=8, calib_chunks=6, chunk_tokens=40)
    c = synth.to_numpy(inp.calib)
    whole = oracle.calib_absmax(c)
    amax = None
    for part in np.array_split(c, 5):
        amax = oracle.calib_absmax(part, amax)
    np.testing.assert_array_equal(whole, amax)
    # resuming twice over the same data changes nothing (max is idempotent)
    np.testing.assert_array_equal(oracle.calib_absmax(c, whole), whole)
    # and matches numpy's reduction
    np.testing.assert_array_equal(whole, np.abs(oracle.bf16_to_f32(c)).max(axis=0))


@pytest.mark.parametrize("cfg", [synth.TINY, synth.ATTN_PROJ, synth.LARGE])
def test_smoothing_reduces_error_on_outliers(cfg):
    """On outlier-bearing inputs the smoothed W8A8 output is closer to X W than
    plain per-tensor W8A8 (direction given by the accuracy table of page
    "4.2 W8A8 量化与 SmoothQuant" section 7.2 and the worked example)."""
    c = synth.CONFIGS[cfg]
    inp = synth.make(cfg, M=64, K=256, N=64, calib_chunks=2 if c.calib_chunks else 0, chunk_tokens=128)
    x, w = synth.to_numpy(inp.x), synth.to_numpy(inp.w)
    cal = synth.to_numpy(inp.calib)
    y = oracle.matmul_f64(x, w)
    gran = oracle.PER_TENSOR if c.gran == "per_tensor" else oracle.PER_TOKEN
    base = oracle.rel_fro(oracle.w8a8_linear(x, w, None, oracle.PER_TENSOR)["y32"], y)
    for a in c.alphas:
        sm = oracle.rel_fro(oracle.w8a8_linear(x, w, a, gran, calib=cal)["y32"], y)
        assert sm < base


def test_tiny_group_where_multiplier_overflows():
    """A group whose max is below 127/FLT_MAX: the multiplier is +inf, zero
    elements code to 0 and non-zero ones saturate with their sign."""
    X = np.zeros((1, 16), np.float32)
    X[0, :4] = [1e-38, -5e-39, 0.0, 2e-45]
    xq, xs = oracle.quant_act(X, None, oracle.PER_TOKEN)
    assert xq[0, :4].tolist() == [127, -127, 0, 127]
    assert not xq[0, 4:].any()
    assert xs[0] == np.float32(np.float32(1e-38) / np.float32(127.0))


# ---- static per-tensor activation scale (page "4.2 W8A8 量化与 SmoothQuant" 7.1) ----

def _static_w8a8(X, W, alpha, calib):
    """The W8A8 path with the per-tensor activation scale fixed by calibration."""
    s = inv_s = None
    if alpha is not None:
        s, inv_s = oracle.smooth_factors(oracle.calib_absmax(calib), oracle.weight_rowmax(W), alpha)
    a = oracle.static_act_max(calib, inv_s)
    wq, ws = oracle.quant_weight(W, s)
    xq, xs = oracle.quant_act_static(X, inv_s, a)
    y32, _ = oracle.dequant(oracle.gemm_i8(xq, wq), xs, oracle.PER_TENSOR, ws)
    return a, xq, xs, y32


def test_static_scale_worked_example_errors(worked):
    """Calibrating on X itself (as the worked example does), the static
    per-tensor scale is the example's per-tensor scale: its two printed errors
    (1.95 % unsmoothed, 0.15 % smoothed) and its steps 0.378 -> 0.0244 come out."""
    g, X, W = worked
    e = g["relative_error_percent"]["per_tensor_act_per_channel_w"]
    st = g["per_tensor_step"]
    Y = oracle.matmul_f64(X, W)
    a0, _, xs0, y0 = _static_w8a8(X, W, None, X)
    a1, xq1, xs1, y1 = _static_w8a8(X, W, g["alpha"], X)
    assert a0 == np.float32(48.0)
    assert round(float(xs0[0]), st["before_decimals"]) == st["before"]
    assert round(float(xs1[0]), st["after_decimals"]) == st["after"]
    assert xq1[:, 0].tolist() == g["channel1_codes"]["after"]
    assert round(100 * oracle.rel_fro(y0, Y), e["before_decimals"]) == e["before"]
    assert round(100 * oracle.rel_fro(y1, Y), e["after_decimals"]) == e["after"]


def test_static_scale_clips_beyond_calibrated_range():
    """Run-time values beyond the calibrated maximum saturate at +-127; the
    scale does not move; values inside the range code as with a dynamic
    per-tensor scale whose maximum is the calibrated one."""
    rng = np.random.default_rng(11)
    K = 64
    calib = rng.standard_normal((32, K)).astype(np.float32)
    inv_s = (0.5 + rng.random(K)).astype(np.float32)
    a = oracle.static_act_max(calib, inv_s)
    assert a == np.float32(np.abs(calib * inv_s[None, :]).max())
    x = rng.standard_normal((4, K)).astype(np.float32)
    x[1, 3] = 3.0 * a / inv_s[3]      # three times the calibrated range
    x[2, 7] = -5.0 * a / inv_s[7]
    xq, xs = oracle.quant_act_static(x, inv_s, a)
    assert xs[0] == np.float32(a / np.float32(127.0))
    assert xq[1, 3] == 127 and xq[2, 7] == -127
    # inside the range: the same codes as a per-tensor quantization whose maximum is a
    r = np.float32(127.0) / a
    xp = (x * inv_s[None, :]).astype(np.float32)
    inside = np.abs(xp) <= a
    ref = np.clip(np.rint((xp * r).astype(np.float32)), -127, 127).astype(np.int8)
    np.testing.assert_array_equal(xq[inside], ref[inside])


def test_static_scale_equals_dynamic_on_its_own_calibration():
    """Quantizing the calibration tensor itself with its static scale gives the
    dynamic per-tensor result bit for bit."""
    rng = np.random.default_rng(12)
    calib = (rng.standard_normal((48, 96)) * np.where(rng.random(96) < 0.05, 80.0, 1.0)).astype(np.float32)
    inv_s = (1.0 / (0.3 + rng.random(96))).astype(np.float32)
    a = oracle.static_act_max(calib, inv_s)
    xq_s, xs_s = oracle.quant_act_static(calib, inv_s, a)
    xq_d, xs_d = oracle.quant_act(calib, inv_s, oracle.PER_TENSOR)
    np.testing.assert_array_equal(xq_s, xq_d)
    np.testing.assert_array_equal(xs_s, xs_d)


def test_static_scale_zero():
    xq, xs = oracle.quant_act_static(np.ones((2, 16), np.float32), None, 0.0)
    assert xs[0] == 0.0 and not xq.any()


# ---- LayerNorm fold (page "4.2 W8A8 量化与 SmoothQuant" section 6) -------------

def _bf16(a):
    return oracle.f32_to_bf16(np.asarray(a, np.float32))


def test_layernorm_quant_closed_form():
    """x = [1, 2, 3, 4], gamma = 1, beta = 0, eps = 0: mu = 2.5, var = 1.25, so
    LN(x) = (x - 2.5) / sqrt(1.25) = [-1.342, -0.447, 0.447, 1.342]; per-token
    codes 127 * LN / max|LN| = [-127, -42, 42, 127] (-42.33 rounds to -42)."""
    x = _bf16([[1, 2, 3, 4]])
    xq, xs = oracle.layernorm_quant(x, np.ones(4, np.float32), None, 0.0)
    assert xq.tolist() == [[-127, -42, 42, 127]]
    assert abs(float(xs[0]) - 1.5 / np.sqrt(1.25) / 127) < 1e-7


def _ln_ref(xf, gamma, beta, eps):
    mu = xf.mean(axis=1, keepdims=True)
    var = ((xf - mu) ** 2).mean(axis=1, keepdims=True)
    return (xf - mu) / np.sqrt(var + eps) * gamma[None, :] + (0 if beta is None else beta[None, :])


@pytest.mark.parametrize("eps", [1e-5, 1e-3])
def test_layernorm_quant_matches_fp64_layernorm(eps):
    """Against numpy's fp64 LayerNorm (biased variance, eps inside the root,
    gamma then beta): scales agree to fp32 rounding, codes agree except for
    rare ties broken the other way (by at most 1)."""
    rng = np.random.default_rng(21)
    M, K = 64, 512
    xf = (rng.standard_normal((M, K)) * np.where(rng.random(K) < 0.02, 30.0, 1.0) + 0.3).astype(np.float32)
    x = _bf16(xf)
    xf = oracle.bf16_to_f32(x).astype(np.float64)
    gamma = (0.5 + rng.random(K)).astype(np.float32)
    beta = (0.1 * rng.standard_normal(K)).astype(np.float32)
    xq, xs = oracle.layernorm_quant(x, gamma, beta, eps)
    z = _ln_ref(xf, gamma.astype(np.float64), beta.astype(np.float64), eps)
    m = np.abs(z).max(axis=1)
    np.testing.assert_allclose(xs, m / 127, rtol=3e-7)
    ref = np.clip(np.rint(z * (127 / m)[:, None]), -127, 127)
    d = np.abs(xq.astype(np.int64) - ref)
    assert d.max() <= 1 and (d > 0).mean() < 1e-3


def test_layernorm_quant_constant_row_is_beta():
    """A constant row has zero variance: LN(x) = beta exactly, whatever eps."""
    K = 32
    beta = np.linspace(-1.0, 1.0, K).astype(np.float32)
    x = _bf16(np.full((1, K), 3.25))
    xq, xs = oracle.layernorm_quant(x, np.ones(K, np.float32), beta, 1e-5)
    q, s = oracle.quant_act(beta[None, :], None, oracle.PER_TOKEN)
    np.testing.assert_array_equal(xq, q)
    np.testing.assert_array_equal(xs, s)


def test_layernorm_plain_closed_form():
    """The definition on x = [1, 2, 3, 4], gamma = 1, no beta, eps = 0:
    z = (x - 2.5) / sqrt(1.25), codes [-127, -42, 42, 127], scale 1.5 / sqrt(1.25) / 127."""
    r = oracle.layernorm_quant_plain(_bf16([[1, 2, 3, 4]]), np.ones(4, np.float32), None, 0.0)
    assert r["codes"].tolist() == [[-127, -42, 42, 127]]
    assert r["mu"][0] == 2.5 and r["var"][0] == 1.25
    assert abs(r["scale"][0] - 1.5 / np.sqrt(1.25) / 127) < 1e-15


def test_layernorm_plain_against_exact_rationals():
    """Brute force on tiny rows: mean and biased variance in exact rationals
    (fractions), the normalised values from them; the fp64 definition agrees
    to fp64 rounding, and a constant row gives beta exactly."""
    from fractions import Fraction
    import math

    rng = np.random.default_rng(24)
    M, K = 5, 48
    xf = (rng.standard_normal((M, K)) * 3.0 + 1.0).astype(np.float32)
    xf[1] = 0.75
    x = _bf16(xf)
    gamma = (0.5 + rng.random(K)).astype(np.float32)
    beta = (0.2 * rng.standard_normal(K)).astype(np.float32)
    eps = np.float32(1e-5)
    r = oracle.layernorm_quant_plain(x, gamma, beta, float(eps))
    xv = oracle.bf16_to_f32(x)
    for i in range(M):
        row = [Fraction(float(v)) for v in xv[i]]
        mu = sum(row) / K
        var = sum((v - mu) ** 2 for v in row) / K
        assert r["mu"][i] == float(mu) and abs(r["var"][i] - float(var)) <= 4e-16 * float(var)
        sd = math.sqrt(float(var + Fraction(float(eps))))
        z = [float(v - mu) / sd * float(gamma[j]) + float(beta[j]) for j, v in enumerate(row)]
        np.testing.assert_allclose(r["z"][i], z, rtol=1e-14, atol=1e-15)
    np.testing.assert_array_equal(r["z"][1], beta.astype(np.float64))


@pytest.mark.parametrize("K,seed", [(256, 25), (2048, 26), (12288, 27)])
@pytest.mark.parametrize("with_beta", [True, False])
def test_layernorm_contract_within_bound_of_definition(K, seed, with_beta):
    """The library's LayerNorm arithmetic (the contract oracle: grid statistics,
    fp32 normalisation) against the plain fp64 definition, within the bound
    derived from that arithmetic (tests/ln_bound.py): scales within it, codes
    equal away from rounding boundaries and within one at them."""
    import ln_bound

    rng = np.random.default_rng(seed)
    M = 24
    out = rng.choice(K, max(1, K // 100), replace=False)
    xf = rng.standard_normal((M, K)) + 0.25
    xf[:, out] *= 50.0
    xf[0] = 1.5
    xf[2] = 0.0
    x = _bf16(xf.astype(np.float32))
    gamma = (0.5 + rng.random(K)).astype(np.float32)
    gamma[out[0]] = 40.0
    beta = (0.1 * rng.standard_normal(K)).astype(np.float32) if with_beta else None
    xq, xs = oracle.layernorm_quant(x, gamma, beta, 1e-5)
    plain = oracle.layernorm_quant_plain(x, gamma, beta, 1e-5)
    ln_bound.check(xq, xs, oracle.bf16_to_f32(x).astype(np.float64), gamma, beta, 1e-5, plain)


def test_layernorm_bound_rejects_a_wrong_variance():
    """The bound has teeth: the contract's codes measured against a definition
    with a planted mistake (unbiased variance, K - 1) fail the check."""
    import ln_bound

    rng = np.random.default_rng(28)
    M, K = 16, 64
    x = _bf16((rng.standard_normal((M, K)) * 2.0).astype(np.float32))
    gamma = np.ones(K, np.float32)
    xq, xs = oracle.layernorm_quant(x, gamma, None, 1e-5)
    wrong = oracle.layernorm_quant_plain(x, gamma, None, 1e-5)
    xf = oracle.bf16_to_f32(x).astype(np.float64)
    wrong["var"] = wrong["var"] * K / (K - 1)
    wrong["z"] = (xf - wrong["mu"][:, None]) / np.sqrt(wrong["var"] + np.float32(1e-5))[:, None]
    wrong["m"] = np.abs(wrong["z"]).max(axis=1)
    wrong["q"] = wrong["z"] * (127.0 / wrong["m"])[:, None]
    wrong["codes"] = np.clip(np.rint(wrong["q"]), -127, 127).astype(np.int8)
    wrong["scale"] = wrong["m"] / 127
    with pytest.raises(AssertionError):
        ln_bound.check(xq, xs, xf, gamma, None, 1e-5, wrong)


def test_fold_is_layernorm_times_inverse_factor():
    """LN with (gamma / s, beta / s) is LN(x) diag(s)^-1: against the fp64
    LayerNorm divided by s, codes agree within 1 and scales to fp32 rounding."""
    rng = np.random.default_rng(22)
    M, K = 32, 256
    x = _bf16(rng.standard_normal((M, K)) * 2.0)
    gamma = (0.5 + rng.random(K)).astype(np.float32)
    beta = (0.2 * rng.standard_normal(K)).astype(np.float32)
    s = np.exp(rng.standard_normal(K)).astype(np.float32)
    inv_s = (np.float32(1.0) / s).astype(np.float32)
    g2, b2 = oracle.fold_layernorm(gamma, beta, inv_s)
    np.testing.assert_array_equal(g2, (gamma * inv_s).astype(np.float32))
    xq, xs = oracle.layernorm_quant(x, g2, b2, 1e-5)
    z = _ln_ref(oracle.bf16_to_f32(x).astype(np.float64), gamma.astype(np.float64), beta.astype(np.float64),
                1e-5) / s.astype(np.float64)[None, :]
    m = np.abs(z).max(axis=1)
    np.testing.assert_allclose(xs, m / 127, rtol=1e-6)
    ref = np.clip(np.rint(z * (127 / m)[:, None]), -127, 127)
    assert np.abs(xq.astype(np.int64) - ref).max() <= 1


def test_folded_w8a8_error_matches_smoothed_path():
    """The folded runtime (LN with gamma', beta' -> per-token codes -> GEMM with
    diag(s) W codes) reaches about the error of quantizing LN(x) diag(s)^-1
    directly, far below the unsmoothed error on outlier channels."""
    rng = np.random.default_rng(23)
    M, K, N = 96, 512, 128
    x = _bf16(rng.standard_normal((M, K)))
    out = rng.choice(K, 6, replace=False)
    gamma = np.ones(K, np.float32)
    gamma[out] = 60.0  # outlier channels come from the LayerNorm weight
    beta = (0.05 * rng.standard_normal(K)).astype(np.float32)
    w = (0.02 * rng.standard_normal((K, N))).astype(np.float32)
    ln = _ln_ref(oracle.bf16_to_f32(x).astype(np.float64), gamma.astype(np.float64), beta.astype(np.float64),
                 1e-5).astype(np.float32)
    Y = oracle.matmul_f64(ln, w)
    s, inv_s = oracle.smooth_factors(oracle.calib_absmax(ln), oracle.weight_rowmax(w), 0.5)
    g2, b2 = oracle.fold_layernorm(gamma, beta, inv_s)
    xq, xs = oracle.layernorm_quant(x, g2, b2, 1e-5)
    wq, ws = oracle.quant_weight(w, s)
    y_fold, _ = oracle.dequant(oracle.gemm_i8(xq, wq), xs, oracle.PER_TOKEN, ws)
    e_fold = oracle.rel_fro(y_fold, Y)
    e_direct = oracle.rel_fro(oracle.w8a8_linear(ln, w, 0.5, oracle.PER_TOKEN)["y32"], Y)
    e_plain = oracle.rel_fro(oracle.w8a8_linear(ln, w, None, oracle.PER_TOKEN)["y32"], Y)
    assert abs(e_fold - e_direct) < 0.1 * e_direct
    assert e_fold < 0.5 * e_plain


# ---- alpha grid search (page "4.2 W8A8 量化与 SmoothQuant" sections 5.1, 5.2) ----

def test_alpha_search_has_an_interior_optimum():
    """Section 5.1: alpha too small leaves the activation error dominant, too
    large makes the weights the problem; the optimum lies inside, and on data
    with 100x outlier channels the page's effective range 0.4-0.6 contains it."""
    rng = np.random.default_rng(31)
    M, K, N = 64, 512, 192
    x = rng.standard_normal((M, K)).astype(np.float32)
    out = rng.choice(K, 6, replace=False)
    x[:, out] *= 100.0
    calib = rng.standard_normal((256, K)).astype(np.float32)
    calib[:, out] *= 100.0
    w = (0.02 * rng.standard_normal((K, N))).astype(np.float32)
    grid = [round(0.1 * i, 1) for i in range(11)]
    best, errs = oracle.search_alpha(x, w, calib, grid)
    assert errs[0.0] > errs[best] and errs[1.0] > errs[best]
    assert 0.4 <= best <= 0.6
    # the curve falls towards the optimum from both ends
    assert errs[0.0] > errs[0.2] > errs[best] and errs[1.0] > errs[0.8] > errs[best]


# ---- LLM.int8()-style decomposition (page "4.2 W8A8 量化与 SmoothQuant" section 2;
# page "量化：只压权重，与训练后量化（PTQ）", SmoothQuant W8A8 results paragraph) ------

def _bf16(a):
    return oracle.f32_to_bf16(np.asarray(a, np.float32))


def test_llm_int8_threshold_selects_the_pages_outlier_channel(worked):
    """With the pages' threshold 6, the worked example's outlier set is the
    channel the page names as its outlier channel, and nothing else."""
    g, X, W = worked
    thr = _gold("printed_constants.json")["llm_int8_threshold"]["threshold"]
    idx, keep = oracle.outlier_columns(oracle.calib_absmax(X), thr)
    assert idx.tolist() == [g["outlier_channel_1based"] - 1]
    assert keep.tolist() == [0.0 if j == g["outlier_channel_1based"] - 1 else 1.0 for j in range(X.shape[1])]


def test_llm_int8_threshold_is_strict():
    """'Exceeds' the threshold: a channel whose max equals it stays regular;
    the next fp32 value above it is an outlier."""
    t = np.float32(6.0)
    amax = np.array([t, np.nextafter(t, np.float32(np.inf)), np.nextafter(t, np.float32(0)), 0.0, 1e30],
                    np.float32)
    idx, keep = oracle.outlier_columns(amax, float(t))
    assert idx.tolist() == [1, 4]
    assert keep.tolist() == [1.0, 0.0, 1.0, 1.0, 0.0]


def test_llm_int8_codes_on_worked_example(worked):
    """The per-token scale of the INT8 part comes from the regular channels
    only: fp64 closed form round(127 x / max over regular channels), with the
    outlier channel's codes 0."""
    g, X, W = worked
    xb, wb = _bf16(X), _bf16(W)
    wq, ws = oracle.quant_weight(wb, None)
    r = oracle.llm_int8(xb, wb, wq, ws, 6.0)
    xf = oracle.bf16_to_f32(xb).astype(np.float64)
    reg = [0, 2]
    want = np.zeros((3, 3), np.int64)
    for i in range(3):
        m = np.abs(xf[i, reg]).max()
        for j in reg:
            want[i, j] = int(np.round(xf[i, j] * 127.0 / m))
    np.testing.assert_array_equal(r["xq"].astype(np.int64), want)
    np.testing.assert_allclose(r["x_scale"], np.abs(xf[:, reg]).max(axis=1) / 127.0, rtol=2 ** -23)


def test_llm_int8_integer_case_is_exact():
    """No rounding anywhere: regular channels hold integers with each token's
    regular max exactly 127 (x_scale = 1), outlier channels integers above the
    threshold 127, W integers with each column's max 127 (w_scale = 1).  Then
    both halves are exact and the result is the integer product, checked by
    brute force in Python integers."""
    rng = np.random.default_rng(5)
    M, K, N = 5, 24, 7
    out = [3, 10, 17]
    x = rng.integers(-127, 128, (M, K))
    x[:, out] = rng.integers(128, 257, (M, len(out))) * rng.choice([-1, 1], (M, len(out)))
    reg = [j for j in range(K) if j not in out]
    for i in range(M):
        x[i, reg[i % len(reg)]] = 127 if i % 2 else -127
        x[i, reg] = np.clip(x[i, reg], -127, 127)
    w = rng.integers(-127, 128, (K, N))
    for k in range(N):
        w[(5 * k) % K, k] = -127 if k % 2 else 127
    xb, wb = _bf16(x), _bf16(w)
    assert (oracle.bf16_to_f32(xb) == x).all() and (oracle.bf16_to_f32(wb) == w).all()
    wq, ws = oracle.quant_weight(wb, None)
    r = oracle.llm_int8(xb, wb, wq, ws, 127.0)
    assert r["idx"].tolist() == out
    want = [[sum(int(x[i, j]) * int(w[j, k]) for j in range(K)) for k in range(N)] for i in range(M)]
    np.testing.assert_array_equal(r["y32"].astype(np.int64), np.array(want))
    # the bound is the sum of |x w| over the outlier channels only
    b = [[sum(abs(int(x[i, j]) * int(w[j, k])) for j in out) for k in range(N)] for i in range(M)]
    np.testing.assert_array_equal(r["bound"], np.array(b, np.float64))


def test_llm_int8_without_outliers_is_the_w8a8_baseline():
    """A threshold above every channel max leaves no outlier: the product is
    the unsmoothed per-token W8A8 path (the pinned step-4/5 baseline)."""
    rng = np.random.default_rng(6)
    x = _bf16(rng.standard_normal((16, 96)))
    w = _bf16(0.02 * rng.standard_normal((96, 40)))
    wq, ws = oracle.quant_weight(w, None)
    r = oracle.llm_int8(x, w, wq, ws, 1e30)
    b = oracle.w8a8_linear(x, w, None, oracle.PER_TOKEN)
    assert r["idx"].size == 0
    np.testing.assert_array_equal(r["xq"], b["xq"])
    np.testing.assert_array_equal(r["y32"], b["y32"])
    np.testing.assert_array_equal(r["ybf16"], b["ybf16"])


def test_llm_int8_all_outliers_is_the_16bit_product():
    """A negative threshold makes every channel an outlier: the INT8 part is
    empty and the result is X W, i.e. numpy's fp64 product rounded to fp32
    (within one fp32 ulp: the two fp64 sums differ in order)."""
    rng = np.random.default_rng(7)
    x = _bf16(rng.standard_normal((9, 70)))
    w = _bf16(0.02 * rng.standard_normal((70, 33)))
    wq, ws = oracle.quant_weight(w, None)
    r = oracle.llm_int8(x, w, wq, ws, -1.0)
    assert r["idx"].size == 70
    assert (r["xq"] == 0).all()
    ref = oracle.matmul_f64(x, w).astype(np.float32)
    ulp = np.spacing(np.abs(ref))
    assert (np.abs(r["y32"] - ref) <= ulp).all()


@pytest.mark.parametrize("cfg", [synth.ATTN_PROJ, synth.MLP_UP])
def test_llm_int8_keeps_accuracy_on_outlier_data(cfg):
    """The pages' comparison: direct W8A8 collapses on outlier activations,
    while the mixed-precision route keeps 16-bit accuracy (and SmoothQuant
    matches it).  On a reduced draw of the configuration's recipe, the
    decomposed product's error is far below the unsmoothed per-token W8A8
    error and not above the smoothed one by more than a small factor."""
    inp = synth.make(cfg, M=48, K=512, N=96, calib_chunks=2, chunk_tokens=64)
    x, w = synth.to_numpy(inp.x), synth.to_numpy(inp.w)
    wq, ws = oracle.quant_weight(w, None)
    r = oracle.llm_int8(x, w, wq, ws, 6.0)
    assert set(inp.out_idx.tolist()) <= set(r["idx"].tolist())
    Y = oracle.matmul_f64(x, w)
    e_mixed = oracle.rel_fro(r["y32"], Y)
    e_plain = oracle.rel_fro(oracle.w8a8_linear(x, w, None, oracle.PER_TOKEN)["y32"], Y)
    e_smooth = oracle.rel_fro(
        oracle.w8a8_linear(x, w, 0.5, oracle.PER_TOKEN, calib=synth.to_numpy(inp.calib))["y32"], Y)
    assert e_mixed < 0.2 * e_plain
    assert e_mixed < 2.0 * e_smooth


def test_outlier_channel_takes_the_largest_factor():
    """The effect the explainer page "SmoothQuant大模型平滑量化技术" describes, on
    data of this test's own making: one input channel carries values about 60x
    the others on every token.  At alpha = 0.5 that channel gets the largest
    smoothing factor, its smoothed maximum falls to the geometric mean of the
    two maxima (far below the raw one), and the per-tensor W8A8 error of the
    product drops.  Direction only: the page prints no values."""
    rng = np.random.default_rng(7)
    T, K, N = 32, 12, 6
    X = rng.standard_normal((T, K)).astype(np.float32)
    X[:, 5] *= 60.0
    W = (0.1 * rng.standard_normal((K, N))).astype(np.float32)
    ax, aw = oracle.calib_absmax(X), oracle.weight_rowmax(W)
    s, inv_s = oracle.smooth_factors(ax, aw, 0.5)
    assert int(np.argmax(s)) == 5
    smoothed_max = np.abs(X * inv_s[None, :]).max(axis=0)
    np.testing.assert_allclose(smoothed_max, np.sqrt(ax.astype(np.float64) * aw), rtol=1e-6)
    assert smoothed_max[5] < ax[5] / 10
    y = oracle.matmul_f64(X, W)
    plain = oracle.rel_fro(oracle.w8a8_linear(X, W, None, oracle.PER_TENSOR)["y32"], y)
    smooth = oracle.rel_fro(oracle.w8a8_linear(X, W, 0.5, oracle.PER_TENSOR, calib=X)["y32"], y)
    assert smooth < plain
