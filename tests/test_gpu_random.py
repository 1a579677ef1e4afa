"""Seeded random shapes for the calls whose fixed cases live elsewhere: the
fused LayerNorm + codes kernel (against the library's contract), the steps 2-4
call sq_prepare_and_quant_act (against the oracle's steps 2, 3 and 4 directly)
the static per-tensor scale and the few-token (decode) GEMM kernels.  Every
output is compared bit for bit; the draws cover ragged token counts, channel
counts up to the kernels' limits and both granularities."""
import numpy as np
import pytest
import torch

import oracle
import post_quantization_act_amd as sq
import synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _np(t):
    return synth.to_numpy(t)


def _acts(M, K, g, kind="normal", factor=60.0, dtype=torch.bfloat16):
    n_out = max(1, K // 100)
    idx = torch.randperm(K, generator=g)[:n_out]
    return synth.activations(M, K, kind, idx, torch.full((n_out,), factor), dtype, g, "cpu"), idx


def _ln_cases(n, seed):
    """M up to 900, K a multiple of 16 up to 16384, with or without beta, and
    every other case a row stride padded by a multiple of 8 elements."""
    r = np.random.default_rng(seed)
    return [(int(r.integers(1, 901)), 16 * int(r.integers(1, 1025)), bool(r.random() < 0.7),
             8 * int(r.integers(1, 9)) if i % 2 else 0) for i in range(n)]


@pytest.mark.parametrize("M,K,with_beta,pad", _ln_cases(12, 4242))
def test_random_layernorm_shapes(M, K, with_beta, pad):
    print(f"random layernorm M={M} K={K} beta={with_beta} pad={pad}", flush=True)
    g = torch.Generator(device="cpu")
    g.manual_seed(M * 31 + K)
    x, idx = _acts(M, K, g, kind="t4", factor=30.0)
    x = (x.float() + 0.5).to(torch.bfloat16)  # a non-zero mean
    gamma = (torch.rand(K, generator=g) + 0.5).float()
    gamma[idx[:1]] = 25.0
    beta = (torch.randn(K, generator=g) * 0.1).float() if with_beta else None
    xq = torch.empty(M, K, dtype=torch.int8, device=DEV)
    xs = torch.empty(M, dtype=torch.float32, device=DEV)
    xd = torch.zeros(M, K + pad, dtype=torch.bfloat16, device=DEV)[:, :K] if pad else torch.empty_like(x, device=DEV)
    xd.copy_(x.to(DEV))
    sq.sq_layernorm_quant(xd, gamma.to(DEV), None if beta is None else beta.to(DEV), 1e-5, xq, xs)
    torch.cuda.synchronize()
    xq_o, xs_o = oracle.layernorm_quant(_np(x), gamma.numpy(), None if beta is None else beta.numpy(), 1e-5)
    np.testing.assert_array_equal(_np(xs), xs_o)
    np.testing.assert_array_equal(_np(xq), xq_o)


def _prep_cases(n, seed):
    """K a multiple of 16 up to 8192 (both sides of the one-launch limit of
    4096), N up to 3000 (half multiples of 8: the one-read weight pass), bf16 or
    fp32 W and X, either granularity, alpha from a grid that holds the exact
    forms and general values."""
    r = np.random.default_rng(seed)
    out = []
    for i in range(n):
        M = int(r.integers(1, 1201))
        K = 16 * int(r.integers(1, 513))
        N = int(r.integers(8, 3001))
        if i % 2 == 0:
            N = 8 * max(1, N // 8)
        wt = torch.bfloat16 if r.random() < 0.8 else torch.float32
        xt = torch.bfloat16 if r.random() < 0.8 else torch.float32
        gran = sq.SQ_PER_TOKEN if r.random() < 0.7 else sq.SQ_PER_TENSOR
        alpha = float(r.choice([0.0, 0.3, 0.5, 0.65, 0.8, 1.0]))
        out.append((M, K, N, wt, xt, gran, alpha))
    return out


@pytest.mark.parametrize("M,K,N,wt,xt,gran,alpha", _prep_cases(12, 777))
def test_random_prepare_and_quant_act(M, K, N, wt, xt, gran, alpha):
    print(f"random steps 2-4 M={M} K={K} N={N} {wt} {xt} gran={gran} alpha={alpha}", flush=True)
    g = torch.Generator(device="cpu")
    g.manual_seed(M + 3 * K + 5 * N)
    x, idx = _acts(M, K, g, dtype=xt)
    w = synth.weights(K, N, 0.02, wt, g, "cpu")
    amax = (torch.rand(K, generator=g) * 3 + 0.01).float()
    amax[idx] *= 60.0
    f32 = dict(dtype=torch.float32, device=DEV)
    s, inv_s, aw = torch.empty(K, **f32), torch.empty(K, **f32), torch.empty(K, **f32)
    wq = torch.empty(N, K, dtype=torch.int8, device=DEV)
    w_scale = torch.empty(N, **f32)
    xq = torch.empty(M, K, dtype=torch.int8, device=DEV)
    x_scale = torch.empty(1 if gran == sq.SQ_PER_TENSOR else M, **f32)
    nb = sq.sq_workspace_size(sq.SQ_OP_PREPARE_AND_QUANT_ACT, M, N, K, gran)
    ws = torch.empty(max(nb, 16), dtype=torch.uint8, device=DEV)
    sq.sq_prepare_and_quant_act(amax.to(DEV), w.to(DEV), alpha, s, inv_s, aw, wq, w_scale, x.to(DEV), gran, xq,
                                x_scale, ws)
    torch.cuda.synchronize()
    aw_o = oracle.weight_rowmax(_np(w))
    s_o, inv_o = oracle.smooth_factors(amax.numpy(), aw_o, alpha)
    wq_o, ws_o = oracle.quant_weight(_np(w), s_o)
    xq_o, xs_o = oracle.quant_act(_np(x), inv_o, gran)
    for name, got, ref in (("amax_w", aw, aw_o), ("s", s, s_o), ("inv_s", inv_s, inv_o), ("wq", wq, wq_o),
                           ("w_scale", w_scale, ws_o), ("xq", xq, xq_o), ("x_scale", x_scale, xs_o)):
        np.testing.assert_array_equal(_np(got), ref, err_msg=name)


def _static_cases(n, seed):
    r = np.random.default_rng(seed)
    return [(int(r.integers(1, 1501)), 16 * int(r.integers(1, 1281)), int(r.integers(1, 600)),
             float(r.choice([0.5, 1.0, 3.0]))) for _ in range(n)]


@pytest.mark.parametrize("M,K,T,boost", _static_cases(8, 99))
def test_random_static_scale(M, K, T, boost):
    """The calibrated maximum from the channel maxima, then codes of run-time
    tokens up to 3x beyond the calibrated range (saturation), K up to 20480
    (the two-pass kernel beyond 16384 channels)."""
    print(f"random static M={M} K={K} T={T} boost={boost}", flush=True)
    g = torch.Generator(device="cpu")
    g.manual_seed(M * 7 + K + T)
    calib, idx = _acts(T, K, g)
    x = synth.activations(M, K, "normal", idx, torch.full((len(idx),), 60.0 * boost), torch.bfloat16, g, "cpu")
    inv_s = torch.exp(torch.randn(K, generator=g) * 0.4).float()
    amax = torch.zeros(K, dtype=torch.float32, device=DEV)
    sq.sq_calib_absmax(calib.to(DEV), amax)
    a = torch.empty(1, dtype=torch.float32, device=DEV)
    sq.sq_static_act_max(amax, inv_s.to(DEV), a)
    xq = torch.empty(M, K, dtype=torch.int8, device=DEV)
    xs = torch.empty(1, dtype=torch.float32, device=DEV)
    sq.sq_quant_act_static(x.to(DEV), inv_s.to(DEV), a, xq, xs)
    torch.cuda.synchronize()
    a_o = oracle.static_act_max(_np(calib), inv_s.numpy())
    assert _np(a)[0] == a_o
    xq_o, xs_o = oracle.quant_act_static(_np(x), inv_s.numpy(), a_o)
    np.testing.assert_array_equal(_np(xs), xs_o)
    np.testing.assert_array_equal(_np(xq), xq_o)


def _decode_cases(n, seed):
    """Few-token products: M <= 16, K a multiple of 2048 up to 16384 (the
    weight-streaming ring, 1 to 8 chunks per wavefront) or any multiple of 16
    (the other decode kernel), N from one 16-channel group to 40000 (up to the
    ring's group limit per block), bf16 or fp32 output, either granularity."""
    r = np.random.default_rng(seed)
    out = []
    for i in range(n):
        M = int(r.integers(1, 17))
        K = 2048 * int(r.integers(1, 9)) if i % 3 else 16 * int(r.integers(1, 700))
        N = int(r.integers(1, 40001)) if i % 2 else 16 * int(r.integers(1, 200))
        out.append((M, K, N, bool(r.random() < 0.6), sq.SQ_PER_TOKEN if r.random() < 0.7 else sq.SQ_PER_TENSOR))
    return out


@pytest.mark.parametrize("M,K,N,bf16_out,gran", _decode_cases(10, 1616))
def test_random_decode_gemm(M, K, N, bf16_out, gran):
    print(f"random decode M={M} K={K} N={N} bf16={bf16_out} gran={gran} {sq.sq_gemm_kernel_name(M, N, K)[:24]}",
          flush=True)
    g = torch.Generator(device="cpu")
    g.manual_seed(M * 131 + K + N)
    codes = lambda r, c: torch.clamp(torch.round(torch.randn(r, c, generator=g) * 30.0), -127, 127).to(torch.int8)
    xq, wq = codes(M, K), codes(N, K)
    xs = (torch.rand(1 if gran == sq.SQ_PER_TENSOR else M, generator=g) * 1e-2 + 1e-4).float()
    ws = (torch.rand(N, generator=g) * 1e-2 + 1e-4).float()
    yt = torch.bfloat16 if bf16_out else torch.float32
    xd, xsd, wd, wsd = xq.to(DEV), xs.to(DEV), wq.to(DEV), ws.to(DEV)
    y = torch.empty(M, N, dtype=yt, device=DEV)
    sq.sq_gemm_w8a8(xd, xsd, gran, wd, wsd, y)  # the deployed call: no accumulator store
    y_acc = torch.empty(M, N, dtype=yt, device=DEV)
    acc = torch.empty(M, N, dtype=torch.int32, device=DEV)
    sq.sq_gemm_w8a8(xd, xsd, gran, wd, wsd, y_acc, acc)
    torch.cuda.synchronize()
    acc_o = oracle.gemm_i8(xq.numpy(), wq.numpy(), nthreads=8)
    y32_o, ybf_o = oracle.dequant(acc_o, xs.numpy(), gran, ws.numpy())
    np.testing.assert_array_equal(acc.cpu().numpy(), acc_o)
    np.testing.assert_array_equal(_np(y), ybf_o if bf16_out else y32_o)
    np.testing.assert_array_equal(_np(y_acc), ybf_o if bf16_out else y32_o)
