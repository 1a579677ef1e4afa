"""LayerNorm fold on the GPU: sq_fold_layernorm and the fused LayerNorm +
per-token INT8 kernel equal the library's contract (the oracle's fixed-point
statistics and fp32 normalisation) bit for bit, and stay within the derived
bound of the plain fp64 LayerNorm definition (every row layout of the kernel,
ragged token counts, constant and all-zero rows, no bias); the folded runtime
path (fold -> LayerNorm codes -> GEMM) equals the oracle's."""
import numpy as np
import pytest
import torch

import ln_bound
import oracle
import post_quantization_act_amd as sq
import synth
from post_quantization_act_amd import pipeline

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _np(t):
    return synth.to_numpy(t)


def _rows(M, K, seed):
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    n_out = max(1, K // 100)
    idx = torch.randperm(K, generator=g)[:n_out]
    x = synth.activations(M, K, "normal", idx, torch.full((n_out,), 50.0), torch.bfloat16, g, "cpu")
    x = x + 0.25  # a non-zero mean
    x = x.to(torch.bfloat16)
    gamma = (torch.rand(K, generator=g) + 0.5).float()
    gamma[idx[:1]] = 40.0
    beta = (torch.randn(K, generator=g) * 0.1).float()
    return x, gamma, beta


@pytest.mark.parametrize("M,K", [(130, 256), (13, 1024), (64, 2048), (37, 4096), (9, 8192), (40, 12288),
                                 (5, 16384),
                                 # rows shared by teams of one block: more rows than teams in the grid, a last
                                 # pass where most teams are past M, fewer rows than one block's teams, ragged
                                 # channel groups
                                 (800, 12288), (770, 10256), (517, 16384), (3, 12288), (1000, 9232)])
@pytest.mark.parametrize("with_beta", [True, False])
def test_layernorm_quant_matches_oracle(M, K, with_beta):
    print(f"layernorm M={M} K={K} beta={with_beta}", flush=True)
    x, gamma, beta = _rows(M, K, M * 3 + K)
    x[0] = 1.5           # constant row: zero variance
    if M > 2:
        x[2] = 0.0       # all-zero row
    b = beta if with_beta else None
    xq = torch.empty(M, K, dtype=torch.int8, device=DEV)
    xs = torch.empty(M, dtype=torch.float32, device=DEV)
    sq.sq_layernorm_quant(x.to(DEV), gamma.to(DEV), None if b is None else b.to(DEV), 1e-5, xq, xs)
    torch.cuda.synchronize()
    xq_o, xs_o = oracle.layernorm_quant(_np(x), gamma.numpy(), None if b is None else b.numpy(), 1e-5)
    np.testing.assert_array_equal(_np(xs), xs_o)
    np.testing.assert_array_equal(_np(xq), xq_o)


@pytest.mark.parametrize("M,K", [(130, 256), (13, 1024), (64, 2048), (37, 4096), (9, 8192), (40, 12288),
                                 (5, 16384)])
@pytest.mark.parametrize("with_beta", [True, False])
def test_layernorm_quant_within_bound_of_definition(M, K, with_beta):
    """The kernel against the plain fp64 LayerNorm (two-pass mean and biased
    variance, eps inside the root, then per-token codes), not against its own
    contract: scales within the derived bound, codes equal to the definition's
    except within the bound of a rounding boundary, and there within one."""
    print(f"layernorm vs definition M={M} K={K} beta={with_beta}", flush=True)
    x, gamma, beta = _rows(M, K, M * 5 + K + 1)
    x[0] = 1.5
    if M > 2:
        x[2] = 0.0
    b = beta if with_beta else None
    xq = torch.empty(M, K, dtype=torch.int8, device=DEV)
    xs = torch.empty(M, dtype=torch.float32, device=DEV)
    sq.sq_layernorm_quant(x.to(DEV), gamma.to(DEV), None if b is None else b.to(DEV), 1e-5, xq, xs)
    torch.cuda.synchronize()
    bn = None if b is None else b.numpy()
    plain = oracle.layernorm_quant_plain(_np(x), gamma.numpy(), bn, 1e-5)
    xf = oracle.bf16_to_f32(_np(x)).astype(np.float64)
    ln_bound.check(_np(xq), _np(xs), xf, gamma.numpy(), bn, 1e-5, plain)


def test_fold_layernorm_matches_oracle():
    g = torch.Generator(device="cpu")
    g.manual_seed(4)
    K = 4112
    gamma, beta = torch.rand(K, generator=g) + 0.5, torch.randn(K, generator=g)
    inv_s = torch.exp(torch.randn(K, generator=g)).float()
    go, bo = torch.empty(K, device=DEV), torch.empty(K, device=DEV)
    sq.sq_fold_layernorm(gamma.to(DEV), beta.to(DEV), inv_s.to(DEV), go, bo)
    torch.cuda.synchronize()
    go_o, bo_o = oracle.fold_layernorm(gamma.numpy(), beta.numpy(), inv_s.numpy())
    np.testing.assert_array_equal(_np(go), go_o)
    np.testing.assert_array_equal(_np(bo), bo_o)


def test_folded_runtime_path_matches_oracle():
    """Calibrate on LayerNorm outputs, fold 1/s into gamma and beta, then the
    runtime: LayerNorm codes of the raw rows and the GEMM with diag(s) W."""
    M, K, N, T = 96, 2048, 520, 256
    x, gamma, beta = _rows(M, K, 77)
    xc, _, _ = _rows(T, K, 78)
    # calibration activations: the LayerNorm outputs of the calibration rows (fp64, then bf16)
    xf = oracle.bf16_to_f32(_np(xc)).astype(np.float64)
    mu = xf.mean(axis=1, keepdims=True)
    ln = (xf - mu) / np.sqrt(((xf - mu) ** 2).mean(axis=1, keepdims=True) + 1e-5) * gamma.numpy() + beta.numpy()
    calib = torch.from_numpy(ln.astype(np.float32)).to(torch.bfloat16)
    g = torch.Generator(device="cpu")
    g.manual_seed(79)
    w = synth.weights(K, N, 0.02, torch.bfloat16, g, "cpu")

    b = pipeline.W8A8Buffers.allocate(M, N, K, sq.SQ_PER_TOKEN, DEV)
    pipeline.calibrate(calib.to(DEV), b.amax_x)
    pipeline.prepare_weights(w.to(DEV), 0.5, b)
    g2, b2 = torch.empty(K, device=DEV), torch.empty(K, device=DEV)
    sq.sq_fold_layernorm(gamma.to(DEV), beta.to(DEV), b.inv_s, g2, b2)
    sq.sq_layernorm_quant(x.to(DEV), g2, b2, 1e-5, b.xq, b.x_scale)
    sq.sq_gemm_w8a8(b.xq, b.x_scale, sq.SQ_PER_TOKEN, b.wq, b.w_scale, b.y)
    torch.cuda.synchronize()

    s, inv_s = oracle.smooth_factors(oracle.calib_absmax(_np(calib)), oracle.weight_rowmax(_np(w)), 0.5)
    go, bo = oracle.fold_layernorm(gamma.numpy(), beta.numpy(), inv_s)
    xq_o, xs_o = oracle.layernorm_quant(_np(x), go, bo, 1e-5)
    wq_o, ws_o = oracle.quant_weight(_np(w), s)
    _, ybf = oracle.dequant(oracle.gemm_i8(xq_o, wq_o, nthreads=8), xs_o, oracle.PER_TOKEN, ws_o)
    np.testing.assert_array_equal(_np(b.xq), xq_o)
    np.testing.assert_array_equal(_np(b.y), ybf)
