"""Migration-strength grid search on the GPU: every alpha's W8A8 output equals
the oracle's (so the errors agree to the rounding of the two fp64 norms) and
the search picks the oracle's alpha."""
import numpy as np
import pytest
import torch

import oracle
import post_quantization_act_amd as sq
import synth
from post_quantization_act_amd import pipeline

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.mark.parametrize("kind,factor", [("normal", 100.0), ("t4", 200.0)])
def test_alpha_search_matches_oracle(kind, factor):
    print(f"alpha search {kind} x{factor}", flush=True)
    M, K, N, T = 128, 1024, 384, 512
    g = torch.Generator(device="cpu")
    g.manual_seed(int(factor))
    idx = torch.randperm(K, generator=g)[:10]
    fac = torch.full((10,), factor)
    x = synth.activations(M, K, kind, idx, fac, torch.bfloat16, g, "cpu")
    calib = synth.activations(T, K, kind, idx, fac, torch.bfloat16, g, "cpu")
    w = synth.weights(K, N, 0.02, torch.bfloat16, g, "cpu")
    grid = [round(0.05 * i, 2) for i in range(21)]

    amax = torch.zeros(K, dtype=torch.float32, device=DEV)
    sq.sq_calib_absmax(calib.to(DEV), amax)
    best, errs = pipeline.search_alpha(x.to(DEV), w.to(DEV), amax, grid)
    torch.cuda.synchronize()
    best_o, errs_o = oracle.search_alpha(synth.to_numpy(x), synth.to_numpy(w), synth.to_numpy(calib), grid)
    assert best == best_o
    for a in grid:
        assert abs(errs[a] - errs_o[a]) <= 1e-9 * errs_o[a], a
    assert errs[0.0] > errs[best] and errs[1.0] > errs[best]


# ---- the search's criterion, called directly -------------------------------------------

U64 = 2.0 ** -53  # unit roundoff of fp64


def _f64_bound(x, w):
    """Both sides sum K fp64 products (exact widenings of bf16 / fp32 values) in
    some order, so each is within K u sum_k |x w| of the exact value (the
    standard bound on a recursive sum): allow twice that between them."""
    K = x.shape[1]
    xf, wf = oracle.as_f32(x).astype(np.float64), oracle.as_f32(w).astype(np.float64)  # bf16 bits widened
    return 2.0 * K * U64 * (np.abs(xf) @ np.abs(wf))


@pytest.mark.parametrize("M,K,N,xt,wt,padx,padw", [
    (130, 208, 300, torch.bfloat16, torch.bfloat16, 0, 0),   # 3 row tiles, 3 column tiles, ragged tails
    (64, 16, 128, torch.float32, torch.bfloat16, 0, 0),      # exactly one tile, one k chunk
    (1, 4096, 5, torch.bfloat16, torch.float32, 8, 3),       # one token, strided x and w
    (257, 1024, 129, torch.float32, torch.float32, 16, 1),   # fp32 both, odd column stride
])
def test_matmul_f64_matches_oracle(M, K, N, xt, wt, padx, padw):
    print(f"matmul_f64 {M}x{K}x{N} {xt} {wt} pad {padx},{padw}", flush=True)
    g = torch.Generator(device="cpu")
    g.manual_seed(M * 7 + N)
    idx = torch.randperm(K, generator=g)[: max(1, K // 100)]
    fac = torch.full((len(idx),), 80.0)
    x_full = synth.activations(M, K + padx, "t4", idx, fac, xt, g, "cpu")
    w_full = synth.weights(K, N + padw, 0.02, wt, g, "cpu")
    x, w = x_full[:, :K], w_full[:, :N]
    y = torch.empty(M, N, dtype=torch.float64, device=DEV)
    sq.sq_matmul_f64(x_full.to(DEV)[:, :K], w_full.to(DEV)[:, :N], y)
    xo, wo = synth.to_numpy(x), synth.to_numpy(w)
    ref = oracle.matmul_f64(xo, wo)
    got = y.cpu().numpy()
    assert np.all(np.abs(got - ref) <= _f64_bound(xo, wo))


def test_matmul_f64_full_size_sampled():
    """The search's reference product at the size the benchmark scores its
    alpha sweep on (256 tokens of the 8192 x 12288 x 49152 workload): 256
    entries spread over all row and column tiles, each against the oracle."""
    M, K, N = 256, 12288, 49152
    print(f"matmul_f64 full size {M}x{K}x{N}", flush=True)
    g = torch.Generator(device=DEV)
    g.manual_seed(4242)
    idx = torch.randperm(K, generator=torch.Generator().manual_seed(5))[:61]
    x = synth.activations(M, K, "t4", idx, torch.full((61,), 200.0), torch.bfloat16, g, DEV)
    w = synth.weights(K, N, 0.015, torch.bfloat16, g, DEV)
    y = torch.empty(M, N, dtype=torch.float64, device=DEV)
    sq.sq_matmul_f64(x, w, y)
    rows = torch.linspace(0, M - 1, 16).round().long().to(DEV)
    cols = torch.linspace(0, N - 1, 16).round().long().to(DEV)
    xo = synth.to_numpy(x[rows].cpu())
    wo = synth.to_numpy(w[:, cols].cpu())
    ref = oracle.matmul_f64(xo, wo)
    got = y[rows][:, cols].cpu().numpy()
    assert np.all(np.abs(got - ref) <= _f64_bound(xo, wo))


@pytest.mark.parametrize("M,N", [(3, 16), (257, 1000), (700, 1000), (256, 49152)])
def test_rel_error_matches_oracle(M, N):
    """Sizes below one element per thread up to the full-size sample (many
    grid-stride passes).  The two sides add n = M N non-negative fp64 terms in
    different orders, each within (n - 1) u of the exact sum; the square roots
    halve that, so the quotients agree to n u."""
    print(f"rel_error {M}x{N}", flush=True)
    g = torch.Generator(device="cpu")
    g.manual_seed(M + N)
    y_ref = torch.randn(M, N, generator=g, dtype=torch.float64) * 3.0
    y = (y_ref + 0.01 * torch.randn(M, N, generator=g, dtype=torch.float64)).float()
    ws = torch.empty(sq.sq_workspace_size(sq.SQ_OP_REL_ERROR, M, N, 0), dtype=torch.uint8, device=DEV)
    err = torch.empty(1, dtype=torch.float64, device=DEV)
    sq.sq_rel_error(y.to(DEV), y_ref.to(DEV), err, ws)
    ref = oracle.rel_fro(y.numpy(), y_ref.numpy())
    assert abs(err.item() - ref) <= M * N * U64 * ref


def test_rel_error_special_cases():
    """Equal inputs give exactly 0; an all-zero reference gives the IEEE
    quotient (x / 0 = inf, 0 / 0 = NaN), and so does an empty one; the
    workspace's previous contents do not matter (every partial is rewritten)."""
    ws = torch.full((sq.sq_workspace_size(sq.SQ_OP_REL_ERROR, 4, 64, 0),), 255, dtype=torch.uint8, device=DEV)
    err = torch.empty(1, dtype=torch.float64, device=DEV)
    y = torch.randn(4, 64, device=DEV)
    sq.sq_rel_error(y, y.double(), err, ws)
    assert err.item() == 0.0
    z = torch.zeros(4, 64, dtype=torch.float64, device=DEV)
    sq.sq_rel_error(torch.ones(4, 64, device=DEV), z, err, ws)
    assert err.item() == float("inf")
    sq.sq_rel_error(torch.zeros(4, 64, device=DEV), z, err, ws)
    assert np.isnan(err.item())
    err.fill_(1.0)
    sq.sq_rel_error(torch.empty(0, 64, device=DEV), torch.empty(0, 64, dtype=torch.float64, device=DEV), err, ws)
    assert np.isnan(err.item())  # no elements: 0 / 0


def test_matmul_f64_unaligned_views():
    """Operands that start mid-row (element alignment only) and odd strides."""
    M, K, N = 33, 64, 40
    print(f"matmul_f64 unaligned views {M}x{K}x{N}", flush=True)
    g = torch.Generator(device="cpu")
    g.manual_seed(77)
    x_full = synth.activations(M, K + 5, "normal", None, None, torch.bfloat16, g, "cpu")
    w_full = synth.weights(K, N + 3, 0.02, torch.float32, g, "cpu")
    x, w = x_full[:, 3:K + 3], w_full[:, 1:N + 1]
    y = torch.empty(M, N, dtype=torch.float64, device=DEV)
    sq.sq_matmul_f64(x_full.to(DEV)[:, 3:K + 3], w_full.to(DEV)[:, 1:N + 1], y)
    xo, wo = synth.to_numpy(x.contiguous()), synth.to_numpy(w.contiguous())
    assert np.all(np.abs(y.cpu().numpy() - oracle.matmul_f64(xo, wo)) <= _f64_bound(xo, wo))


def test_matmul_f64_empty_sizes():
    """K = 0 writes zeros (the empty sum); M = 0 or N = 0 enqueues nothing."""
    y = torch.full((5, 24), 7.0, dtype=torch.float64, device=DEV)
    sq.sq_matmul_f64(torch.empty(5, 0, dtype=torch.bfloat16, device=DEV),
                     torch.empty(0, 24, dtype=torch.float32, device=DEV), y)
    assert torch.count_nonzero(y).item() == 0
    y0 = torch.empty(0, 24, dtype=torch.float64, device=DEV)
    sq.sq_matmul_f64(torch.empty(0, 32, dtype=torch.bfloat16, device=DEV),
                     torch.ones(32, 24, dtype=torch.bfloat16, device=DEV), y0)
