"""Parity at the five workloads' full sizes, in the launch configuration the
benchmark times (bf16 output, no int32 side output).

The oracle recomputes, on the host, everything it can afford in full (channel
maxima, weight row maxima, factors) and samples the rest: the codes and scales
of a set of output channels and of a set of tokens, and the bf16 outputs where
those tokens and channels cross.  Every sampled value must match bit for bit.
A second launch with the int32 side output is checked at full size by
Freivalds' test (acc . r == Xq . (Wq^T r) for random +-1 vectors r), a
property that holds at any size."""
import numpy as np
import pytest
import torch

import oracle
import post_quantization_act_amd as sq
import synth
from post_quantization_act_amd import pipeline

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _np(t):
    return synth.to_numpy(t)


def _say(msg):
    print(msg, flush=True)


def _sample(n, k, seed):
    rng = np.random.default_rng(seed)
    idx = rng.choice(n, size=min(k, n), replace=False)
    return np.unique(np.concatenate([idx, [0, n - 1]]))


@pytest.mark.parametrize("name", synth.ALL)
def test_full_size_config(name):
    cfg = synth.CONFIGS[name]
    tag = cfg.seed_tag
    alpha = 0.5
    gran = sq.SQ_PER_TENSOR if cfg.gran == "per_tensor" else sq.SQ_PER_TOKEN
    ogran = oracle.PER_TENSOR if cfg.gran == "per_tensor" else oracle.PER_TOKEN
    _say(f"workload {cfg.name}: drawing inputs on the GPU")
    inp = synth.make(cfg, device=DEV)
    M, K, N = cfg.M, cfg.K, cfg.N
    b = pipeline.W8A8Buffers.allocate(M, N, K, gran, DEV)
    pipeline.smoothquant_w8a8(inp.x, inp.w, inp.calib, alpha, gran, b)
    torch.cuda.synchronize()
    _say("  GPU path done; oracle: channel maxima and factors")

    x, w = _np(inp.x), _np(inp.w)
    amax = oracle.calib_absmax(_np(inp.calib))
    np.testing.assert_array_equal(_np(b.amax_x), amax, err_msg="amax_x")
    aw = oracle.weight_rowmax(w)
    np.testing.assert_array_equal(_np(b.amax_w), aw, err_msg="amax_w")
    s, inv_s = oracle.smooth_factors(amax, aw, alpha)
    np.testing.assert_array_equal(_np(b.s), s, err_msg="s")
    np.testing.assert_array_equal(_np(b.inv_s), inv_s, err_msg="inv_s")

    _say("  oracle: sampled output channels and tokens")
    cols = _sample(N, 96, tag)
    wq_o, ws_o = oracle.quant_weight(np.ascontiguousarray(w[:, cols]), s)
    np.testing.assert_array_equal(_np(b.w_scale)[cols], ws_o, err_msg="w_scale")
    np.testing.assert_array_equal(_np(b.wq)[cols], wq_o, err_msg="wq")

    if ogran == oracle.PER_TENSOR:
        xq_all, xs_o = oracle.quant_act(x, inv_s, ogran)
        np.testing.assert_array_equal(_np(b.x_scale), xs_o, err_msg="x_scale")
        np.testing.assert_array_equal(_np(b.xq), xq_all, err_msg="xq")
        rows = _sample(M, 96, tag + 10)
        xq_o = xq_all[rows]
        xs_rows = xs_o
    else:
        rows = _sample(M, 96, tag + 10)
        xq_o, xs_rows = oracle.quant_act(np.ascontiguousarray(x[rows]), inv_s, ogran)
        np.testing.assert_array_equal(_np(b.x_scale)[rows], xs_rows, err_msg="x_scale")
        np.testing.assert_array_equal(_np(b.xq)[rows], xq_o, err_msg="xq")

    acc_o = oracle.gemm_i8(xq_o, wq_o, nthreads=8)
    _, ybf_o = oracle.dequant(acc_o, xs_rows, ogran, ws_o)
    y_gpu = _np(b.y)[np.ix_(rows, cols)]
    np.testing.assert_array_equal(y_gpu, ybf_o, err_msg="y bf16 (sampled)")
    _say(f"  sampled {len(rows)} tokens x {len(cols)} channels bit-exact")


@pytest.mark.parametrize("name", [synth.ATTN_PROJ, synth.MLP_UP, synth.DECODE, synth.LARGE])
def test_full_size_gemm_freivalds(name):
    """int32 accumulators of the full product: acc . r == Xq . (Wq^T r)."""
    cfg = synth.CONFIGS[name]
    tag = cfg.seed_tag
    M, K, N = cfg.M, cfg.K, cfg.N
    g = torch.Generator(device=DEV)
    g.manual_seed(1000 + tag)
    xq = torch.randint(-127, 128, (M, K), dtype=torch.int8, device=DEV, generator=g)
    wq = torch.randint(-127, 128, (N, K), dtype=torch.int8, device=DEV, generator=g)
    xs = torch.rand(M, device=DEV, generator=g) * 0.01
    ws = torch.rand(N, device=DEV, generator=g) * 0.01
    y = torch.empty(M, N, dtype=torch.bfloat16, device=DEV)
    acc = torch.empty(M, N, dtype=torch.int32, device=DEV)
    sq.sq_gemm_w8a8(xq, xs, sq.SQ_PER_TOKEN, wq, ws, y, acc)
    torch.cuda.synchronize()
    _say(f"workload {cfg.name}: GEMM {M}x{N}x{K} done; Freivalds on the host")
    A = _np(xq).astype(np.int64)
    B = _np(wq).astype(np.int64)
    C = _np(acc).astype(np.int64)
    rng = np.random.default_rng(tag)
    for _ in range(2):
        r = rng.choice(np.array([-1, 1], dtype=np.int64), size=N)
        lhs = C @ r
        rhs = A @ (B.T @ r)
        np.testing.assert_array_equal(lhs, rhs)
    # the bf16 outputs on a sample are the oracle's epilogue of those int32 values
    rows, cols = _sample(M, 64, 7), _sample(N, 64, 8)
    _, ybf = oracle.dequant(np.ascontiguousarray(_np(acc)[np.ix_(rows, cols)]), _np(xs)[rows], oracle.PER_TOKEN,
                            _np(ws)[cols])
    np.testing.assert_array_equal(_np(y)[np.ix_(rows, cols)], ybf)


def test_all_alphas_large_config_factors():
    """Factors for every alpha of the large workload, from one weight pass."""
    cfg = synth.CONFIGS[synth.LARGE]
    K = cfg.K
    g = torch.Generator(device="cpu")
    g.manual_seed(5)
    ax = (torch.rand(K, generator=g) * 300 + 0.01).float()
    aw = (torch.rand(K, generator=g) * 0.1 + 0.001).float()
    for a in cfg.alphas + (0.0, 1.0):
        s_ = torch.empty(K, device=DEV)
        i_ = torch.empty(K, device=DEV)
        sq.sq_smooth_factors(ax.to(DEV), None, a, s_, i_, aw.to(DEV))
        torch.cuda.synchronize()
        so, io = oracle.smooth_factors(ax.numpy(), aw.numpy(), a)
        np.testing.assert_array_equal(_np(s_), so, err_msg=f"s alpha={a}")
        np.testing.assert_array_equal(_np(i_), io, err_msg=f"inv_s alpha={a}")
