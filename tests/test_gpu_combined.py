"""sq_prepare_and_quant_act (steps 2-4 in one call) on the GPU.

It must equal sq_prepare_weights followed by sq_quant_act bit for bit (both
are checked against the oracle elsewhere), on the one-launch path (bf16 W and
X, per token, K <= 4096: weight and activation codes share a launch), on its
fallback to two code launches (K > 4096), and on the inputs that take the two
calls internally; one case is also compared with the oracle directly."""
import numpy as np
import pytest
import torch

import oracle
import post_quantization_act_amd as sq
import synth
from post_quantization_act_amd import pipeline

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _say(msg):
    print(msg, flush=True)


def _np(t):
    return synth.to_numpy(t)


def _inputs(M, K, N, wt, xt, seed):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    n_out = max(1, K // 100)
    idx = torch.randperm(K, generator=g, device=DEV)[:n_out]
    fac = torch.full((n_out,), 80.0, device=DEV)
    x = synth.activations(M, K, "normal", idx, fac, xt, g, DEV)
    w = synth.weights(K, N, 0.02, wt, g, DEV)
    amax = (torch.rand(K, generator=g, device=DEV) * 3 + 0.01).float()
    amax[idx] *= 80.0
    return x, w, amax


def _both(x, w, amax, alpha, gran):
    M, K = x.shape
    N = w.shape[1]
    f32 = dict(dtype=torch.float32, device=DEV)
    outs = []
    for combined in (True, False):
        s, inv_s, aw = torch.empty(K, **f32), torch.empty(K, **f32), torch.empty(K, **f32)
        wq = torch.empty(N, K, dtype=torch.int8, device=DEV)
        w_scale = torch.empty(N, **f32)
        xq = torch.full((M, K), 99, dtype=torch.int8, device=DEV)
        x_scale = torch.empty(1 if gran == sq.SQ_PER_TENSOR else M, **f32)
        if combined:
            nb = sq.sq_workspace_size(sq.SQ_OP_PREPARE_AND_QUANT_ACT, M, N, K, gran)
            ws = torch.empty(max(nb, 16), dtype=torch.uint8, device=DEV)
            sq.sq_prepare_and_quant_act(amax, w, alpha, s, inv_s, aw, wq, w_scale, x, gran, xq, x_scale, ws)
        else:
            nbp = sq.sq_workspace_size(sq.SQ_OP_PREPARE_WEIGHTS, M, N, K, gran)
            nba = sq.sq_workspace_size(sq.SQ_OP_QUANT_ACT, M, N, K, gran)
            wsp = torch.empty(max(nbp, 16), dtype=torch.uint8, device=DEV)
            wsa = torch.empty(max(nba, 16), dtype=torch.uint8, device=DEV) if nba else None
            sq.sq_prepare_weights(amax, w, alpha, s, inv_s, aw, wq, w_scale, wsp)
            sq.sq_quant_act(x, inv_s, gran, xq, x_scale, wsa)
        torch.cuda.synchronize()
        outs.append(dict(s=s, inv_s=inv_s, amax_w=aw, wq=wq, w_scale=w_scale, xq=xq, x_scale=x_scale))
    return outs


CASES = [
    # M, K, N, alpha, W dtype, X dtype, granularity
    (2048, 4096, 4096, 0.5, torch.bfloat16, torch.bfloat16, sq.SQ_PER_TOKEN),   # the attention projection
    (300, 1024, 520, 0.5, torch.bfloat16, torch.bfloat16, sq.SQ_PER_TOKEN),     # one 8-channel group per thread
    (513, 4096, 1000, 0.75, torch.bfloat16, torch.bfloat16, sq.SQ_PER_TOKEN),   # ragged tiles, general alpha
    (1, 256, 64, 1.0, torch.bfloat16, torch.bfloat16, sq.SQ_PER_TOKEN),         # one token
    (4100, 512, 256, 0.5, torch.bfloat16, torch.bfloat16, sq.SQ_PER_TOKEN),     # more rows than row blocks
    (16400, 4096, 256, 0.5, torch.bfloat16, torch.bfloat16, sq.SQ_PER_TOKEN),  # codes above 64 MB: streaming stores
    (64, 4096, 20000, 0.5, torch.bfloat16, torch.bfloat16, sq.SQ_PER_TOKEN),   # weight codes above 64 MB: streaming stores
    (64, 8192, 256, 0.5, torch.bfloat16, torch.bfloat16, sq.SQ_PER_TOKEN),      # K > 4096: two code launches
    (96, 512, 384, 0.5, torch.bfloat16, torch.bfloat16, sq.SQ_PER_TENSOR),      # the two calls
    (96, 512, 384, 0.5, torch.bfloat16, torch.float32, sq.SQ_PER_TOKEN),        # fp32 X: the two calls
    (96, 512, 384, 0.5, torch.float32, torch.bfloat16, sq.SQ_PER_TOKEN),        # fp32 W: the two calls
    (96, 512, 1001, 0.5, torch.bfloat16, torch.bfloat16, sq.SQ_PER_TOKEN),      # N % 8 != 0: the two calls
    (0, 512, 384, 0.5, torch.bfloat16, torch.bfloat16, sq.SQ_PER_TOKEN),        # empty batch: weights only
]


@pytest.mark.parametrize("M,K,N,alpha,wt,xt,gran", CASES)
def test_combined_equals_two_calls(M, K, N, alpha, wt, xt, gran):
    _say(f"prepare_and_quant_act M={M} K={K} N={N} alpha={alpha} w={wt} x={xt} gran={gran}")
    x, w, amax = _inputs(M, K, N, wt, xt, M * 131 + K * 7 + N)
    a, b = _both(x, w, amax, alpha, gran)
    for name in a:
        assert torch.equal(a[name].view(torch.int8) if a[name].dtype == torch.int8 else a[name].view(torch.int32),
                           b[name].view(torch.int8) if b[name].dtype == torch.int8 else b[name].view(torch.int32)), name


def test_combined_matches_oracle():
    """A small one-launch case straight against the oracle's steps 2-4."""
    M, K, N = 130, 512, 264
    x, w, amax = _inputs(M, K, N, torch.bfloat16, torch.bfloat16, 77)
    a, _ = _both(x, w, amax, 0.5, sq.SQ_PER_TOKEN)
    xn, wn, an = _np(x), _np(w), _np(amax)
    aw = oracle.weight_rowmax(wn)
    s, inv_s = oracle.smooth_factors(an, aw, 0.5)
    np.testing.assert_array_equal(_np(a["amax_w"]), aw)
    np.testing.assert_array_equal(_np(a["s"]), s)
    np.testing.assert_array_equal(_np(a["inv_s"]), inv_s)
    wq, ws = oracle.quant_weight(wn, s)
    np.testing.assert_array_equal(_np(a["wq"]), wq)
    np.testing.assert_array_equal(_np(a["w_scale"]), ws)
    xq, xs = oracle.quant_act(xn, inv_s, oracle.PER_TOKEN)
    np.testing.assert_array_equal(_np(a["xq"]), xq)
    np.testing.assert_array_equal(_np(a["x_scale"]), xs)


def test_pipeline_fused_equals_unfused():
    """smoothquant_w8a8 through the combined call equals the separate calls, output included."""
    M, K, N = 256, 1024, 512
    inp = synth.make(synth.ATTN_PROJ, device=DEV, M=M, K=K, N=N, calib_chunks=2, chunk_tokens=128)
    ys = []
    for fused in (True, False):
        b = pipeline.W8A8Buffers.allocate(M, N, K, sq.SQ_PER_TOKEN, DEV)
        pipeline.smoothquant_w8a8(inp.x, inp.w, inp.calib, 0.5, sq.SQ_PER_TOKEN, b, fused=fused)
        torch.cuda.synchronize()
        ys.append(b.y.view(torch.int16).clone())
    assert torch.equal(ys[0], ys[1])


def test_combined_weight_rows_not_aligned():
    """W as a view with an odd row stride (rows not 16-byte aligned) takes the two calls."""
    M, K, N = 64, 256, 200
    x, w, amax = _inputs(M, K, N, torch.bfloat16, torch.bfloat16, 5)
    wide = torch.zeros(K, N + 3, dtype=torch.bfloat16, device=DEV)
    wide[:, :N] = w
    wv = wide[:, :N]
    assert wv.stride(0) == N + 3
    a, b = _both(x, wv, amax, 0.5, sq.SQ_PER_TOKEN)
    for name in a:
        assert torch.equal(a[name], b[name]), name
