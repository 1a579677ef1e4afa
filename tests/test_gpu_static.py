"""Static per-tensor activation scale on the GPU: the calibrated maximum the
library derives from the channel maxima equals the oracle's direct definition
(max |X'| over the calibration tokens), and codes, scale and the W8A8 output
equal the oracle's bit for bit, including run-time tokens beyond the
calibrated range and rows longer than the register-resident kernels hold."""
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


@pytest.mark.parametrize("M,K,N,T,smoothed,boost", [
    (300, 1024, 520, 512, True, 1.0),     # run-time tokens drawn like the calibration ones
    (257, 4096, 384, 256, True, 4.0),     # run-time outliers 4x the calibrated range: saturation
    (64, 20480, 256, 64, True, 2.0),      # rows beyond 16384 channels (two-pass kernel)
    (40, 512, 136, 128, False, 1.5),      # unsmoothed (inv_s = NULL)
])
def test_static_path_matches_oracle(M, K, N, T, smoothed, boost):
    print(f"static M={M} K={K} N={N} T={T} smoothed={smoothed} boost={boost}", flush=True)
    g = torch.Generator(device="cpu")
    g.manual_seed(M + K + N)
    n_out = max(1, K // 100)
    idx = torch.randperm(K, generator=g)[:n_out]
    fac = torch.full((n_out,), 100.0)
    calib = synth.activations(T, K, "normal", idx, fac, torch.bfloat16, g, "cpu")
    x = synth.activations(M, K, "normal", idx, fac * boost, torch.bfloat16, g, "cpu")
    w = synth.weights(K, N, 0.02, torch.bfloat16, g, "cpu")

    gran = sq.SQ_PER_TENSOR
    b = pipeline.W8A8Buffers.allocate(M, N, K, gran, DEV)
    xd, wd, cd = x.to(DEV), w.to(DEV), calib.to(DEV)
    a_st = torch.empty(1, dtype=torch.float32, device=DEV)
    if smoothed:
        pipeline.calibrate(cd, b.amax_x)
        pipeline.prepare_weights(wd, 0.5, b)
        inv = b.inv_s
    else:
        pipeline.calibrate(cd, b.amax_x)
        pipeline.prepare_weights(wd, None, b)
        inv = None
    sq.sq_static_act_max(b.amax_x, inv, a_st)
    sq.sq_quant_act_static(xd, inv, a_st, b.xq, b.x_scale)
    sq.sq_gemm_w8a8(b.xq, b.x_scale, gran, b.wq, b.w_scale, b.y)
    torch.cuda.synchronize()

    xn, wn, cn = _np(x), _np(w), _np(calib)
    if smoothed:
        s, inv_s = oracle.smooth_factors(oracle.calib_absmax(cn), oracle.weight_rowmax(wn), 0.5)
    else:
        s = inv_s = None
    a = oracle.static_act_max(cn, inv_s)
    assert _np(a_st)[0] == a
    xq_o, xs_o = oracle.quant_act_static(xn, inv_s, a)
    np.testing.assert_array_equal(_np(b.x_scale), xs_o)
    np.testing.assert_array_equal(_np(b.xq), xq_o)
    if boost > 1.0:
        assert (np.abs(xq_o) == 127).sum() >= n_out  # the outlier channels saturate
    wq_o, ws_o = oracle.quant_weight(wn, s)
    np.testing.assert_array_equal(_np(b.wq), wq_o)
    _, ybf = oracle.dequant(oracle.gemm_i8(xq_o, wq_o, nthreads=8), xs_o, oracle.PER_TENSOR, ws_o)
    np.testing.assert_array_equal(_np(b.y), ybf)


def test_static_max_empty_and_zero():
    a = torch.full((1,), 5.0, device=DEV)
    sq.sq_static_act_max(torch.empty(0, device=DEV), None, a)
    torch.cuda.synchronize()
    assert a.item() == 0.0
    x = torch.ones(3, 32, dtype=torch.bfloat16, device=DEV)
    xq = torch.empty(3, 32, dtype=torch.int8, device=DEV)
    xs = torch.empty(1, device=DEV)
    sq.sq_quant_act_static(x, None, a, xq, xs)
    torch.cuda.synchronize()
    assert xs.item() == 0.0 and not xq.any()
