"""sq_quant_weight_noalloc (the library's static scratch instead of a caller
workspace) against sq_quant_weight, through the C ABI, bit for bit: two calls
in a row, the second smaller and with values 100x smaller, so column maxima
left in the scratch by the first call would change the second's scales unless
the call clears them; then an unsmoothed call and a bf16 call at the scratch's
full 65536 columns."""
import numpy as np
import pytest
import torch

import post_quantization_act_amd as sq
import synth

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _w(K, N, scale, dtype, seed):
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    return (synth.weights(K, N, 0.02, torch.float32, g, "cpu") * scale).to(dtype).to(DEV)


def _s(K, seed):
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    return torch.exp(torch.randn(K, generator=g)).float().to(DEV)


def _both(w, s):
    K, N = w.shape
    wq_a = torch.empty(N, K, dtype=torch.int8, device=DEV)
    ws_a = torch.empty(N, dtype=torch.float32, device=DEV)
    wq_b = torch.full((N, K), 7, dtype=torch.int8, device=DEV)
    ws_b = torch.full((N,), -1.0, dtype=torch.float32, device=DEV)
    nb = sq.sq_workspace_size(sq.SQ_OP_QUANT_WEIGHT, 0, N, K)
    wsp = torch.empty(max(nb, 16), dtype=torch.uint8, device=DEV)
    sq.sq_quant_weight(w, s, wq_a, ws_a, wsp)
    sq.sq_quant_weight_noalloc(w, s, wq_b, ws_b)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(ws_b.cpu().numpy(), ws_a.cpu().numpy())
    np.testing.assert_array_equal(wq_b.cpu().numpy(), wq_a.cpu().numpy())


def test_noalloc_matches_quant_weight_twice_then_smaller():
    print("noalloc: 1024 x 12288 bf16, then 512 x 3000 at 1/100 the scale", flush=True)
    _both(_w(1024, 12288, 1.0, torch.bfloat16, 1), _s(1024, 2))
    _both(_w(512, 3000, 0.01, torch.bfloat16, 3), _s(512, 4))


def test_noalloc_unsmoothed_fp32_and_full_scratch():
    print("noalloc: 256 x 1000 fp32 unsmoothed, then 128 x 65536 bf16", flush=True)
    _both(_w(256, 1000, 1.0, torch.float32, 5), None)
    _both(_w(128, 65536, 0.5, torch.bfloat16, 6), _s(128, 7))


def test_noalloc_rejects_more_columns_than_the_scratch():
    w = torch.zeros(16, 65544, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(sq.SqError, match="static scratch"):
        sq.sq_quant_weight_noalloc(w, None, torch.empty(65544, 16, dtype=torch.int8, device=DEV),
                                   torch.empty(65544, dtype=torch.float32, device=DEV))
