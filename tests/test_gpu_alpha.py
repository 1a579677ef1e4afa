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
