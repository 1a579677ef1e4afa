"""The five calls captured into a HIP graph give, on every replay, exactly the
eager results: replays are interleaved with eager passes on other buffers and
with synchronizations, and the captured input tensors are refilled with new
data between replays (the graph reads them where they lie)."""
import pytest
import torch

import post_quantization_act_amd as sq
import synth
from post_quantization_act_amd import pipeline

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
FIELDS = ("amax_x", "amax_w", "s", "inv_s", "wq", "w_scale", "xq", "x_scale", "y")


def _snapshot(b):
    return {f: getattr(b, f).clone() for f in FIELDS}


@pytest.mark.parametrize("gran", [sq.SQ_PER_TOKEN, sq.SQ_PER_TENSOR])
def test_graph_replays_match_eager(gran):
    cfg = synth.CONFIGS[synth.ATTN_PROJ]
    M, K, N = 320, 1024, 768
    a = synth.make(cfg, device=DEV, M=M, K=K, N=N, calib_chunks=2, chunk_tokens=256, variant=0)
    c = synth.make(cfg, device=DEV, M=M, K=K, N=N, calib_chunks=2, chunk_tokens=256, variant=1)
    print(f"graph test gran={gran}", flush=True)

    # eager references on both input sets
    ref_b = pipeline.W8A8Buffers.allocate(M, N, K, gran, DEV)
    pipeline.smoothquant_w8a8(a.x, a.w, a.calib, 0.5, gran, ref_b)
    ref_a = _snapshot(ref_b)
    pipeline.smoothquant_w8a8(c.x, c.w, c.calib, 0.5, gran, ref_b)
    ref_c = _snapshot(ref_b)
    torch.cuda.synchronize()

    # captured pass over its own copies of set a
    x, w, calib = a.x.clone(), a.w.clone(), a.calib.clone()
    b = pipeline.W8A8Buffers.allocate(M, N, K, gran, DEV)
    g = pipeline.CapturedPass(x, w, calib, 0.5, gran, b)
    other = pipeline.W8A8Buffers.allocate(M, N, K, gran, DEV)
    for rep in range(3):
        g.replay()
        torch.cuda.synchronize()
        for f in FIELDS:
            assert torch.equal(getattr(b, f), ref_a[f]), (rep, f)
        # eager work in between on other buffers
        pipeline.smoothquant_w8a8(c.x, c.w, c.calib, 0.5, gran, other)
        torch.cuda.synchronize()
        for f in FIELDS:
            assert torch.equal(getattr(other, f), ref_c[f]), (rep, "eager", f)
    # new data in the captured inputs: the replay computes on it
    x.copy_(c.x)
    w.copy_(c.w)
    calib.copy_(c.calib)
    for rep in range(2):
        g.replay()
        torch.cuda.synchronize()
        for f in FIELDS:
            assert torch.equal(getattr(b, f), ref_c[f]), ("refilled", rep, f)


def test_two_streams_at_once_match_one_stream():
    """Two default-priority streams run the five calls on their own inputs and
    buffers at the same time, several passes each without waiting for the
    other; every result equals the same pass run alone (the library keeps no
    state between calls other than the per-device CU count)."""
    cfg = synth.CONFIGS[synth.ATTN_PROJ]
    M, K, N = 1024, 2048, 2048
    sets = [synth.make(cfg, device=DEV, M=M, K=K, N=N, calib_chunks=2, chunk_tokens=512, variant=v)
            for v in range(2)]
    grans = (sq.SQ_PER_TOKEN, sq.SQ_PER_TENSOR)
    print("two streams", flush=True)
    refs = []
    for s, gran in zip(sets, grans):
        rb = pipeline.W8A8Buffers.allocate(M, N, K, gran, DEV)
        pipeline.smoothquant_w8a8(s.x, s.w, s.calib, 0.6, gran, rb)
        torch.cuda.synchronize()
        refs.append(_snapshot(rb))
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    bufs = [pipeline.W8A8Buffers.allocate(M, N, K, gran, DEV) for gran in grans]
    torch.cuda.synchronize()
    for _ in range(3):
        for s, gran, b, st in zip(sets, grans, bufs, streams):
            pipeline.smoothquant_w8a8(s.x, s.w, s.calib, 0.6, gran, b, stream=st)
    torch.cuda.synchronize()
    for ref, b in zip(refs, bufs):
        got = _snapshot(b)
        for f in FIELDS:
            assert torch.equal(got[f], ref[f]), f
