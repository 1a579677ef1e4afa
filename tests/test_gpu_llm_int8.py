"""LLM.int8()-style mixed-precision comparator on the GPU against the oracle.

The outlier set, its count, the keep mask, the INT8 codes and scales and the
gathered 16-bit operands must equal the oracle's bit for bit.  The output adds
a 16-bit sum that the bf16 matrix cores accumulate in fp32 in their own order,
so it is compared within a bound derived from that arithmetic:

  y16_gpu differs from the exact sum S by at most n16 * 2^-23 * B, where
  B = sum over outlier channels of |x w| (each of at most n16 fp32 additions
  errs by at most 2^-23 of a partial sum bounded by B); the oracle's y16 is S
  rounded once (2^-24 |S|); the final fl(y8 + y16) adds 2^-24 |y| on each
  side.  fp32 output: |dy| <= (n16 + 2) 2^-23 B + 2^-22 |y|.  bf16 output adds
  the two roundings to bf16, 2^-8 |y| each (one bf16 ulp in all).
Cases whose 16-bit half is exact (small integers) are compared bit for bit."""
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


def _bf16_from_np(a):
    return torch.from_numpy(oracle.f32_to_bf16(np.asarray(a, np.float32)).view(np.int16)).view(torch.bfloat16)


def _tolerance(r, n16, out_bf16):
    y = np.abs(r["y32"].astype(np.float64))
    tol = (n16 + 2) * 2.0 ** -23 * r["bound"] + 2.0 ** -22 * y + 1e-38
    if out_bf16:
        tol = tol + 2.0 ** -7 * (y + tol)
    return tol


def _run(x, w, thr, y_dtype=torch.bfloat16):
    M, K = x.shape
    N = w.shape[1]
    b = pipeline.LlmInt8Buffers.allocate(M, N, K, DEV, y_dtype=y_dtype)
    xd, wd = x.to(DEV), w.to(DEV)
    pipeline.llm_int8_prepare(wd, b)
    pipeline.llm_int8_forward(xd, wd, thr, b)
    torch.cuda.synchronize()
    return b


def _compare(b, x, w, thr, out_bf16, rows=None):
    xn, wn = _np(x), _np(w)
    K = xn.shape[1]
    wq, ws = oracle.quant_weight(wn, None)
    assert np.array_equal(b.wq.cpu().numpy(), wq) and np.array_equal(b.w_scale.cpu().numpy(), ws)
    amax = oracle.calib_absmax(xn)
    r = oracle.llm_int8(xn, wn, wq, ws, thr, amax_x=amax, rows=rows)
    n = int(b.count.item())
    idx = r["idx"]
    assert n == idx.size
    np.testing.assert_array_equal(b.idx.cpu().numpy()[:n], idx)
    np.testing.assert_array_equal(b.keep.cpu().numpy(), r["keep"])
    sel = slice(None) if rows is None else np.asarray(rows)
    np.testing.assert_array_equal(b.xq.cpu().numpy()[sel], r["xq"])
    np.testing.assert_array_equal(b.x_scale.cpu().numpy()[sel], r["x_scale"])
    # gathered operands: the outlier columns / rows, zero up to the next multiple of 16
    n16 = (n + 15) // 16 * 16
    xo = _np(b.x_o.cpu())[:, :n16]
    wo = _np(b.w_ot.cpu())[:, :n16]
    want_x = np.zeros((xn.shape[0], n16), np.uint16)
    want_x[:, :n] = xn[:, idx]
    want_w = np.zeros((wn.shape[1], n16), np.uint16)
    want_w[:, :n] = wn[idx, :].T
    np.testing.assert_array_equal(xo, want_x)
    np.testing.assert_array_equal(wo, want_w)
    # output
    y = b.y.cpu()
    y = y.float().numpy() if out_bf16 else y.numpy()
    y = y[sel]
    ref = oracle.bf16_to_f32(r["ybf16"]) if out_bf16 else r["y32"]
    d = np.abs(y.astype(np.float64) - ref.astype(np.float64))
    tol = _tolerance(r, n16, out_bf16)
    bad = np.argwhere(d > tol)
    assert bad.size == 0, f"{len(bad)} outputs beyond the bound, first {bad[:3].tolist()} d={d[tuple(bad[0])]}"
    return n, float((d == 0).mean())


def _outlier_data(M, K, N, n_out, seed, fac=100.0):
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    idx = torch.randperm(K, generator=g)[:n_out]
    f = torch.full((n_out,), fac)
    x = synth.activations(M, K, "normal", idx, f, torch.bfloat16, g, "cpu")
    w = synth.weights(K, N, 0.02, torch.bfloat16, g, "cpu")
    return x, w


@pytest.mark.parametrize("M,K,N,n_out,out_bf16", [
    (256, 512, 256, 5, True),      # ring 128x128 tiles
    (300, 1024, 520, 11, True),    # ring, ragged M and N
    (300, 1024, 520, 11, False),   # fp32 output
    (130, 272, 72, 3, True),       # K % 128 != 0: register-staged kernel
    (513, 2048, 1000, 20, True),   # ring 256x128 tiles, ragged
    (12, 2048, 4096, 20, True),    # M <= 16: general kernel for the outlier variant
    (64, 256, 64, 40, True),       # 40 outliers: three 16-channel steps
    (256, 128, 66536, 5, True),    # 260 tiles of 256 x 256: one whole round + the last columns as 256 x 128
])
def test_llm_int8_matches_oracle(M, K, N, n_out, out_bf16):
    print(f"llm_int8 M={M} K={K} N={N} n_out={n_out} bf16={out_bf16} "
          f"kernel={sq.sq_gemm_outlier_kernel_name(M, N, K)}", flush=True)
    x, w = _outlier_data(M, K, N, n_out, M * 7 + K + N)
    b = _run(x, w, 6.0, torch.bfloat16 if out_bf16 else torch.float32)
    n, exact = _compare(b, x, w, 6.0, out_bf16)
    assert n >= n_out
    print(f"  outliers {n}, bit-identical fraction {exact:.4f}", flush=True)


def test_llm_int8_integer_case_bit_exact():
    """Small-integer inputs make both halves exact (x_scale = w_scale = 1 and
    integer sums below 2^24), so the GPU output equals the oracle's exactly."""
    rng = np.random.default_rng(11)
    for (M, K, N) in [(256, 256, 256), (130, 272, 72), (9, 2048, 128)]:
        print(f"integer case M={M} K={K} N={N}", flush=True)
        out = sorted(rng.choice(K, 9, replace=False).tolist())
        x = rng.integers(-127, 128, (M, K))
        x[:, out] = rng.integers(128, 257, (M, 9)) * rng.choice([-1, 1], (M, 9))
        reg = [j for j in range(K) if j not in out]
        for i in range(M):
            x[i, reg[(3 * i) % len(reg)]] = 127
        w = rng.integers(-127, 128, (K, N))
        for k in range(N):
            w[(7 * k) % K, k] = -127
        xt, wt = _bf16_from_np(x), _bf16_from_np(w)
        b = _run(xt, wt, 127.0, torch.float32)
        want = x.astype(np.int64) @ w.astype(np.int64)
        assert np.abs(want).max() < 2 ** 24
        np.testing.assert_array_equal(b.y.cpu().numpy().astype(np.int64), want)
        _compare(b, xt, wt, 127.0, False)


def test_llm_int8_without_outliers_equals_w8a8():
    """A threshold above every channel leaves count = 0: the output is the
    unsmoothed per-token W8A8 output of the plain GEMM, bit for bit."""
    M, K, N = 200, 1024, 384
    x, w = _outlier_data(M, K, N, 10, 3)
    b = _run(x, w, 1e30)
    assert int(b.count.item()) == 0
    ref = pipeline.W8A8Buffers.allocate(M, N, K, sq.SQ_PER_TOKEN, DEV)
    pipeline.prepare_weights(w.to(DEV), None, ref)
    pipeline.forward(x.to(DEV), sq.SQ_PER_TOKEN, ref, smoothed=False)
    torch.cuda.synchronize()
    assert torch.equal(b.y.view(torch.int16).cpu(), ref.y.view(torch.int16).cpu())


def test_llm_int8_all_outliers():
    """A negative threshold sends every channel to the 16-bit half (the INT8
    codes are all 0); the result is X W within the fp32 summation bound."""
    M, K, N = 96, 256, 160
    x, w = _outlier_data(M, K, N, 3, 5)
    b = _run(x, w, -1.0, torch.float32)
    assert int(b.count.item()) == K
    assert int(b.xq.abs().sum().item()) == 0
    _compare(b, x, w, -1.0, False)


def test_llm_int8_outlier_columns_edges():
    """Selection alone: values equal to the threshold stay regular, chunks of
    the 1024-thread scan with none, some and all channels selected, and a
    ragged last chunk."""
    K = 3088  # three full chunks and a ragged one
    a = np.full(K, 1.0, np.float32)
    a[1024:2048] = 7.0                                    # a chunk that is all outliers
    a[[5, 17, 1023, 2048, 3087]] = [6.0, np.nextafter(np.float32(6), np.float32(7)), 100.0, 6.5, 9.0]
    amax = torch.from_numpy(a).to(DEV)
    idx = torch.full((K,), -1, dtype=torch.int32, device=DEV)
    cnt = torch.zeros(1, dtype=torch.int32, device=DEV)
    keep = torch.empty(K, dtype=torch.float32, device=DEV)
    sq.sq_outlier_columns(amax, 6.0, idx, cnt, keep)
    torch.cuda.synchronize()
    want_idx, want_keep = oracle.outlier_columns(a, 6.0)
    n = int(cnt.item())
    assert n == want_idx.size == 1024 + 4
    np.testing.assert_array_equal(idx.cpu().numpy()[:n], want_idx)
    np.testing.assert_array_equal(keep.cpu().numpy(), want_keep)


def test_llm_int8_empty_and_small():
    """M = 0 enqueues nothing; K = 16 with a single outlier channel."""
    b = pipeline.LlmInt8Buffers.allocate(0, 64, 128, DEV)
    x = torch.empty(0, 128, dtype=torch.bfloat16, device=DEV)
    w = torch.randn(128, 64).to(torch.bfloat16).to(DEV)
    pipeline.llm_int8_prepare(w, b)
    pipeline.llm_int8_forward(x, w, 6.0, b)
    torch.cuda.synchronize()
    x, w = _outlier_data(33, 16, 40, 1, 9)
    b = _run(x, w, 6.0)
    assert int(b.count.item()) >= 1
    _compare(b, x, w, 6.0, True)


def test_llm_int8_attention_projection_full_size():
    """The 2048 x 4096 x 4096 attention-projection workload (41 outlier
    channels x U[50, 150]): the outlier set, codes and gathered operands in
    full, the output on a seeded sample of token rows."""
    inp = synth.make(synth.ATTN_PROJ, with_w=True, calib_chunks=1, chunk_tokens=16)
    print("llm_int8 full size 2048x4096x4096 kernel=" + sq.sq_gemm_outlier_kernel_name(2048, 4096, 4096),
          flush=True)
    b = _run(inp.x, inp.w, 6.0)
    rows = np.sort(np.random.default_rng(1).choice(2048, 12, replace=False))
    n, exact = _compare(b, inp.x, inp.w, 6.0, True, rows=rows)
    assert set(inp.out_idx.tolist()) <= set(b.idx.cpu().numpy()[:n].tolist())
    print(f"  outliers {n}, bit-identical fraction {exact:.4f}", flush=True)


def _random_cases(n, seed):
    """Seeded draws: M in [1, 800], K a multiple of 16 up to 4096, N up to
    3000, 0-60 outlier channels, threshold 3, 6 or 10, bf16 or fp32 output."""
    r = np.random.default_rng(seed)
    return [(int(r.integers(1, 801)), 16 * int(r.integers(1, 257)), int(r.integers(1, 3001)),
             int(r.integers(0, 61)), float(r.choice([3.0, 6.0, 10.0])), bool(r.random() < 0.6)) for _ in range(n)]


@pytest.mark.parametrize("M,K,N,n_out,thr,out_bf16", _random_cases(8, 6060))
def test_llm_int8_random_shapes(M, K, N, n_out, thr, out_bf16):
    print(f"llm_int8 random M={M} K={K} N={N} n_out={n_out} thr={thr} bf16={out_bf16}", flush=True)
    x, w = _outlier_data(M, K, N, min(n_out, K), M * 11 + K + N, fac=40.0)
    b = _run(x, w, thr, torch.bfloat16 if out_bf16 else torch.float32)
    _compare(b, x, w, thr, out_bf16)
