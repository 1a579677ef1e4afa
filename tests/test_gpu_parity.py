"""GPU parity: every output of the HIP path equals the CPU oracle's, bit for
bit, on the same seeded inputs (codes, scales, factors, int32 accumulators,
fp32 and bf16 outputs).  Shapes span several tiles of every kernel and end in
ragged tails; edge cases cover empty inputs, all-zero rows, alpha = 0 and 1,
fp32 and bf16 inputs, per-token and per-tensor scales, K beyond the
register-resident activation path, and every finite bf16 bit pattern."""
import json
import os

import numpy as np
import pytest
import torch

import oracle
import post_quantization_act_amd as sq
import synth
from post_quantization_act_amd import pipeline

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _np(t):
    return synth.to_numpy(t)


def _say(msg):
    print(msg, flush=True)


def _run_gpu(x, w, calib, alpha, gran, y_dtype=torch.bfloat16, with_acc=True):
    M, K = x.shape
    N = w.shape[1]
    b = pipeline.W8A8Buffers.allocate(M, N, K, gran, DEV, y_dtype=y_dtype, with_acc=with_acc)
    pipeline.smoothquant_w8a8(x, w, calib, alpha, gran, b)
    torch.cuda.synchronize()
    return b


def _compare(b, o, alpha, y_dtype):
    if alpha is not None:
        np.testing.assert_array_equal(_np(b.amax_x), o["amax_x"], err_msg="amax_x")
        np.testing.assert_array_equal(_np(b.amax_w), o["amax_w"], err_msg="amax_w")
        np.testing.assert_array_equal(_np(b.s), o["s"], err_msg="s")
        np.testing.assert_array_equal(_np(b.inv_s), o["inv_s"], err_msg="inv_s")
    np.testing.assert_array_equal(_np(b.w_scale), o["w_scale"], err_msg="w_scale")
    np.testing.assert_array_equal(_np(b.wq), o["wq"], err_msg="wq")
    np.testing.assert_array_equal(_np(b.x_scale), o["x_scale"], err_msg="x_scale")
    np.testing.assert_array_equal(_np(b.xq), o["xq"], err_msg="xq")
    if b.acc is not None:
        np.testing.assert_array_equal(_np(b.acc), o["acc"], err_msg="acc")
    if y_dtype == torch.bfloat16:
        np.testing.assert_array_equal(_np(b.y), o["ybf16"], err_msg="y bf16")
    else:
        np.testing.assert_array_equal(_np(b.y), o["y32"], err_msg="y fp32")


def _inputs(M, K, N, dtype, seed, n_out=None, factor=100.0, T=None, kind="normal"):
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    n_out = max(1, K // 100) if n_out is None else n_out
    idx = torch.randperm(K, generator=g)[:n_out]
    fac = torch.full((n_out,), factor)
    x = synth.activations(M, K, kind, idx, fac, dtype, g, "cpu")
    w = synth.weights(K, N, 0.02, dtype, g, "cpu")
    calib = synth.activations(T if T is not None else max(M, 1), K, kind, idx, fac, dtype, g, "cpu")
    return x, w, calib


CASES = [
    # M, K, N, dtype, gran, alpha, T
    (1, 16, 1, torch.bfloat16, sq.SQ_PER_TOKEN, 0.5, 3),
    (7, 48, 5, torch.float32, sq.SQ_PER_TENSOR, 0.5, 9),
    (129, 272, 300, torch.bfloat16, sq.SQ_PER_TOKEN, 0.5, 200),
    (300, 144, 260, torch.bfloat16, sq.SQ_PER_TENSOR, 0.75, 77),
    (64, 4112, 136, torch.bfloat16, sq.SQ_PER_TOKEN, 0.4, 130),
    (33, 16400, 40, torch.bfloat16, sq.SQ_PER_TOKEN, 0.5, 40),
    (5, 8192, 24, torch.float32, sq.SQ_PER_TOKEN, 1.0, 17),
    (256, 256, 512, torch.bfloat16, sq.SQ_PER_TOKEN, 0.0, 512),
    (130, 1024, 257, torch.bfloat16, sq.SQ_PER_TOKEN, 0.6, 1000),
    (520, 512, 130, torch.float32, sq.SQ_PER_TENSOR, 0.5, 64),
    (96, 12288, 200, torch.bfloat16, sq.SQ_PER_TOKEN, 0.5, 300),
    # 256 x 128 GEMM path (three-stage ring), ragged M and N, three stages (prologue only)
    (2100, 384, 3000, torch.bfloat16, sq.SQ_PER_TOKEN, 0.5, 512),
    # 256 x 128 path, ragged M, N % 4 != 0 (element-wise output stores), eight stages
    (2000, 1024, 3998, torch.bfloat16, sq.SQ_PER_TOKEN, 0.5, 256),
    # 128 x 128 path (258 tiles of 256 x 128 would need two rounds over 256 CUs), N < 128
    (33000, 384, 100, torch.bfloat16, sq.SQ_PER_TOKEN, 0.5, 256),
    # enough output tiles for the 256 x 256 GEMM path, ragged M, N % 4 != 0, three stages
    (4100, 384, 16398, torch.bfloat16, sq.SQ_PER_TOKEN, 0.5, 256),
    # exactly one round of 256 x 256 tiles over 256 CUs, two stages
    (4096, 256, 4096, torch.bfloat16, sq.SQ_PER_TOKEN, 0.5, 256),
    # decode path (M <= 16): ragged N, K not a multiple of 64, per-tensor scale
    (16, 1040, 100, torch.bfloat16, sq.SQ_PER_TOKEN, 0.5, 64),
    # LDS-ring decode path (K % 2048 == 0): 257 channel groups over 256 blocks, per-tensor
    (9, 4096, 4100, torch.bfloat16, sq.SQ_PER_TENSOR, 0.5, 64),
    # ring decode: N % 4 != 0 (element-wise stores), 63 groups
    (16, 2048, 1001, torch.bfloat16, sq.SQ_PER_TOKEN, 0.5, 64),
    # ring decode: one token, K = 16384 (eight stages per wavefront), per-tensor
    (1, 16384, 300, torch.bfloat16, sq.SQ_PER_TENSOR, 0.5, 16),
    # ring decode: 7 channel groups per block, ragged last group
    (16, 4096, 28000, torch.bfloat16, sq.SQ_PER_TOKEN, 0.5, 64),
    # ring decode: 10 channel groups per block, 13 tokens
    (13, 2048, 37000, torch.bfloat16, sq.SQ_PER_TOKEN, 0.5, 64),
    # ring decode: 513 groups, so one block takes three; K = 6144
    (12, 6144, 8200, torch.bfloat16, sq.SQ_PER_TOKEN, 0.5, 64),
    # K a multiple of 16 but not of 128: register-staged GEMM path with a K tail
    (300, 1040, 520, torch.bfloat16, sq.SQ_PER_TENSOR, 0.5, 300),
    # 260 tiles of 256 x 256: one whole round on the first 65536 columns, the last 1000 as 256 x 128 tiles
    (256, 128, 66536, torch.bfloat16, sq.SQ_PER_TOKEN, 0.5, 64),
    # the same split with N % 4 != 0 (element-wise stores in both launches)
    (256, 128, 66538, torch.bfloat16, sq.SQ_PER_TOKEN, 0.5, 64),
]


@pytest.mark.parametrize("M,K,N,dtype,gran,alpha,T", CASES)
@pytest.mark.parametrize("y_dtype", [torch.bfloat16, torch.float32])
def test_pipeline_matches_oracle(M, K, N, dtype, gran, alpha, T, y_dtype):
    _say(f"case M={M} K={K} N={N} {dtype} gran={gran} alpha={alpha} T={T} y={y_dtype}")
    x, w, calib = _inputs(M, K, N, dtype, seed=M * 7 + K * 3 + N, T=T)
    b = _run_gpu(x.to(DEV), w.to(DEV), calib.to(DEV), alpha, gran, y_dtype)
    o = oracle.w8a8_linear(_np(x), _np(w), alpha, gran, calib=_np(calib), nthreads=8)
    _compare(b, o, alpha, y_dtype)


def _random_cases(n, seed):
    """n seeded draws over the path's shape space: M in [1, 700], K a multiple
    of 16 in [16, 3072], N in [1, 1200] (a third of them multiples of 8),
    bf16 or fp32 inputs, either granularity, alpha from a grid, the deployed
    or the accumulator-storing epilogue."""
    r = np.random.default_rng(seed)
    out = []
    for i in range(n):
        M = int(r.integers(1, 701))
        K = 16 * int(r.integers(1, 193))
        N = int(r.integers(1, 1201))
        if i % 3 == 0:
            N = 8 * max(1, N // 8)
        dtype = torch.bfloat16 if r.random() < 0.75 else torch.float32
        gran = sq.SQ_PER_TOKEN if r.random() < 0.7 else sq.SQ_PER_TENSOR
        alpha = float(r.choice([0.0, 0.25, 0.4, 0.5, 0.6, 0.75, 0.85, 1.0]))
        T = int(r.integers(1, 400))
        out.append((M, K, N, dtype, gran, alpha, T, bool(r.random() < 0.5)))
    return out


@pytest.mark.parametrize("M,K,N,dtype,gran,alpha,T,with_acc", _random_cases(16, 20261203))
def test_random_shapes_match_oracle(M, K, N, dtype, gran, alpha, T, with_acc):
    """Seeded random shapes, every output compared with the oracle's."""
    _say(f"random M={M} K={K} N={N} {dtype} gran={gran} alpha={alpha} T={T} acc={with_acc}")
    x, w, calib = _inputs(M, K, N, dtype, seed=M + 13 * K + 7 * N, T=T)
    b = _run_gpu(x.to(DEV), w.to(DEV), calib.to(DEV), alpha, gran, torch.bfloat16, with_acc=with_acc)
    o = oracle.w8a8_linear(_np(x), _np(w), alpha, gran, calib=_np(calib), nthreads=8)
    _compare(b, o, alpha, torch.bfloat16)


# Shapes whose bf16 output takes the LDS-staged epilogue (N % 8 == 0, no int32
# accumulator store) with ragged edges, one per tile launch: (M, K, N, the
# kernel-name fragment the shape must select).
DEPLOYED_EPILOGUE = [
    (4100, 384, 16392, "k_gemm_ring<256,256,4,2,2> (256x256"),        # 256 x 256 tiles, ragged M
    (4100, 512, 8200, "k_gemm_persist<256,256,4,2,2>"),               # persistent 256 x 256, ragged M and N
    (500, 128, 66536, "on the remaining columns"),                   # column split, ragged M and last launch
    (2100, 384, 3000, "k_gemm_ring<256,128,4,2,3> (256x128"),        # 256 x 128 tiles, ragged M and N
    (33000, 256, 104, "k_gemm_ring<128,128,2,4,2>"),                 # 128 x 128 tiles, N < one tile
]


@pytest.mark.parametrize("M,K,N,dtype,gran,alpha,T", CASES)
def test_deployed_epilogue_matches_oracle(M, K, N, dtype, gran, alpha, T):
    """The call as deployed: bf16 output and no int32 accumulator store, so the
    ring kernels take their LDS-staged bf16 epilogue wherever N % 8 == 0;
    every output element against the oracle's."""
    _say(f"deployed case M={M} K={K} N={N} {dtype} gran={gran} alpha={alpha} T={T}")
    x, w, calib = _inputs(M, K, N, dtype, seed=M * 7 + K * 3 + N + 1, T=T)
    b = _run_gpu(x.to(DEV), w.to(DEV), calib.to(DEV), alpha, gran, torch.bfloat16, with_acc=False)
    o = oracle.w8a8_linear(_np(x), _np(w), alpha, gran, calib=_np(calib), nthreads=8)
    _compare(b, o, alpha, torch.bfloat16)


@pytest.mark.parametrize("M,K,N,kernel", DEPLOYED_EPILOGUE)
def test_deployed_epilogue_ragged_tiles(M, K, N, kernel):
    """Ragged M and N with N % 8 == 0 on each tile launch of the GEMM, bf16
    output, no accumulator store: the LDS-staged epilogue's edge handling,
    compared element by element with the oracle."""
    _say(f"deployed ragged M={M} K={K} N={N}")
    assert kernel in sq.sq_gemm_kernel_name(M, N, K)
    x, w, calib = _inputs(M, K, N, torch.bfloat16, seed=M + 11 * N + K, T=256)
    b = _run_gpu(x.to(DEV), w.to(DEV), calib.to(DEV), 0.5, sq.SQ_PER_TOKEN, torch.bfloat16, with_acc=False)
    o = oracle.w8a8_linear(_np(x), _np(w), 0.5, sq.SQ_PER_TOKEN, calib=_np(calib), nthreads=8)
    _compare(b, o, 0.5, torch.bfloat16)


@pytest.mark.parametrize("gran", [sq.SQ_PER_TOKEN, sq.SQ_PER_TENSOR])
def test_unsmoothed_baseline_matches_oracle(gran):
    x, w, calib = _inputs(200, 320, 150, torch.bfloat16, seed=5)
    b = _run_gpu(x.to(DEV), w.to(DEV), None, None, gran)
    o = oracle.w8a8_linear(_np(x), _np(w), None, gran, nthreads=8)
    _compare(b, o, None, torch.bfloat16)


@pytest.mark.parametrize("gran,key", [(sq.SQ_PER_TENSOR, "per_tensor_act_per_channel_w"),
                                      (sq.SQ_PER_TOKEN, "per_token_act_per_channel_w")])
def test_worked_example_on_gpu(gran, key):
    """The page's 3x3 example, zero-padded to K = 16 input channels (padding
    channels are all zero, so they change no maximum and no product)."""
    g = json.load(open(os.path.join(GOLD, "worked_example.json")))
    X = np.zeros((3, 16), np.float32)
    W = np.zeros((16, 2), np.float32)
    X[:, :3] = np.array(g["X"], np.float32)
    W[:3, :] = np.array(g["W"], np.float32)
    xt, wt = torch.from_numpy(X).to(DEV), torch.from_numpy(W).to(DEV)
    b = _run_gpu(xt, wt, xt, g["alpha"], gran, torch.float32)
    o = oracle.w8a8_linear(X, W, g["alpha"], gran)
    _compare(b, o, g["alpha"], torch.float32)
    Y = oracle.matmul_f64(X, W)
    e = g["relative_error_percent"][key]
    assert round(100 * oracle.rel_fro(_np(b.y), Y), e["after_decimals"]) == e["after"]
    base = _run_gpu(xt, wt, None, None, gran, torch.float32)
    assert round(100 * oracle.rel_fro(_np(base.y), Y), e["before_decimals"]) == e["before"]
    if gran == sq.SQ_PER_TENSOR:
        assert _np(b.xq)[:, 0].tolist() == g["channel1_codes"]["after"]
        assert _np(base.xq)[:, 0].tolist() == g["channel1_codes"]["before"]


def _finite_bf16_patterns():
    p = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    finite = ((p.astype(np.uint32) >> 7) & 0xFF) != 0xFF
    return p[finite]


@pytest.mark.parametrize("inv_scale", ["ones", "pow2", "random"])
def test_exhaustive_bf16_element_map_activations(inv_scale):
    """Every finite bf16 pattern goes through smoothing and coding, per token
    (inverse factors <= 1 keep every smoothed value finite).  The first rows
    hold only subnormal and tiny values, where 127/max overflows."""
    pats = _finite_bf16_patterns()
    K = 256
    rows = -(-pats.size // K)
    buf = np.zeros(rows * K, np.uint16)
    buf[:pats.size] = pats
    X = buf.reshape(rows, K)
    rng = np.random.default_rng(1)
    if inv_scale == "ones":
        inv = np.ones(K, np.float32)
    elif inv_scale == "pow2":
        inv = (2.0 ** rng.integers(-20, 1, K)).astype(np.float32)
    else:
        inv = rng.uniform(1e-3, 1.0, K).astype(np.float32)
    xt = torch.from_numpy(X.view(np.int16)).view(torch.bfloat16).to(DEV)
    it = torch.from_numpy(inv).to(DEV)
    xq = torch.empty(rows, K, dtype=torch.int8, device=DEV)
    xs = torch.empty(rows, dtype=torch.float32, device=DEV)
    sq.sq_quant_act(xt, it, sq.SQ_PER_TOKEN, xq, xs)
    torch.cuda.synchronize()
    oq, os_ = oracle.quant_act(X, inv, oracle.PER_TOKEN)
    np.testing.assert_array_equal(_np(xs), os_)
    np.testing.assert_array_equal(_np(xq), oq)


def test_exhaustive_bf16_element_map_weights():
    """Every finite bf16 pattern goes through weight smoothing and coding."""
    pats = _finite_bf16_patterns()
    N = 128
    K = -(-pats.size // N)
    K = (K + 15) // 16 * 16
    buf = np.zeros(K * N, np.uint16)
    buf[:pats.size] = pats
    W = buf.reshape(K, N)
    s = np.random.default_rng(2).uniform(0.25, 1.0, K).astype(np.float32)
    wt = torch.from_numpy(W.view(np.int16)).view(torch.bfloat16).to(DEV)
    st = torch.from_numpy(s).to(DEV)
    wq = torch.empty(N, K, dtype=torch.int8, device=DEV)
    ws = torch.empty(N, dtype=torch.float32, device=DEV)
    work = torch.empty(sq.sq_workspace_size(sq.SQ_OP_QUANT_WEIGHT, 0, N, K), dtype=torch.uint8, device=DEV)
    sq.sq_quant_weight(wt, st, wq, ws, work)
    torch.cuda.synchronize()
    oq, os_ = oracle.quant_weight(W, s)
    np.testing.assert_array_equal(_np(ws), os_)
    np.testing.assert_array_equal(_np(wq), oq)


def test_calibration_chunks_and_resume():
    x, w, calib = _inputs(8, 1024, 8, torch.bfloat16, seed=3, T=1000)
    ct = calib.to(DEV)
    a1 = torch.zeros(1024, device=DEV)
    sq.sq_calib_absmax(ct, a1)
    a2 = torch.zeros(1024, device=DEV)
    for part in torch.split(ct, [1, 300, 77, 622]):
        sq.sq_calib_absmax(part, a2)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(_np(a1), _np(a2))
    np.testing.assert_array_equal(_np(a1), oracle.calib_absmax(_np(calib)))
    sq.sq_calib_absmax(ct, a1)  # idempotent
    torch.cuda.synchronize()
    np.testing.assert_array_equal(_np(a1), _np(a2))
    # sq_calib_reset starts a new calibration: a larger earlier maximum is gone
    a2.fill_(1e30)
    sq.sq_calib_reset(a2)
    sq.sq_calib_absmax(ct, a2)
    odd = torch.full((1000 + 16,), 7.0, device=DEV)  # a length that is no multiple of the fill block
    sq.sq_calib_reset(odd[:1000])
    torch.cuda.synchronize()
    np.testing.assert_array_equal(_np(a2), _np(a1))
    assert not odd[:1000].any() and bool((odd[1000:] == 7.0).all())


def test_strided_inputs():
    """Row strides larger than the row (views into wider buffers)."""
    x, w, calib = _inputs(70, 256, 96, torch.bfloat16, seed=9, T=100)
    xw = torch.zeros(70, 256 + 64, dtype=torch.bfloat16)
    xw[:, :256] = x
    ww = torch.zeros(256, 96 + 8, dtype=torch.bfloat16)
    ww[:, :96] = w
    cw = torch.zeros(100, 256 + 16, dtype=torch.bfloat16)
    cw[:, :256] = calib
    b = _run_gpu(xw.to(DEV)[:, :256], ww.to(DEV)[:, :96], cw.to(DEV)[:, :256], 0.5, sq.SQ_PER_TOKEN)
    o = oracle.w8a8_linear(_np(x), _np(w), 0.5, oracle.PER_TOKEN, calib=_np(calib))
    _compare(b, o, 0.5, torch.bfloat16)


@pytest.mark.parametrize("dtype,N,pad", [(torch.bfloat16, 100, 4), (torch.float32, 101, 3), (torch.bfloat16, 8, 0)])
def test_strided_weight_ragged_columns(dtype, N, pad):
    """16-byte aligned weight rows with N % 8 != 0 (the last 8-column group of a
    row is partly past N) and K not a multiple of the 128-row weight tile."""
    K = 208
    x, w, calib = _inputs(70, K, N, dtype, seed=13, T=90)
    ww = torch.zeros(K, N + pad, dtype=dtype)
    ww[:, :N] = w
    b = _run_gpu(x.to(DEV), ww.to(DEV)[:, :N], calib.to(DEV), 0.5, sq.SQ_PER_TOKEN)
    o = oracle.w8a8_linear(_np(x), _np(w), 0.5, oracle.PER_TOKEN, calib=_np(calib))
    _compare(b, o, 0.5, torch.bfloat16)


def test_zero_rows_and_columns():
    x, w, calib = _inputs(40, 128, 70, torch.bfloat16, seed=4, T=40)
    x[3] = 0
    x[:, 5] = 0
    calib[:, 5] = 0   # dead input channel: floored maxima
    w[:, 9] = 0       # dead output channel: scale 0, codes 0, y = 0
    w[17] = 0
    b = _run_gpu(x.to(DEV), w.to(DEV), calib.to(DEV), 0.5, sq.SQ_PER_TOKEN)
    o = oracle.w8a8_linear(_np(x), _np(w), 0.5, oracle.PER_TOKEN, calib=_np(calib))
    _compare(b, o, 0.5, torch.bfloat16)
    assert float(_np(b.x_scale)[3]) == 0.0
    assert float(_np(b.w_scale)[9]) == 0.0


def test_k_zero_and_empty():
    # K = 0: scales are 0 and y = 0
    xq = torch.empty(4, 0, dtype=torch.int8, device=DEV)
    wq = torch.empty(3, 0, dtype=torch.int8, device=DEV)
    xs = torch.ones(4, device=DEV)
    ws = torch.ones(3, device=DEV)
    y = torch.full((4, 3), 7.0, dtype=torch.float32, device=DEV)
    sq.sq_gemm_w8a8(xq, xs, sq.SQ_PER_TOKEN, wq, ws, y)
    torch.cuda.synchronize()
    assert (y == 0).all()
    # M = 0 and T = 0 do nothing
    amax = torch.full((32,), 3.0, device=DEV)
    sq.sq_calib_absmax(torch.empty(0, 32, dtype=torch.bfloat16, device=DEV), amax)
    torch.cuda.synchronize()
    assert (amax == 3.0).all()


def test_determinism_repeat_runs():
    x, w, calib = _inputs(512, 2048, 1024, torch.bfloat16, seed=12, T=1024)
    xd, wd, cd = x.to(DEV), w.to(DEV), calib.to(DEV)
    b1 = _run_gpu(xd, wd, cd, 0.5, sq.SQ_PER_TOKEN)
    b2 = _run_gpu(xd, wd, cd, 0.5, sq.SQ_PER_TOKEN)
    for name in ("amax_x", "s", "wq", "w_scale", "xq", "x_scale", "acc", "y"):
        assert torch.equal(getattr(b1, name), getattr(b2, name)), name


PREP_CASES = [
    # K, N, alpha, dtype.  bf16 W with N % 8 == 0 takes the one-read pass: every
    # row layout of it (rows per iteration x 8-column groups per thread), both
    # factor kinds (alpha in {0, 1/2, 1} without pow, others with it), ragged rows
    # per block, blocks with fewer rows than one iteration takes, ragged groups.
    (131072, 1024, 0.5, torch.bfloat16),  # 4 rows per iteration, one group, 512 blocks of 256 rows
    (65536, 2048, 0.75, torch.bfloat16),  # 4 rows, two groups, general alpha
    (32768, 4096, 0.5, torch.bfloat16),   # 4 rows, four groups
    (4096, 4096, 0.5, torch.bfloat16),    # the attention-projection weight: 16 rows per block
    (16384, 8192, 0.4, torch.bfloat16),   # 4 rows, eight groups, general alpha
    (2000, 8192, 1.0, torch.bfloat16),    # 4 rows, eight groups, 8 rows per block (250 blocks)
    (8192, 16384, 0.0, torch.bfloat16),   # 2 rows, eight groups, alpha = 0
    (3008, 16376, 0.3, torch.bfloat16),   # 2 rows, eight groups (the last partly masked), general alpha
    (304, 800, 0.5, torch.bfloat16),      # 2 rows per block for 4 row slots: two slots idle
    (16, 4096, 1.0, torch.bfloat16),      # one row per block
    (1008, 2048, 0.75, torch.bfloat16),   # 4 rows per block, general alpha
    (5472, 24576, 1.0, torch.bfloat16),   # six groups, alpha = 1, 22 rows per block, last block 16
    (5472, 24600, 0.5, torch.bfloat16),   # 3075 groups: eight per thread, the last ones partly masked
    (4096, 32768, 0.6, torch.bfloat16),   # eight groups, general alpha
    (2736, 49152, 0.5, torch.bfloat16),   # 1024 threads, six groups: 5 in registers, 1 in LDS
    (1504, 3000, 0.5, torch.bfloat16),    # 1024 threads, 4 rows, two groups (375 of 512 used)
    (784, 6000, 1.0, torch.bfloat16),     # 1024 threads, 4 rows, four groups (750 of 1024 used)
    (3008, 12000, 0.0, torch.bfloat16),   # 1024 threads, 2 rows, four groups (1500 of 2048 used)
    (1008, 20000, 0.5, torch.bfloat16),   # 1024 threads, 1 row, three groups (2500 of 3072 used)
    (3408, 40008, 1.0, torch.bfloat16),   # 5001 groups over 1024 threads: the LDS group partly masked
    # the two-call sequence: general alpha beyond 32768 columns, N % 8 != 0, fp32
    (304, 1001, 0.5, torch.bfloat16),
    (2736, 49152, 0.75, torch.bfloat16),
    (112, 1001, 0.5, torch.bfloat16),
    (208, 512, 0.5, torch.float32),
]


@pytest.mark.parametrize("K,N,alpha,dtype", PREP_CASES)
def test_prepare_weights_matches_two_calls(K, N, alpha, dtype):
    """sq_prepare_weights == sq_smooth_factors + sq_quant_weight, bit for bit, and
    both equal the oracle (factors in full, codes on sampled channels)."""
    _say(f"prepare_weights K={K} N={N} alpha={alpha} {dtype}")
    g = torch.Generator(device=DEV)
    g.manual_seed(K * 31 + N)
    n_out = max(1, K // 100)
    idx = torch.randperm(K, generator=g, device=DEV)[:n_out]
    wd = synth.weights(K, N, 0.02, dtype, g, DEV)
    wd[idx[: max(1, n_out // 2)]] *= 8.0  # a few heavy weight rows (exact in bf16)
    ad = (torch.rand(K, generator=g, device=DEV) * 3 + 0.01).float()
    ad[idx] *= 100.0
    f32 = dict(dtype=torch.float32, device=DEV)
    res = []
    for fused in (True, False):
        s_, i_, aw = torch.empty(K, **f32), torch.empty(K, **f32), torch.empty(K, **f32)
        wq = torch.empty(N, K, dtype=torch.int8, device=DEV)
        wsc = torch.empty(N, **f32)
        if fused:
            ws = torch.empty(sq.sq_workspace_size(sq.SQ_OP_PREPARE_WEIGHTS, 0, N, K), dtype=torch.uint8, device=DEV)
            sq.sq_prepare_weights(ad, wd, alpha, s_, i_, aw, wq, wsc, ws)
        else:
            ws = torch.empty(sq.sq_workspace_size(sq.SQ_OP_QUANT_WEIGHT, 0, N, K), dtype=torch.uint8, device=DEV)
            sq.sq_smooth_factors(ad, wd, alpha, s_, i_, aw)
            sq.sq_quant_weight(wd, s_, wq, wsc, ws)
        torch.cuda.synchronize()
        res.append((s_, i_, aw, wq, wsc))
        del ws
    for a, b, name in zip(res[0], res[1], ("s", "inv_s", "amax_w", "wq", "w_scale")):
        assert torch.equal(a, b), name
    w = _np(wd)
    aw_o = oracle.weight_rowmax(w)
    s_o, i_o = oracle.smooth_factors(_np(ad), aw_o, alpha)
    np.testing.assert_array_equal(_np(res[0][2]), aw_o)
    np.testing.assert_array_equal(_np(res[0][0]), s_o)
    np.testing.assert_array_equal(_np(res[0][1]), i_o)
    cols = np.unique(np.linspace(0, N - 1, 24).astype(int))
    wq_o, ws_o = oracle.quant_weight(np.ascontiguousarray(w[:, cols]), s_o)
    np.testing.assert_array_equal(_np(res[0][4])[cols], ws_o)
    np.testing.assert_array_equal(_np(res[0][3])[cols], wq_o)


def test_prepare_weights_without_amax_w_and_empty():
    K, N = 256, 768
    g = torch.Generator(device="cpu")
    g.manual_seed(9)
    w = synth.weights(K, N, 0.02, torch.bfloat16, g, "cpu").to(DEV)
    ax = (torch.rand(K, generator=g) + 0.1).float().to(DEV)
    f32 = dict(dtype=torch.float32, device=DEV)
    s1, i1, s2, i2 = (torch.empty(K, **f32) for _ in range(4))
    wq1, wq2 = (torch.empty(N, K, dtype=torch.int8, device=DEV) for _ in range(2))
    w1, w2 = torch.empty(N, **f32), torch.empty(N, **f32)
    ws = torch.empty(sq.sq_workspace_size(sq.SQ_OP_PREPARE_WEIGHTS, 0, N, K), dtype=torch.uint8, device=DEV)
    sq.sq_prepare_weights(ax, w, 0.5, s1, i1, None, wq1, w1, ws)
    ws2 = torch.empty(sq.sq_workspace_size(sq.SQ_OP_QUANT_WEIGHT, 0, N, K), dtype=torch.uint8, device=DEV)
    sq.sq_smooth_factors(ax, w, 0.5, s2, i2, None)
    sq.sq_quant_weight(w, s2, wq2, w2, ws2)
    torch.cuda.synchronize()
    assert torch.equal(s1, s2) and torch.equal(wq1, wq2) and torch.equal(w1, w2)
    # K = 0: every scale is 0
    w0 = torch.empty(0, 8, dtype=torch.bfloat16, device=DEV)
    e = torch.empty(0, **f32)
    wsc = torch.full((8,), 7.0, **f32)
    sq.sq_prepare_weights(e, w0, 0.5, e, e, None, torch.empty(8, 0, dtype=torch.int8, device=DEV), wsc, None)
    torch.cuda.synchronize()
    assert torch.equal(wsc, torch.zeros(8, **f32))


@pytest.mark.parametrize("M,N", [(256, 256), (8, 64), (300, 130)])
def test_gemm_largest_k_extremes(M, N):
    """K = 131072, the largest the library takes: with every code at +-127 the
    int32 accumulators reach +-K 127^2 = +-2114060288, just below 2^31, and must
    come out exact (ring, decode and ragged tiles); random codes at the same K
    pass Freivalds' check."""
    K = 131072
    _say(f"gemm K={K} M={M} N={N}: kernel {sq.sq_gemm_kernel_name(M, N, K)}")
    xq = torch.full((M, K), 127, dtype=torch.int8, device=DEV)
    sign = torch.where(torch.arange(N, device=DEV) % 2 == 0, 1, -1).to(torch.int8)
    wq = (torch.full((N, K), 127, dtype=torch.int8, device=DEV) * sign[:, None]).contiguous()
    xs = torch.full((M,), 1.0 / 127, device=DEV)
    ws = torch.full((N,), 2.0 ** -20, device=DEV)
    y = torch.empty(M, N, dtype=torch.float32, device=DEV)
    acc = torch.empty(M, N, dtype=torch.int32, device=DEV)
    sq.sq_gemm_w8a8(xq, xs, sq.SQ_PER_TOKEN, wq, ws, y, acc)
    torch.cuda.synchronize()
    peak = K * 127 * 127
    assert peak < 2 ** 31
    want = np.where(np.arange(N) % 2 == 0, peak, -peak).astype(np.int64)
    np.testing.assert_array_equal(_np(acc).astype(np.int64), np.broadcast_to(want, (M, N)))
    y_o, _ = oracle.dequant(_np(acc), _np(xs), oracle.PER_TOKEN, _np(ws))
    np.testing.assert_array_equal(_np(y), y_o)
    # random codes: acc . r == Xq . (Wq^T r) in int64
    g = torch.Generator(device=DEV)
    g.manual_seed(M + N)
    xq = torch.randint(-127, 128, (M, K), dtype=torch.int8, device=DEV, generator=g)
    wq = torch.randint(-127, 128, (N, K), dtype=torch.int8, device=DEV, generator=g)
    sq.sq_gemm_w8a8(xq, xs, sq.SQ_PER_TOKEN, wq, ws, y, acc)
    torch.cuda.synchronize()
    A, B, C = _np(xq).astype(np.int64), _np(wq).astype(np.int64), _np(acc).astype(np.int64)
    rng = np.random.default_rng(N)
    for _ in range(2):
        r = rng.choice(np.array([-1, 1], dtype=np.int64), size=N)
        np.testing.assert_array_equal(C @ r, A @ (B.T @ r))


@pytest.mark.parametrize("M", [40, 8])
def test_gemm_weight_codes_beyond_4gib(M):
    """Wq of 65568 x 65536 codes (4.3 GB, past 32-bit byte offsets): the ring
    and the weight-streaming decode kernels are ruled out, and the kernels that
    run instead (the register-staged GEMM for M = 40, the general decode kernel
    for M = 8) must index it with 64-bit offsets; sampled outputs, including
    the last channels, against the oracle."""
    N, K = 65568, 65536
    assert N * K >= 2 ** 32
    _say(f"gemm beyond 4 GiB M={M} N={N} K={K}: kernel {sq.sq_gemm_kernel_name(M, N, K)}")
    g = torch.Generator(device=DEV)
    g.manual_seed(4 * M + 1)
    xq = torch.randint(-127, 128, (M, K), dtype=torch.int8, device=DEV, generator=g)
    wq = torch.randint(-127, 128, (N, K), dtype=torch.int8, device=DEV, generator=g)
    xs = torch.rand(M, device=DEV, generator=g) * 1e-3 + 1e-5
    ws = torch.rand(N, device=DEV, generator=g) * 1e-3 + 1e-5
    y = torch.empty(M, N, dtype=torch.bfloat16, device=DEV)
    acc = torch.empty(M, N, dtype=torch.int32, device=DEV)
    sq.sq_gemm_w8a8(xq, xs, sq.SQ_PER_TOKEN, wq, ws, y, acc)
    torch.cuda.synchronize()
    cols = torch.cat([torch.arange(0, 64, device=DEV), torch.arange(N // 2, N // 2 + 32, device=DEV),
                      torch.arange(N - 64, N, device=DEV)])
    acc_o = oracle.gemm_i8(_np(xq), _np(wq[cols]), nthreads=8)
    _, ybf_o = oracle.dequant(acc_o, _np(xs), oracle.PER_TOKEN, _np(ws[cols]))
    np.testing.assert_array_equal(_np(acc[:, cols]), acc_o)
    np.testing.assert_array_equal(_np(y[:, cols]), ybf_o)
    del xq, wq, y, acc
    torch.cuda.empty_cache()


def test_quantization_inputs_beyond_4gib():
    """Calibration tokens, activations and weights of 4.3 GB each (bf16,
    2^31 elements and more: past 32-bit element and byte offsets): the running
    maximum over all of them, per-token codes of sampled rows (first, middle,
    last) and weight codes of sampled output channels (each column's codes
    depend on that column only) against the oracle."""
    T, K = 131072, 16384
    Kw, N = 32768, 65568
    _say(f"quantization beyond 4 GiB: x {T}x{K}, w {Kw}x{N}")
    g = torch.Generator(device=DEV)
    g.manual_seed(31)
    x = (torch.randn(T, K, device=DEV, generator=g) * 2).to(torch.bfloat16)
    x[:, 77] *= 50
    amax = torch.zeros(K, dtype=torch.float32, device=DEV)
    sq.sq_calib_absmax(x, amax)
    inv_s = (torch.rand(K, device=DEV, generator=g) + 0.5).float()
    xq = torch.empty(T, K, dtype=torch.int8, device=DEV)
    xs = torch.empty(T, dtype=torch.float32, device=DEV)
    sq.sq_quant_act(x, inv_s, sq.SQ_PER_TOKEN, xq, xs)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(_np(amax), oracle.calib_absmax(_np(x)))
    rows = torch.cat([torch.arange(0, 16, device=DEV), torch.arange(T // 2, T // 2 + 16, device=DEV),
                      torch.arange(T - 16, T, device=DEV)])
    xq_o, xs_o = oracle.quant_act(_np(x[rows]), _np(inv_s), oracle.PER_TOKEN)
    np.testing.assert_array_equal(_np(xq[rows]), xq_o)
    np.testing.assert_array_equal(_np(xs[rows]), xs_o)
    del x, xq, xs
    torch.cuda.empty_cache()

    w = (torch.randn(Kw, N, device=DEV, generator=g) * 0.02).to(torch.bfloat16)
    s = (torch.rand(Kw, device=DEV, generator=g) + 0.5).float()
    wq = torch.empty(N, Kw, dtype=torch.int8, device=DEV)
    w_scale = torch.empty(N, dtype=torch.float32, device=DEV)
    nb = sq.sq_workspace_size(sq.SQ_OP_QUANT_WEIGHT, 0, N, Kw)
    sq.sq_quant_weight(w, s, wq, w_scale, torch.empty(nb, dtype=torch.uint8, device=DEV))
    torch.cuda.synchronize()
    cols = torch.cat([torch.arange(0, 32, device=DEV), torch.arange(N // 2, N // 2 + 32, device=DEV),
                      torch.arange(N - 32, N, device=DEV)])
    wq_o, ws_o = oracle.quant_weight(_np(w[:, cols]), _np(s))
    np.testing.assert_array_equal(_np(wq[cols]), wq_o)
    np.testing.assert_array_equal(_np(w_scale[cols]), ws_o)
    del w, wq
    torch.cuda.empty_cache()


def test_per_tensor_dynamic_large_x_streams():
    """Dynamic per-tensor codes of an x above 256 MB (16400 x 8192 bf16): the max
    pass takes its nontemporal-load branch (smaller x is read as plain loads).
    The maximum is checked through the oracle's calibrated-maximum function on
    all of x, the codes on sampled rows (static codes with that maximum equal
    the dynamic ones, a CPU pin)."""
    M, K = 16400, 8192
    _say(f"per-tensor dynamic M={M} K={K}")
    g = torch.Generator(device=DEV)
    g.manual_seed(11)
    idx = torch.randperm(K, generator=g, device=DEV)[: K // 100]
    fac = torch.full((idx.numel(),), 100.0, device=DEV)
    x = synth.activations(M, K, "normal", idx, fac, torch.bfloat16, g, DEV)
    inv_s = (torch.rand(K, generator=g, device=DEV) + 0.5).float()
    xq = torch.empty(M, K, dtype=torch.int8, device=DEV)
    xs = torch.empty(1, dtype=torch.float32, device=DEV)
    nb = sq.sq_workspace_size(sq.SQ_OP_QUANT_ACT, M, 1, K, sq.SQ_PER_TENSOR)
    ws = torch.empty(max(nb, 16), dtype=torch.uint8, device=DEV)
    sq.sq_quant_act(x, inv_s, sq.SQ_PER_TENSOR, xq, xs, ws)
    torch.cuda.synchronize()
    xn, isn = _np(x), _np(inv_s)
    a = oracle.static_act_max(xn, isn)
    rows = [0, 1, 4097, M // 2, M - 2, M - 1]
    oq, os_ = oracle.quant_act_static(xn[rows], isn, a)
    np.testing.assert_array_equal(_np(xs), os_)
    np.testing.assert_array_equal(_np(xq[rows]), oq)
