"""Host-side checks of the C ABI: the library loads, exports every symbol the
header declares, sizes workspaces, and rejects bad arguments before it
enqueues anything.  No call here reaches a kernel launch: each one carries an
argument that validation refuses (fake pointers are never dereferenced)."""
import ctypes
import os
import re

import pytest

import post_quantization_act_amd as sq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_symbols():
    text = open(os.path.join(ROOT, "include", "sq.h")).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_]+\s*\*?\s*(sq_[a-z0-9_]+)\s*\(", text, re.M)))


def test_library_exports_every_declared_symbol():
    L = sq.lib()
    declared = _declared_symbols()
    assert set(declared) >= {"sq_calib_absmax", "sq_smooth_factors", "sq_quant_weight", "sq_quant_act",
                             "sq_gemm_w8a8", "sq_workspace_size", "sq_status_str", "sq_last_error"}
    for name in declared:
        assert hasattr(L, name), name
    assert set(declared) == set(sq.EXPORTED_SYMBOLS)


def test_library_is_gfx950_code():
    out = open(sq.lib_path(), "rb").read()
    assert b"gfx950" in out
    assert b"gfx942" not in out and b"sm_" not in out[:0]


def test_status_strings_and_version():
    assert sq.sq_status_str(0) == "SQ_OK"
    assert sq.sq_status_str(-1) == "SQ_ERR_INVALID_ARG"
    assert sq.sq_status_str(-3) == "SQ_ERR_WORKSPACE"
    assert re.match(r"^\d+\.\d+\.\d+$", sq.sq_version())


def test_gemm_kernel_choice():
    """The shape rule of the GEMM dispatch (for a 256-CU device; without a GPU
    the library assumes 256): decode kernels for M <= 16, the LDS ring kernel
    for K % 128 == 0 (the tile shape whose rounds over the CUs, weighted by
    relative stage time 1.6 / 1.0 / 1.2 for 256 x 256 / 256 x 128 / two
    128 x 128 blocks, cost least), the register-staged kernel otherwise."""
    assert sq.sq_gemm_kernel_name(16, 28672, 8192).startswith("k_gemm_decode_ring")
    assert sq.sq_gemm_kernel_name(16, 100, 1040).startswith("k_gemm_decode (")
    assert sq.sq_gemm_kernel_name(2048, 4096, 4096).startswith("k_gemm_ring<256,128")
    assert sq.sq_gemm_kernel_name(33000, 100, 384).startswith("k_gemm_ring<128,128")
    assert sq.sq_gemm_kernel_name(4096, 14336, 4096).startswith("k_gemm_persist<256,256")
    assert sq.sq_gemm_kernel_name(4096, 4096, 4096).startswith("k_gemm_persist<256,256")  # one full round
    assert sq.sq_gemm_kernel_name(4096, 4096, 384).startswith("k_gemm_ring<256,256")  # K % 256 != 0
    assert sq.sq_gemm_kernel_name(2400, 8000, 4096).startswith("k_gemm_ring<256,128")   # 320 tiles: 2 rounds
    assert sq.sq_gemm_kernel_name(3072, 4096, 4096).startswith("k_gemm_persist<256,256")   # 192 tiles, 1 round
    assert sq.sq_gemm_kernel_name(8192, 49152, 12288).startswith("k_gemm_persist<256,256")
    assert sq.sq_gemm_kernel_name(300, 520, 1040).startswith("k_gemm_generic")
    # 896 tiles of 256 x 256 (3.5 rounds): 3 rounds of them, then the last 2048 columns as 256 x 128 tiles
    assert "whole rounds" in sq.sq_gemm_kernel_name(4096, 14336, 4096)
    assert "whole rounds" in sq.sq_gemm_kernel_name(256, 66536, 128)
    assert "whole rounds" not in sq.sq_gemm_kernel_name(8192, 49152, 12288)  # 24 whole rounds
    assert sq.sq_gemm_kernel_name(0, 5, 16).startswith("none")


def test_workspace_sizes():
    assert sq.sq_workspace_size(sq.SQ_OP_QUANT_WEIGHT, 0, 4096, 4096) >= 4096 * 4
    assert sq.sq_workspace_size(sq.SQ_OP_QUANT_WEIGHT, 0, 0, 4096) == 0
    assert sq.sq_workspace_size(sq.SQ_OP_QUANT_ACT, 2048, 0, 4096, sq.SQ_PER_TOKEN) == 0
    assert sq.sq_workspace_size(sq.SQ_OP_QUANT_ACT, 2048, 0, 4096, sq.SQ_PER_TENSOR) >= 4
    assert sq.sq_workspace_size(sq.SQ_OP_CALIB_ABSMAX, 1, 1, 16) == 0
    # prepare_weights: column maxima + one partial row of N maxima per block (<= 256 blocks)
    assert sq.sq_workspace_size(sq.SQ_OP_PREPARE_WEIGHTS, 0, 4096, 4096) >= 4096 * 4 + 256 * 4096 * 4
    assert sq.sq_workspace_size(sq.SQ_OP_PREPARE_WEIGHTS, 0, 4096, 100) >= 4096 * 4 + 100 * 4096 * 4
    assert sq.sq_workspace_size(sq.SQ_OP_PREPARE_WEIGHTS, 0, 4096, 300) < 4096 * 4 + 256 * 4096 * 4  # 150 blocks
    assert sq.sq_workspace_size(sq.SQ_OP_PREPARE_WEIGHTS, 0, 0, 4096) == 0
    # plus the power tables of a general alpha: 32768 + 1 + K doubles
    assert sq.sq_workspace_size(sq.SQ_OP_PREPARE_WEIGHTS, 0, 4096, 4096) >= (
        4096 * 4 + 256 * 4096 * 4 + (32769 + 4096) * 8)
    # prepare_and_quant_act: prepare_weights' workspace, then (256-byte aligned) quant_act's
    for g in (sq.SQ_PER_TOKEN, sq.SQ_PER_TENSOR):
        p = sq.sq_workspace_size(sq.SQ_OP_PREPARE_WEIGHTS, 2048, 4096, 4096, g)
        a = sq.sq_workspace_size(sq.SQ_OP_QUANT_ACT, 2048, 4096, 4096, g)
        assert sq.sq_workspace_size(sq.SQ_OP_PREPARE_AND_QUANT_ACT, 2048, 4096, 4096, g) == (p + 255) // 256 * 256 + a


FAKE = ctypes.c_void_p(0x10000)       # 16-byte aligned, never dereferenced
MISALIGNED = ctypes.c_void_p(0x10004)


def _L():
    return sq.lib()


def _expect(rc, status, pattern):
    assert rc == status, (rc, sq.sq_last_error())
    assert re.search(pattern, sq.sq_last_error()), sq.sq_last_error()


def test_calib_reset_rejects():
    L = _L()
    _expect(L.sq_calib_reset(FAKE, -1, None), -1, "negative")
    _expect(L.sq_calib_reset(None, 16, None), -1, "amax is NULL")
    _expect(L.sq_calib_reset(ctypes.c_void_p(0x10002), 16, None), -1, "4-byte aligned")
    assert L.sq_calib_reset(None, 0, None) == 0  # nothing to clear, nothing enqueued


def test_calib_rejects_bad_k_and_null():
    L = _L()
    _expect(L.sq_calib_absmax(FAKE, sq.SQ_BF16, 8, 20, 20, FAKE, None), -1, "multiple of 16")
    _expect(L.sq_calib_absmax(None, sq.SQ_BF16, 8, 32, 32, FAKE, None), -1, "x is NULL")
    _expect(L.sq_calib_absmax(FAKE, sq.SQ_BF16, 8, 32, 16, FAKE, None), -1, "row stride")
    _expect(L.sq_calib_absmax(MISALIGNED, sq.SQ_BF16, 8, 32, 32, FAKE, None), -1, "aligned")
    _expect(L.sq_calib_absmax(FAKE, sq.SQ_BF16, 8, 32, 36, FAKE, None), -1, "multiple of 16 bytes")
    _expect(L.sq_calib_absmax(FAKE, 7, 8, 32, 32, FAKE, None), -2, "dtype")
    _expect(L.sq_calib_absmax(FAKE, sq.SQ_BF16, 8, 32, 32, None, None), -1, "amax is NULL")
    _expect(L.sq_calib_absmax(FAKE, sq.SQ_BF16, -1, 32, 32, FAKE, None), -1, "negative")


def test_empty_calls_succeed_without_work():
    L = _L()
    assert L.sq_calib_absmax(None, sq.SQ_BF16, 0, 32, 32, FAKE, None) == 0
    assert L.sq_gemm_w8a8(None, None, 0, None, None, 0, 16, 32, None, sq.SQ_BF16, None, None, 0, None) == 0
    assert sq.sq_last_error() == ""


def test_smooth_factors_rejects():
    L = _L()
    f = ctypes.c_float
    _expect(L.sq_smooth_factors(FAKE, FAKE, sq.SQ_BF16, 32, 16, 16, f(1.5), FAKE, FAKE, None, None), -1, "alpha")
    _expect(L.sq_smooth_factors(FAKE, FAKE, sq.SQ_BF16, 32, 16, 16, f(float("nan")), FAKE, FAKE, None, None), -1,
            "alpha")
    _expect(L.sq_smooth_factors(FAKE, None, sq.SQ_BF16, 32, 16, 16, f(0.5), FAKE, FAKE, None, None), -1,
            "precomputed amax_w")
    _expect(L.sq_smooth_factors(FAKE, FAKE, sq.SQ_BF16, 32, 0, 16, f(0.5), FAKE, FAKE, None, None), -1,
            "N = 0")
    _expect(L.sq_smooth_factors(FAKE, FAKE, sq.SQ_BF16, 32, 16, 16, f(0.5), None, FAKE, None, None), -1,
            "s is NULL")


def test_quant_weight_rejects():
    L = _L()
    _expect(L.sq_quant_weight(FAKE, sq.SQ_BF16, 32, 64, 64, FAKE, FAKE, FAKE, None, 0, None), -3, "workspace")
    _expect(L.sq_quant_weight(FAKE, sq.SQ_BF16, 32, 64, 64, FAKE, FAKE, FAKE, FAKE, 16, None), -3, "workspace")
    _expect(L.sq_quant_weight(FAKE, sq.SQ_BF16, 32, 64, 64, FAKE, MISALIGNED, FAKE, FAKE, 4096, None), -1, "wq")
    _expect(L.sq_quant_weight(FAKE, sq.SQ_BF16, 33, 64, 64, FAKE, FAKE, FAKE, FAKE, 4096, None), -1, "K = 33")


def test_quant_weight_noalloc_rejects():
    """Beyond the 65536 columns of the static scratch, and the usual argument
    checks, all before the scratch's device address is looked up."""
    L = _L()
    _expect(L.sq_quant_weight_noalloc(FAKE, sq.SQ_BF16, 32, 65537, 65537, FAKE, FAKE, FAKE, None), -3,
            "static scratch")
    _expect(L.sq_quant_weight_noalloc(FAKE, sq.SQ_BF16, 32, 64, 64, FAKE, MISALIGNED, FAKE, None), -1, "wq")
    _expect(L.sq_quant_weight_noalloc(FAKE, sq.SQ_BF16, 33, 64, 64, FAKE, FAKE, FAKE, None), -1, "K = 33")
    _expect(L.sq_quant_weight_noalloc(None, sq.SQ_BF16, 32, 64, 64, FAKE, FAKE, FAKE, None), -1, "w is NULL")


def test_quant_act_rejects():
    L = _L()
    _expect(L.sq_quant_act(FAKE, sq.SQ_BF16, 4, 32, 32, FAKE, 5, FAKE, FAKE, None, 0, None), -2, "granularity")
    _expect(L.sq_quant_act(FAKE, sq.SQ_BF16, 4, 32, 32, FAKE, sq.SQ_PER_TENSOR, FAKE, FAKE, None, 0, None), -3,
            "workspace")
    _expect(L.sq_quant_act(FAKE, sq.SQ_BF16, 4, 32, 32, MISALIGNED, sq.SQ_PER_TOKEN, FAKE, FAKE, None, 0, None),
            -1, "inv_s")
    _expect(L.sq_quant_act(FAKE, sq.SQ_BF16, 4, 32, 32, FAKE, sq.SQ_PER_TOKEN, None, FAKE, None, 0, None), -1,
            "xq is NULL")


def test_gemm_rejects():
    L = _L()
    _expect(L.sq_gemm_w8a8(FAKE, FAKE, 0, FAKE, FAKE, 4, 4, 24, FAKE, sq.SQ_BF16, None, None, 0, None), -1,
            "multiple of 16")
    _expect(L.sq_gemm_w8a8(FAKE, FAKE, 0, FAKE, FAKE, 4, 4, 16 * 8193 + 16 * 8192, FAKE, sq.SQ_BF16, None, None, 0,
                           None), -1, "multiple of 16|131072")
    _expect(L.sq_gemm_w8a8(MISALIGNED, FAKE, 0, FAKE, FAKE, 4, 4, 32, FAKE, sq.SQ_BF16, None, None, 0, None), -1,
            "aligned")
    _expect(L.sq_gemm_w8a8(FAKE, FAKE, 0, FAKE, FAKE, 4, 4, 32, None, sq.SQ_BF16, None, None, 0, None), -1,
            "y is NULL")
    _expect(L.sq_gemm_w8a8(FAKE, FAKE, 0, FAKE, FAKE, 4, 4, 32, FAKE, 9, None, None, 0, None), -2, "output dtype")
    _expect(L.sq_gemm_w8a8(FAKE, FAKE, 3, FAKE, FAKE, 4, 4, 32, FAKE, sq.SQ_BF16, None, None, 0, None), -2,
            "granularity")


def test_binding_rejects_host_tensors():
    import torch
    x = torch.zeros(4, 32, dtype=torch.bfloat16)
    amax = torch.zeros(32)
    with pytest.raises(ValueError, match="device tensors"):
        sq.sq_calib_absmax(x, amax)


def test_prepare_weights_rejects():
    L = _L()
    f = ctypes.c_float
    args = lambda **kw: [kw.get("amax_x", FAKE), kw.get("w", FAKE), sq.SQ_BF16, kw.get("K", 32), kw.get("N", 64),
                         kw.get("ld", 64), f(kw.get("alpha", 0.5)), kw.get("s", FAKE), FAKE, None,
                         kw.get("wq", FAKE), FAKE, kw.get("ws", FAKE), kw.get("wsb", 1 << 20), None]
    _expect(L.sq_prepare_weights(*args(alpha=1.5)), -1, "alpha")
    _expect(L.sq_prepare_weights(*args(N=0)), -1, "N = 0")
    _expect(L.sq_prepare_weights(*args(s=None)), -1, "s is NULL")
    _expect(L.sq_prepare_weights(*args(wq=MISALIGNED)), -1, "wq")
    _expect(L.sq_prepare_weights(*args(K=33)), -1, "K = 33")
    _expect(L.sq_prepare_weights(*args(ws=None, wsb=0)), -3, "workspace")
    _expect(L.sq_prepare_weights(*args(wsb=64)), -3, "workspace")


def test_prepare_and_quant_act_rejects():
    """Every rejection comes before anything is enqueued (no GPU here)."""
    L = _L()
    f = ctypes.c_float

    def args(**kw):
        return [kw.get("amax_x", FAKE), kw.get("w", FAKE), kw.get("wt", sq.SQ_BF16), kw.get("K", 32), kw.get("N", 64),
                kw.get("ldw", 64), f(kw.get("alpha", 0.5)), kw.get("s", FAKE), kw.get("inv_s", FAKE), None,
                kw.get("wq", FAKE), FAKE, kw.get("x", FAKE), kw.get("xt", sq.SQ_BF16), kw.get("M", 8),
                kw.get("ldx", 32), kw.get("g", sq.SQ_PER_TOKEN), kw.get("xq", FAKE), FAKE, kw.get("ws", FAKE),
                kw.get("wsb", 1 << 20), None]

    fn = L.sq_prepare_and_quant_act
    _expect(fn(*args(alpha=1.5)), -1, "alpha")
    _expect(fn(*args(K=33)), -1, "K = 33")
    _expect(fn(*args(s=None)), -1, "s is NULL")
    _expect(fn(*args(w=None)), -1, "w is NULL")
    _expect(fn(*args(wq=MISALIGNED)), -1, "wq")
    _expect(fn(*args(inv_s=MISALIGNED)), -1, "inv_s is not 16-byte aligned")
    _expect(fn(*args(xq=MISALIGNED)), -1, "xq")
    _expect(fn(*args(x=None)), -1, "x is NULL")
    _expect(fn(*args(ldx=36)), -1, "row stride")
    _expect(fn(*args(g=7)), -2, "granularity")
    _expect(fn(*args(ws=None, wsb=0)), -3, "workspace")
    # per tensor also needs quant_act's 256 bytes after prepare_weights' workspace
    p = sq.sq_workspace_size(sq.SQ_OP_PREPARE_WEIGHTS, 8, 64, 32, sq.SQ_PER_TENSOR)
    _expect(fn(*args(g=sq.SQ_PER_TENSOR, wsb=(p + 255) // 256 * 256)), -3, "workspace")
    # the slow path (fp32 W) rejects with prepare_weights' own checks, also before any launch
    _expect(fn(*args(wt=sq.SQ_F32, alpha=-0.5)), -1, "alpha")


def test_static_scale_rejects():
    L = _L()
    _expect(L.sq_static_act_max(FAKE, None, 32, None, None), -1, "a_static is NULL")
    _expect(L.sq_static_act_max(FAKE, None, 20, FAKE, None), -1, "multiple of 16")
    _expect(L.sq_quant_act_static(FAKE, sq.SQ_BF16, 4, 32, 32, None, None, FAKE, FAKE, None), -1, "a_static is NULL")
    _expect(L.sq_quant_act_static(FAKE, sq.SQ_BF16, 4, 32, 32, None, FAKE, MISALIGNED, FAKE, None), -1, "xq")


def test_layernorm_rejects():
    L = _L()
    f = ctypes.c_float
    _expect(L.sq_layernorm_quant(FAKE, sq.SQ_F32, 4, 32, 32, FAKE, None, f(1e-5), FAKE, FAKE, None), -2, "bf16")
    _expect(L.sq_layernorm_quant(FAKE, sq.SQ_BF16, 4, 16400, 16400, FAKE, None, f(1e-5), FAKE, FAKE, None), -2,
            "16384")
    _expect(L.sq_layernorm_quant(FAKE, sq.SQ_BF16, 4, 32, 32, None, None, f(1e-5), FAKE, FAKE, None), -1,
            "gamma is NULL")
    _expect(L.sq_layernorm_quant(FAKE, sq.SQ_BF16, 4, 32, 32, FAKE, None, f(-1.0), FAKE, FAKE, None), -1, "eps")
    _expect(L.sq_fold_layernorm(None, None, FAKE, 8, FAKE, None, None), -1, "gamma is NULL")
    _expect(L.sq_fold_layernorm(FAKE, FAKE, FAKE, 8, FAKE, None, None), -1, "beta_out is NULL")


def test_llm_int8_entry_points_reject():
    L = _L()
    f = ctypes.c_float
    # outlier selection
    _expect(L.sq_outlier_columns(FAKE, 20, f(6.0), FAKE, FAKE, FAKE, None), -1, "multiple of 16")
    _expect(L.sq_outlier_columns(FAKE, 32, f(float("nan")), FAKE, FAKE, FAKE, None), -1, "NaN")
    _expect(L.sq_outlier_columns(FAKE, 32, f(6.0), FAKE, None, FAKE, None), -1, "count is NULL")
    _expect(L.sq_outlier_columns(FAKE, 32, f(6.0), FAKE, FAKE, MISALIGNED, None), -1, "keep")
    # gather
    g = lambda **kw: [FAKE, kw.get("xt", sq.SQ_BF16), 8, kw.get("K", 32), kw.get("K", 32), FAKE,
                      kw.get("wt", sq.SQ_BF16), 24,
                      24, FAKE, kw.get("count", FAKE), kw.get("kp", 32), kw.get("x_o", FAKE), FAKE, None]
    _expect(L.sq_gather_outliers(*g(xt=sq.SQ_F32)), -2, "bf16")
    _expect(L.sq_gather_outliers(*g(kp=24)), -1, "kp = 24")
    _expect(L.sq_gather_outliers(*g(K=48, kp=32)), -1, "kp = 32")
    _expect(L.sq_gather_outliers(*g(count=None)), -1, "count is NULL")
    _expect(L.sq_gather_outliers(*g(x_o=MISALIGNED)), -1, "x_o")
    # outlier GEMM
    m = lambda **kw: [FAKE, FAKE, kw.get("wq", FAKE), FAKE, 4, 8, kw.get("K", 32), FAKE, FAKE, kw.get("kp", 32),
                      kw.get("count", FAKE), kw.get("y", FAKE), kw.get("yt", sq.SQ_BF16), None]
    _expect(L.sq_gemm_w8a8_outlier(*m(K=24)), -1, "multiple of 16")
    _expect(L.sq_gemm_w8a8_outlier(*m(kp=16)), -1, "kp = 16")
    _expect(L.sq_gemm_w8a8_outlier(*m(count=None)), -1, "count is NULL")
    _expect(L.sq_gemm_w8a8_outlier(*m(wq=MISALIGNED)), -1, "16-byte aligned")
    _expect(L.sq_gemm_w8a8_outlier(*m(y=None)), -1, "y is NULL")
    _expect(L.sq_gemm_w8a8_outlier(*m(yt=9)), -2, "output dtype")


def test_alpha_criterion_entry_points_reject():
    L = _L()
    mm = lambda **kw: [kw.get("x", FAKE), kw.get("xt", sq.SQ_BF16), 8, kw.get("K", 32), kw.get("ldx", 32), FAKE,
                       sq.SQ_F32, kw.get("N", 24), kw.get("ldw", 24), kw.get("y", FAKE), None]
    _expect(L.sq_matmul_f64(*mm(K=24, ldx=24)), -1, "multiple of 16")
    _expect(L.sq_matmul_f64(*mm(xt=5)), -2, "dtype")
    _expect(L.sq_matmul_f64(*mm(x=None)), -1, "x is NULL")
    _expect(L.sq_matmul_f64(*mm(ldx=16)), -1, "row stride")
    _expect(L.sq_matmul_f64(*mm(ldw=20)), -1, "row stride")
    _expect(L.sq_matmul_f64(*mm(y=None)), -1, "y_ref is NULL")
    _expect(L.sq_matmul_f64(*mm(y=MISALIGNED)), -1, "8-byte aligned")
    _expect(L.sq_matmul_f64(*mm(N=65535 * 128 + 1, ldw=65535 * 128 + 1)), -1, "out of range")
    assert L.sq_matmul_f64(*mm(N=0, y=None)) == 0  # empty product: nothing enqueued
    need = sq.sq_workspace_size(sq.SQ_OP_REL_ERROR, 8, 24, 0)
    assert need == 8192
    re_ = lambda **kw: [FAKE, kw.get("yr", FAKE), 8, 24, kw.get("err", FAKE), kw.get("ws", FAKE),
                        kw.get("nb", need), None]
    _expect(L.sq_rel_error(*re_(nb=need - 8)), -3, "workspace")
    _expect(L.sq_rel_error(*re_(ws=None)), -3, "workspace")
    _expect(L.sq_rel_error(*re_(err=None)), -1, "err is NULL")
    _expect(L.sq_rel_error(*re_(err=MISALIGNED)), -1, "err is NULL or not 8-byte aligned")
    _expect(L.sq_rel_error(*re_(yr=None)), -1, "y_ref is NULL")
    _expect(L.sq_rel_error(*re_(yr=MISALIGNED)), -1, "y_ref is not 8-byte aligned")
    _expect(L.sq_rel_error(None, FAKE, 8, 24, FAKE, FAKE, need, None), -1, "y is NULL")
    _expect(L.sq_rel_error(FAKE, FAKE, -1, 24, FAKE, FAKE, need, None), -1, "out of range")


def test_outlier_gemm_kernel_choice():
    """The outlier variant uses the same tile kernels, and the general one
    where the plain product would stream weights (M <= 16)."""
    assert sq.sq_gemm_outlier_kernel_name(2048, 4096, 4096) == sq.sq_gemm_kernel_name(2048, 4096, 4096)
    assert sq.sq_gemm_outlier_kernel_name(16, 28672, 8192).startswith("k_gemm_ring")
    assert sq.sq_gemm_outlier_kernel_name(16, 100, 1040).startswith("k_gemm_generic")


def test_last_error_is_per_thread():
    """Each host thread reads the message of its own last failure: threads
    that provoke different rejections at the same time never see each other's
    text (the library's only per-call state is thread-local)."""
    import threading
    L = _L()
    results = {}
    barrier = threading.Barrier(4)

    def worker(i):
        barrier.wait()
        for _ in range(200):
            if i % 2 == 0:
                rc = L.sq_calib_absmax(FAKE, sq.SQ_BF16, 8, 20 + 16 * i, 20 + 16 * i, FAKE, None)
                want = f"K = {20 + 16 * i} must be a multiple of 16"
            else:
                rc = L.sq_calib_reset(None, 16 * i, None)
                want = "amax is NULL"
            msg = sq.sq_last_error()
            if rc != -1 or want not in msg:
                results[i] = msg
                return
        results[i] = "ok"

    ts = [threading.Thread(target=worker, args=(i,)) for i in range(4)]
    for t in ts:
        t.start()
    for t in ts:
        t.join()
    assert results == {i: "ok" for i in range(4)}, results
