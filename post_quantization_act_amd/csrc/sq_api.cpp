// C ABI of the SmoothQuant W8A8 library: argument validation, workspace
// sizing and kernel dispatch.  Nothing here allocates device memory.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <string>

#include "sq.h"
#include "sq_internal.h"

namespace {

thread_local std::string g_last_error;

sq_status fail(sq_status st, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return st;
}

sq_status ok() {
    g_last_error.clear();
    return SQ_OK;
}

sq_status hip_result(hipError_t e, const char* what) {
    if (e != hipSuccess) return fail(SQ_ERR_HIP, "%s: HIP launch failed: %s", what, hipGetErrorString(e));
    return ok();
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t elem_size(sq_dtype t) { return t == SQ_BF16 ? 2 : 4; }

bool dtype_ok(sq_dtype t) { return t == SQ_BF16 || t == SQ_F32; }

constexpr int64_t kMaxK = 131072;          // keeps |acc| <= K * 127^2 < 2^31
constexpr int64_t kMaxMN = (int64_t)1 << 30;

size_t round256(size_t b) { return (b + 255) / 256 * 256; }

// Shared checks of a [rows, cols] input with row stride ld.  Activations
// (need16) must have 16-byte aligned rows; weights only element alignment
// (rows that are not 16-byte aligned take a slower element-wise load path).
sq_status check_matrix(const char* fn, const char* name, const void* p, sq_dtype t, int64_t rows, int64_t cols,
                       int64_t ld, bool need16 = true) {
    if (!dtype_ok(t)) return fail(SQ_ERR_UNSUPPORTED, "%s: %s dtype %d is not SQ_BF16 or SQ_F32", fn, name, (int)t);
    if (rows < 0 || cols < 0) return fail(SQ_ERR_INVALID_ARG, "%s: %s has negative size", fn, name);
    if (ld < cols) return fail(SQ_ERR_INVALID_ARG, "%s: %s row stride %lld < row length %lld", fn, name,
                               (long long)ld, (long long)cols);
    if (rows > 0 && cols > 0) {
        if (!p) return fail(SQ_ERR_INVALID_ARG, "%s: %s is NULL", fn, name);
        if (!need16) {
            if (reinterpret_cast<uintptr_t>(p) % elem_size(t) != 0)
                return fail(SQ_ERR_INVALID_ARG, "%s: %s is not aligned to its element size", fn, name);
            return SQ_OK;
        }
        if (!aligned16(p)) return fail(SQ_ERR_INVALID_ARG, "%s: %s is not 16-byte aligned", fn, name);
        if ((ld * (int64_t)elem_size(t)) % 16 != 0)
            return fail(SQ_ERR_INVALID_ARG, "%s: %s row stride %lld elements is not a multiple of 16 bytes", fn,
                        name, (long long)ld);
    }
    return SQ_OK;
}

sq_status check_k(const char* fn, int64_t K) {
    if (K < 0 || K % 16 != 0 || K > kMaxK)
        return fail(SQ_ERR_INVALID_ARG, "%s: K = %lld must be a multiple of 16 in [0, %lld]", fn, (long long)K,
                    (long long)kMaxK);
    return SQ_OK;
}

sq_status check_vec(const char* fn, const char* name, const void* p, int64_t n, bool need16 = false) {
    if (n > 0 && !p) return fail(SQ_ERR_INVALID_ARG, "%s: %s is NULL", fn, name);
    if (n > 0 && need16 && !aligned16(p)) return fail(SQ_ERR_INVALID_ARG, "%s: %s is not 16-byte aligned", fn, name);
    if (n > 0 && (reinterpret_cast<uintptr_t>(p) & 3u))
        return fail(SQ_ERR_INVALID_ARG, "%s: %s is not 4-byte aligned", fn, name);
    return SQ_OK;
}

#define SQ_TRY(expr)                   \
    do {                               \
        sq_status _st = (expr);        \
        if (_st != SQ_OK) return _st;  \
    } while (0)

}  // namespace

extern "C" {

const char* sq_version(void) { return "0.1.0"; }

const char* sq_gemm_kernel_name(int64_t M, int64_t N, int64_t K) { return sqk::gemm_kernel_name(M, N, K); }

const char* sq_last_error(void) { return g_last_error.c_str(); }

const char* sq_status_str(sq_status s) {
    switch (s) {
        case SQ_OK: return "SQ_OK";
        case SQ_ERR_INVALID_ARG: return "SQ_ERR_INVALID_ARG";
        case SQ_ERR_UNSUPPORTED: return "SQ_ERR_UNSUPPORTED";
        case SQ_ERR_WORKSPACE: return "SQ_ERR_WORKSPACE";
        case SQ_ERR_HIP: return "SQ_ERR_HIP";
    }
    return "SQ_UNKNOWN_STATUS";
}

// The power tables of the one-read weight pass: after the column maxima and
// the per-block partial maxima in the SQ_OP_PREPARE_WEIGHTS workspace.
static double* prep_tables(void* ws, int64_t N, int64_t K) {
    return reinterpret_cast<double*>(static_cast<char*>(ws) + round256((size_t)N * sizeof(uint32_t)) +
                                     round256((size_t)sqk::prep_blocks(K) * (size_t)N * sizeof(float)));
}

size_t sq_workspace_size(sq_op op, int64_t M, int64_t N, int64_t K, sq_act_gran g) {
    (void)M;
    (void)K;
    switch (op) {
        case SQ_OP_QUANT_WEIGHT: return N > 0 ? round256((size_t)N * sizeof(uint32_t)) : 0;
        case SQ_OP_PREPARE_WEIGHTS:
            return N > 0 && K > 0 ? round256((size_t)N * sizeof(uint32_t)) +
                                        round256((size_t)sqk::prep_blocks(K) * (size_t)N * sizeof(float)) +
                                        round256((size_t)sqk::prep_table_entries(K) * sizeof(double))
                                  : 0;
        case SQ_OP_QUANT_ACT: return g == SQ_PER_TENSOR ? 256 : 0;
        case SQ_OP_PREPARE_AND_QUANT_ACT:
            return round256(sq_workspace_size(SQ_OP_PREPARE_WEIGHTS, M, N, K, g)) +
                   sq_workspace_size(SQ_OP_QUANT_ACT, M, N, K, g);
        case SQ_OP_REL_ERROR: return (size_t)sqk::rel_error_workspace_bytes();
        default: return 0;
    }
}

sq_status sq_calib_absmax(const void* x, sq_dtype xt, int64_t T, int64_t K, int64_t ldx, float* amax,
                          hipStream_t stream) {
    const char* fn = "sq_calib_absmax";
    SQ_TRY(check_k(fn, K));
    SQ_TRY(check_matrix(fn, "x", x, xt, T, K, ldx));
    SQ_TRY(check_vec(fn, "amax", amax, K));
    if (T == 0 || K == 0) return ok();
    return hip_result(sqk::launch_col_absmax(x, xt == SQ_BF16, T, K, ldx, nullptr,
                                             reinterpret_cast<uint32_t*>(amax), stream), fn);
}

sq_status sq_calib_reset(float* amax, int64_t K, hipStream_t stream) {
    const char* fn = "sq_calib_reset";
    if (K < 0) return fail(SQ_ERR_INVALID_ARG, "%s: K = %lld is negative", fn, (long long)K);
    if (K > kMaxMN) return fail(SQ_ERR_INVALID_ARG, "%s: K = %lld too large", fn, (long long)K);
    SQ_TRY(check_vec(fn, "amax", amax, K));
    if (K == 0) return ok();
    return hip_result(sqk::launch_fill_u32(reinterpret_cast<uint32_t*>(amax), K, 0u, stream), fn);
}

sq_status sq_smooth_factors(const float* amax_x, const void* w, sq_dtype wt, int64_t K, int64_t N, int64_t ldw,
                            float alpha, float* s, float* inv_s, float* amax_w, hipStream_t stream) {
    const char* fn = "sq_smooth_factors";
    SQ_TRY(check_k(fn, K));
    if (!(alpha >= 0.0f && alpha <= 1.0f)) return fail(SQ_ERR_INVALID_ARG, "%s: alpha = %g is not in [0, 1]", fn, alpha);
    SQ_TRY(check_vec(fn, "amax_x", amax_x, K));
    SQ_TRY(check_vec(fn, "s", s, K));
    SQ_TRY(check_vec(fn, "inv_s", inv_s, K));
    if (w) {
        if (N <= 0) return fail(SQ_ERR_INVALID_ARG, "%s: N = %lld must be positive when w is given", fn, (long long)N);
        SQ_TRY(check_matrix(fn, "w", w, wt, K, N, ldw, false));
        if (amax_w) SQ_TRY(check_vec(fn, "amax_w", amax_w, K));
    } else {
        if (!amax_w && K > 0) return fail(SQ_ERR_INVALID_ARG, "%s: need w or a precomputed amax_w", fn);
        SQ_TRY(check_vec(fn, "amax_w", amax_w, K));
    }
    if (K == 0) return ok();
    if (w)
        return hip_result(sqk::launch_row_absmax_factors(w, wt == SQ_BF16, K, N, ldw, amax_x, alpha, s, inv_s,
                                                         amax_w, stream), fn);
    return hip_result(sqk::launch_factors(amax_x, amax_w, K, alpha, s, inv_s, stream), fn);
}

sq_status sq_quant_weight(const void* w, sq_dtype wt, int64_t K, int64_t N, int64_t ldw, const float* s, int8_t* wq,
                          float* w_scale, void* ws, size_t ws_bytes, hipStream_t stream) {
    const char* fn = "sq_quant_weight";
    SQ_TRY(check_k(fn, K));
    if (N > kMaxMN) return fail(SQ_ERR_INVALID_ARG, "%s: N = %lld too large", fn, (long long)N);
    SQ_TRY(check_matrix(fn, "w", w, wt, K, N, ldw, false));
    if (s) SQ_TRY(check_vec(fn, "s", s, K));
    SQ_TRY(check_vec(fn, "w_scale", w_scale, N, true));
    if (K > 0 && N > 0) {
        if (!wq) return fail(SQ_ERR_INVALID_ARG, "%s: wq is NULL", fn);
        if (!aligned16(wq)) return fail(SQ_ERR_INVALID_ARG, "%s: wq is not 16-byte aligned", fn);
    }
    const size_t need = sq_workspace_size(SQ_OP_QUANT_WEIGHT, 0, N, K, SQ_PER_TOKEN);
    if (need > 0 && (!ws || ws_bytes < need || !aligned16(ws)))
        return fail(SQ_ERR_WORKSPACE, "%s: workspace of %zu bytes (16-byte aligned) required, got %zu", fn, need,
                    ws ? ws_bytes : (size_t)0);
    if (N == 0) return ok();
    uint32_t* colmax = static_cast<uint32_t*>(ws);
    if (K == 0)  // no input channels: every column max is 0, so every scale is 0
        return hip_result(sqk::launch_fill_u32(reinterpret_cast<uint32_t*>(w_scale), N, 0u, stream), fn);
    hipError_t e = sqk::launch_fill_u32(colmax, N, 0u, stream);
    if (e == hipSuccess) e = sqk::launch_col_absmax(w, wt == SQ_BF16, K, N, ldw, s, colmax, stream);
    if (e == hipSuccess) e = sqk::launch_quant_weight(w, wt == SQ_BF16, K, N, ldw, s, colmax, wq, w_scale, stream);
    return hip_result(e, fn);
}

sq_status sq_quant_weight_noalloc(const void* w, sq_dtype wt, int64_t K, int64_t N, int64_t ldw, const float* s,
                                  int8_t* wq, float* w_scale, hipStream_t stream) {
    const char* fn = "sq_quant_weight_noalloc";
    SQ_TRY(check_k(fn, K));
    if (N > sqk::noalloc_scratch_cols())
        return fail(SQ_ERR_WORKSPACE, "%s: N = %lld output channels exceed the %lld of the library's static scratch",
                    fn, (long long)N, (long long)sqk::noalloc_scratch_cols());
    SQ_TRY(check_matrix(fn, "w", w, wt, K, N, ldw, false));
    if (s) SQ_TRY(check_vec(fn, "s", s, K));
    SQ_TRY(check_vec(fn, "w_scale", w_scale, N, true));
    if (K > 0 && N > 0) {
        if (!wq) return fail(SQ_ERR_INVALID_ARG, "%s: wq is NULL", fn);
        if (!aligned16(wq)) return fail(SQ_ERR_INVALID_ARG, "%s: wq is not 16-byte aligned", fn);
    }
    if (N == 0) return ok();
    if (K == 0)  // no input channels: every column max is 0, so every scale is 0
        return hip_result(sqk::launch_fill_u32(reinterpret_cast<uint32_t*>(w_scale), N, 0u, stream), fn);
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_result(e, fn);
    if (stream) {
        int sdev = 0;
        e = hipStreamGetDevice(stream, &sdev);
        if (e != hipSuccess) return hip_result(e, fn);
        if (sdev != dev)
            return fail(SQ_ERR_INVALID_ARG, "%s: the stream belongs to device %d, the current device is %d", fn, sdev,
                        dev);
    }
    void* scratch = nullptr;
    e = sqk::noalloc_scratch(dev, &scratch);
    if (e != hipSuccess) return fail(SQ_ERR_HIP, "%s: no device address of the static scratch: %s", fn,
                                     hipGetErrorString(e));
    // the same three launches as sq_quant_weight, with the static scratch as
    // the column maxima (cleared first: it keeps the previous call's values)
    uint32_t* colmax = static_cast<uint32_t*>(scratch);
    e = sqk::launch_fill_u32(colmax, N, 0u, stream);
    if (e == hipSuccess) e = sqk::launch_col_absmax(w, wt == SQ_BF16, K, N, ldw, s, colmax, stream);
    if (e == hipSuccess) e = sqk::launch_quant_weight(w, wt == SQ_BF16, K, N, ldw, s, colmax, wq, w_scale, stream);
    return hip_result(e, fn);
}

sq_status sq_prepare_weights(const float* amax_x, const void* w, sq_dtype wt, int64_t K, int64_t N, int64_t ldw,
                             float alpha, float* s, float* inv_s, float* amax_w, int8_t* wq, float* w_scale, void* ws,
                             size_t ws_bytes, hipStream_t stream) {
    const char* fn = "sq_prepare_weights";
    SQ_TRY(check_k(fn, K));
    if (!(alpha >= 0.0f && alpha <= 1.0f)) return fail(SQ_ERR_INVALID_ARG, "%s: alpha = %g is not in [0, 1]", fn, alpha);
    if (N > kMaxMN) return fail(SQ_ERR_INVALID_ARG, "%s: N = %lld too large", fn, (long long)N);
    if (K > 0 && N <= 0) return fail(SQ_ERR_INVALID_ARG, "%s: N = %lld must be positive", fn, (long long)N);
    SQ_TRY(check_vec(fn, "amax_x", amax_x, K));
    SQ_TRY(check_vec(fn, "s", s, K));
    SQ_TRY(check_vec(fn, "inv_s", inv_s, K));
    if (amax_w) SQ_TRY(check_vec(fn, "amax_w", amax_w, K));
    SQ_TRY(check_matrix(fn, "w", w, wt, K, N, ldw, false));
    SQ_TRY(check_vec(fn, "w_scale", w_scale, N, true));
    if (K > 0 && N > 0) {
        if (!wq) return fail(SQ_ERR_INVALID_ARG, "%s: wq is NULL", fn);
        if (!aligned16(wq)) return fail(SQ_ERR_INVALID_ARG, "%s: wq is not 16-byte aligned", fn);
    }
    const size_t need = sq_workspace_size(SQ_OP_PREPARE_WEIGHTS, 0, N, K, SQ_PER_TOKEN);
    if (need > 0 && (!ws || ws_bytes < need || !aligned16(ws)))
        return fail(SQ_ERR_WORKSPACE, "%s: workspace of %zu bytes (16-byte aligned) required, got %zu", fn, need,
                    ws ? ws_bytes : (size_t)0);
    if (N == 0) return ok();
    if (K == 0)  // no input channels: every column max is 0, so every scale is 0
        return hip_result(sqk::launch_fill_u32(reinterpret_cast<uint32_t*>(w_scale), N, 0u, stream), fn);
    const bool bf16 = wt == SQ_BF16;
    uint32_t* colmax = static_cast<uint32_t*>(ws);
    float* partial = reinterpret_cast<float*>(static_cast<char*>(ws) + round256((size_t)N * sizeof(uint32_t)));
    double* tab = prep_tables(ws, N, K);
    hipError_t e;
    // The one-read pass (row maxima, factors and column maxima together) is
    // faster than the separate passes at every size it supports.
    if (sqk::prep_fused_supported(w, bf16, N, ldw, alpha)) {
        e = sqk::launch_prepare_weights(w, bf16, K, N, ldw, amax_x, alpha, s, inv_s, amax_w, partial, colmax, tab,
                                        stream);
    } else {
        e = sqk::launch_row_absmax_factors(w, bf16, K, N, ldw, amax_x, alpha, s, inv_s, amax_w, stream);
        if (e == hipSuccess) e = sqk::launch_fill_u32(colmax, N, 0u, stream);
        if (e == hipSuccess) e = sqk::launch_col_absmax(w, bf16, K, N, ldw, s, colmax, stream);
    }
    if (e == hipSuccess) e = sqk::launch_quant_weight(w, bf16, K, N, ldw, s, colmax, wq, w_scale, stream);
    return hip_result(e, fn);
}

sq_status sq_quant_act(const void* x, sq_dtype xt, int64_t M, int64_t K, int64_t ldx, const float* inv_s,
                       sq_act_gran g, int8_t* xq, float* x_scale, void* ws, size_t ws_bytes, hipStream_t stream) {
    const char* fn = "sq_quant_act";
    SQ_TRY(check_k(fn, K));
    if (g != SQ_PER_TOKEN && g != SQ_PER_TENSOR) return fail(SQ_ERR_UNSUPPORTED, "%s: granularity %d", fn, (int)g);
    if (M > kMaxMN) return fail(SQ_ERR_INVALID_ARG, "%s: M = %lld too large", fn, (long long)M);
    SQ_TRY(check_matrix(fn, "x", x, xt, M, K, ldx));
    if (inv_s) SQ_TRY(check_vec(fn, "inv_s", inv_s, K, true));
    SQ_TRY(check_vec(fn, "x_scale", x_scale, g == SQ_PER_TENSOR ? (M > 0 ? 1 : 0) : M));
    if (M > 0 && K > 0) {
        if (!xq) return fail(SQ_ERR_INVALID_ARG, "%s: xq is NULL", fn);
        if (!aligned16(xq)) return fail(SQ_ERR_INVALID_ARG, "%s: xq is not 16-byte aligned", fn);
    }
    const size_t need = sq_workspace_size(SQ_OP_QUANT_ACT, M, 0, K, g);
    if (need > 0 && (!ws || ws_bytes < need || !aligned16(ws)))
        return fail(SQ_ERR_WORKSPACE, "%s: workspace of %zu bytes (16-byte aligned) required, got %zu", fn, need,
                    ws ? ws_bytes : (size_t)0);
    if (M == 0) return ok();
    const bool bf = xt == SQ_BF16;
    if (g == SQ_PER_TOKEN)
        return hip_result(sqk::launch_quant_act(x, bf, M, K, ldx, inv_s, 0, xq, x_scale, nullptr, stream), fn);
    uint32_t* gmax = static_cast<uint32_t*>(ws);
    hipError_t e = sqk::launch_fill_u32(gmax, 1, 0u, stream);
    if (e == hipSuccess) e = sqk::launch_quant_act(x, bf, M, K, ldx, inv_s, 1, xq, x_scale, gmax, stream);
    if (e == hipSuccess) e = sqk::launch_quant_act(x, bf, M, K, ldx, inv_s, 2, xq, x_scale, gmax, stream);
    return hip_result(e, fn);
}

sq_status sq_prepare_and_quant_act(const float* amax_x, const void* w, sq_dtype wt, int64_t K, int64_t N,
                                   int64_t ldw, float alpha, float* s, float* inv_s, float* amax_w, int8_t* wq,
                                   float* w_scale, const void* x, sq_dtype xt, int64_t M, int64_t ldx,
                                   sq_act_gran g, int8_t* xq, float* x_scale, void* ws, size_t ws_bytes,
                                   hipStream_t stream) {
    const char* fn = "sq_prepare_and_quant_act";
    // sq_quant_act's checks first, so that a rejection enqueues nothing on
    // either path; sq_prepare_weights makes its own below
    SQ_TRY(check_k(fn, K));
    if (g != SQ_PER_TOKEN && g != SQ_PER_TENSOR) return fail(SQ_ERR_UNSUPPORTED, "%s: granularity %d", fn, (int)g);
    if (M > kMaxMN) return fail(SQ_ERR_INVALID_ARG, "%s: M = %lld too large", fn, (long long)M);
    SQ_TRY(check_matrix(fn, "x", x, xt, M, K, ldx));
    SQ_TRY(check_vec(fn, "inv_s", inv_s, K, true));
    SQ_TRY(check_vec(fn, "x_scale", x_scale, g == SQ_PER_TENSOR ? (M > 0 ? 1 : 0) : M));
    if (M > 0 && K > 0) {
        if (!xq) return fail(SQ_ERR_INVALID_ARG, "%s: xq is NULL", fn);
        if (!aligned16(xq)) return fail(SQ_ERR_INVALID_ARG, "%s: xq is not 16-byte aligned", fn);
    }
    const size_t need = sq_workspace_size(SQ_OP_PREPARE_AND_QUANT_ACT, M, N, K, g);
    if (need > 0 && (!ws || ws_bytes < need || !aligned16(ws)))
        return fail(SQ_ERR_WORKSPACE, "%s: workspace of %zu bytes (16-byte aligned) required, got %zu", fn, need,
                    ws ? ws_bytes : (size_t)0);
    const size_t wsp = round256(sq_workspace_size(SQ_OP_PREPARE_WEIGHTS, M, N, K, g));
    void* ws_a = ws && wsp < ws_bytes ? static_cast<void*>(static_cast<char*>(ws) + wsp) : nullptr;
    const size_t ws_a_bytes = ws_bytes > wsp ? ws_bytes - wsp : 0;

    const bool fast = M > 0 && K > 0 && N > 0 && wt == SQ_BF16 && xt == SQ_BF16 && g == SQ_PER_TOKEN &&
                      sqk::prep_fused_supported(w, true, N, ldw, alpha);
    if (!fast) {
        SQ_TRY(sq_prepare_weights(amax_x, w, wt, K, N, ldw, alpha, s, inv_s, amax_w, wq, w_scale, ws, wsp, stream));
        return sq_quant_act(x, xt, M, K, ldx, inv_s, g, xq, x_scale, ws_a, ws_a_bytes, stream);
    }
    // sq_prepare_weights' checks
    if (!(alpha >= 0.0f && alpha <= 1.0f)) return fail(SQ_ERR_INVALID_ARG, "%s: alpha = %g is not in [0, 1]", fn, alpha);
    if (N > kMaxMN) return fail(SQ_ERR_INVALID_ARG, "%s: N = %lld too large", fn, (long long)N);
    SQ_TRY(check_vec(fn, "amax_x", amax_x, K));
    SQ_TRY(check_vec(fn, "s", s, K));
    if (amax_w) SQ_TRY(check_vec(fn, "amax_w", amax_w, K));
    SQ_TRY(check_matrix(fn, "w", w, wt, K, N, ldw, false));
    SQ_TRY(check_vec(fn, "w_scale", w_scale, N, true));
    if (!wq) return fail(SQ_ERR_INVALID_ARG, "%s: wq is NULL", fn);
    if (!aligned16(wq)) return fail(SQ_ERR_INVALID_ARG, "%s: wq is not 16-byte aligned", fn);

    uint32_t* colmax = static_cast<uint32_t*>(ws);
    float* partial = reinterpret_cast<float*>(static_cast<char*>(ws) + round256((size_t)N * sizeof(uint32_t)));
    hipError_t e = sqk::launch_prepare_weights(w, true, K, N, ldw, amax_x, alpha, s, inv_s, amax_w, partial, colmax,
                                               prep_tables(ws, N, K), stream);
    if (e != hipSuccess) return hip_result(e, fn);
    e = sqk::launch_codes_both(w, K, N, ldw, s, colmax, wq, w_scale, x, M, ldx, inv_s, xq, x_scale, stream);
    if (e == hipErrorNotSupported) {  // K > 4096 or X rows not 16-byte aligned: the two code launches
        e = sqk::launch_quant_weight(w, true, K, N, ldw, s, colmax, wq, w_scale, stream);
        if (e == hipSuccess) e = sqk::launch_quant_act(x, true, M, K, ldx, inv_s, 0, xq, x_scale, nullptr, stream);
    }
    return hip_result(e, fn);
}

sq_status sq_fold_layernorm(const float* gamma, const float* beta, const float* inv_s, int64_t K, float* gamma_out,
                            float* beta_out, hipStream_t stream) {
    const char* fn = "sq_fold_layernorm";
    if (K < 0) return fail(SQ_ERR_INVALID_ARG, "%s: K = %lld is negative", fn, (long long)K);
    SQ_TRY(check_vec(fn, "gamma", gamma, K));
    SQ_TRY(check_vec(fn, "inv_s", inv_s, K));
    SQ_TRY(check_vec(fn, "gamma_out", gamma_out, K));
    if (beta) SQ_TRY(check_vec(fn, "beta_out", beta_out, K));
    return hip_result(sqk::launch_fold_ln(gamma, beta, inv_s, K, gamma_out, beta_out, stream), fn);
}

sq_status sq_layernorm_quant(const void* x, sq_dtype xt, int64_t M, int64_t K, int64_t ldx, const float* gamma,
                             const float* beta, float eps, int8_t* xq, float* x_scale, hipStream_t stream) {
    const char* fn = "sq_layernorm_quant";
    SQ_TRY(check_k(fn, K));
    if (xt != SQ_BF16) return fail(SQ_ERR_UNSUPPORTED, "%s: only bf16 rows are supported", fn);
    if (K > 16384) return fail(SQ_ERR_UNSUPPORTED, "%s: K = %lld above 16384", fn, (long long)K);
    if (M > kMaxMN) return fail(SQ_ERR_INVALID_ARG, "%s: M = %lld too large", fn, (long long)M);
    if (!(eps >= 0.0f)) return fail(SQ_ERR_INVALID_ARG, "%s: eps = %g must be >= 0", fn, eps);
    SQ_TRY(check_matrix(fn, "x", x, xt, M, K, ldx));
    SQ_TRY(check_vec(fn, "gamma", gamma, K, true));
    if (beta) SQ_TRY(check_vec(fn, "beta", beta, K, true));
    SQ_TRY(check_vec(fn, "x_scale", x_scale, M));
    if (M > 0 && K > 0) {
        if (!xq) return fail(SQ_ERR_INVALID_ARG, "%s: xq is NULL", fn);
        if (!aligned16(xq)) return fail(SQ_ERR_INVALID_ARG, "%s: xq is not 16-byte aligned", fn);
    }
    if (M == 0) return ok();
    if (K == 0) return hip_result(sqk::launch_fill_u32(reinterpret_cast<uint32_t*>(x_scale), M, 0u, stream), fn);
    return hip_result(sqk::launch_ln_quant(x, M, K, ldx, gamma, beta, eps, xq, x_scale, stream), fn);
}

sq_status sq_static_act_max(const float* amax_x, const float* inv_s, int64_t K, float* a_static, hipStream_t stream) {
    const char* fn = "sq_static_act_max";
    SQ_TRY(check_k(fn, K));
    SQ_TRY(check_vec(fn, "amax_x", amax_x, K));
    if (inv_s) SQ_TRY(check_vec(fn, "inv_s", inv_s, K));
    SQ_TRY(check_vec(fn, "a_static", a_static, 1));
    return hip_result(sqk::launch_static_max(amax_x, inv_s, K, a_static, stream), fn);
}

sq_status sq_quant_act_static(const void* x, sq_dtype xt, int64_t M, int64_t K, int64_t ldx, const float* inv_s,
                              const float* a_static, int8_t* xq, float* x_scale, hipStream_t stream) {
    const char* fn = "sq_quant_act_static";
    SQ_TRY(check_k(fn, K));
    if (M > kMaxMN) return fail(SQ_ERR_INVALID_ARG, "%s: M = %lld too large", fn, (long long)M);
    SQ_TRY(check_matrix(fn, "x", x, xt, M, K, ldx));
    if (inv_s) SQ_TRY(check_vec(fn, "inv_s", inv_s, K, true));
    SQ_TRY(check_vec(fn, "a_static", a_static, 1));
    SQ_TRY(check_vec(fn, "x_scale", x_scale, M > 0 ? 1 : 0));
    if (M > 0 && K > 0) {
        if (!xq) return fail(SQ_ERR_INVALID_ARG, "%s: xq is NULL", fn);
        if (!aligned16(xq)) return fail(SQ_ERR_INVALID_ARG, "%s: xq is not 16-byte aligned", fn);
    }
    if (M == 0) return ok();
    // mode 2 of the activation kernels: codes from a given tensor maximum (read only)
    uint32_t* a_bits = const_cast<uint32_t*>(reinterpret_cast<const uint32_t*>(a_static));
    return hip_result(sqk::launch_quant_act(x, xt == SQ_BF16, M, K, ldx, inv_s, 2, xq, x_scale, a_bits, stream), fn);
}

sq_status sq_gemm_w8a8(const int8_t* xq, const float* x_scale, sq_act_gran g, const int8_t* wq, const float* w_scale,
                       int64_t M, int64_t N, int64_t K, void* y, sq_dtype yt, int32_t* acc_out, void* ws,
                       size_t ws_bytes, hipStream_t stream) {
    const char* fn = "sq_gemm_w8a8";
    (void)ws;
    (void)ws_bytes;
    SQ_TRY(check_k(fn, K));
    if (g != SQ_PER_TOKEN && g != SQ_PER_TENSOR) return fail(SQ_ERR_UNSUPPORTED, "%s: granularity %d", fn, (int)g);
    if (!dtype_ok(yt)) return fail(SQ_ERR_UNSUPPORTED, "%s: output dtype %d", fn, (int)yt);
    if (M < 0 || N < 0 || M > kMaxMN || N > kMaxMN)
        return fail(SQ_ERR_INVALID_ARG, "%s: M = %lld, N = %lld out of range", fn, (long long)M, (long long)N);
    if (M == 0 || N == 0) return ok();
    if (K > 0) {
        if (!xq || !wq) return fail(SQ_ERR_INVALID_ARG, "%s: xq or wq is NULL", fn);
        if (!aligned16(xq) || !aligned16(wq))
            return fail(SQ_ERR_INVALID_ARG, "%s: xq and wq must be 16-byte aligned", fn);
    }
    SQ_TRY(check_vec(fn, "x_scale", x_scale, g == SQ_PER_TENSOR ? 1 : M));
    SQ_TRY(check_vec(fn, "w_scale", w_scale, N, true));
    if (!y) return fail(SQ_ERR_INVALID_ARG, "%s: y is NULL", fn);
    if (!aligned16(y)) return fail(SQ_ERR_INVALID_ARG, "%s: y is not 16-byte aligned", fn);
    if (acc_out && !aligned16(acc_out)) return fail(SQ_ERR_INVALID_ARG, "%s: acc_out is not 16-byte aligned", fn);
    return hip_result(sqk::launch_gemm_w8a8(xq, x_scale, g == SQ_PER_TENSOR, wq, w_scale, M, N, K, y, yt == SQ_BF16,
                                            acc_out, stream), fn);
}

sq_status sq_outlier_columns(const float* amax_x, int64_t K, float threshold, int32_t* idx, int32_t* count,
                             float* keep, hipStream_t stream) {
    const char* fn = "sq_outlier_columns";
    SQ_TRY(check_k(fn, K));
    if (threshold != threshold) return fail(SQ_ERR_INVALID_ARG, "%s: threshold is NaN", fn);
    SQ_TRY(check_vec(fn, "amax_x", amax_x, K));
    SQ_TRY(check_vec(fn, "idx", idx, K));
    SQ_TRY(check_vec(fn, "keep", keep, K, true));
    SQ_TRY(check_vec(fn, "count", count, 1));
    return hip_result(sqk::launch_outlier_columns(amax_x, K, threshold, idx, count, keep, stream), fn);
}

sq_status sq_gather_outliers(const void* x, sq_dtype xt, int64_t M, int64_t K, int64_t ldx, const void* w,
                             sq_dtype wt, int64_t N, int64_t ldw, const int32_t* idx, const int32_t* count,
                             int64_t kp, void* x_o, void* w_ot, hipStream_t stream) {
    const char* fn = "sq_gather_outliers";
    SQ_TRY(check_k(fn, K));
    if (xt != SQ_BF16 || wt != SQ_BF16) return fail(SQ_ERR_UNSUPPORTED, "%s: x and w must be bf16", fn);
    if (M < 0 || N < 0 || M > kMaxMN || N > kMaxMN)
        return fail(SQ_ERR_INVALID_ARG, "%s: M = %lld, N = %lld out of range", fn, (long long)M, (long long)N);
    SQ_TRY(check_matrix(fn, "x", x, xt, M, K, ldx, false));
    SQ_TRY(check_matrix(fn, "w", w, wt, K, N, ldw, false));
    if (kp % 16 != 0 || kp < (K + 15) / 16 * 16)
        return fail(SQ_ERR_INVALID_ARG, "%s: kp = %lld must be a multiple of 16 and at least K rounded up to 16", fn,
                    (long long)kp);
    SQ_TRY(check_vec(fn, "idx", idx, K));
    SQ_TRY(check_vec(fn, "count", count, 1));
    if (M > 0) SQ_TRY(check_vec(fn, "x_o", x_o, 1, true));
    if (N > 0) SQ_TRY(check_vec(fn, "w_ot", w_ot, 1, true));
    if (K == 0) return ok();  // no channel, so no outlier: nothing is read by the GEMM
    return hip_result(sqk::launch_gather_outliers(static_cast<const uint16_t*>(x), M, ldx,
                                                  static_cast<const uint16_t*>(w), N, ldw, idx, count, kp,
                                                  static_cast<uint16_t*>(x_o), static_cast<uint16_t*>(w_ot), stream),
                      fn);
}

sq_status sq_gemm_w8a8_outlier(const int8_t* xq, const float* x_scale, const int8_t* wq, const float* w_scale,
                               int64_t M, int64_t N, int64_t K, const void* x_o, const void* w_ot, int64_t kp,
                               const int32_t* count, void* y, sq_dtype yt, hipStream_t stream) {
    const char* fn = "sq_gemm_w8a8_outlier";
    SQ_TRY(check_k(fn, K));
    if (!dtype_ok(yt)) return fail(SQ_ERR_UNSUPPORTED, "%s: output dtype %d", fn, (int)yt);
    if (M < 0 || N < 0 || M > kMaxMN || N > kMaxMN)
        return fail(SQ_ERR_INVALID_ARG, "%s: M = %lld, N = %lld out of range", fn, (long long)M, (long long)N);
    if (kp % 16 != 0 || kp < (K + 15) / 16 * 16)
        return fail(SQ_ERR_INVALID_ARG, "%s: kp = %lld must be a multiple of 16 and at least K rounded up to 16", fn,
                    (long long)kp);
    if (M == 0 || N == 0) return ok();
    if (K > 0) {
        if (!xq || !wq) return fail(SQ_ERR_INVALID_ARG, "%s: xq or wq is NULL", fn);
        if (!aligned16(xq) || !aligned16(wq))
            return fail(SQ_ERR_INVALID_ARG, "%s: xq and wq must be 16-byte aligned", fn);
    }
    SQ_TRY(check_vec(fn, "x_scale", x_scale, M));
    SQ_TRY(check_vec(fn, "w_scale", w_scale, N, true));
    SQ_TRY(check_vec(fn, "count", count, 1));
    if (kp > 0) {
        SQ_TRY(check_vec(fn, "x_o", x_o, 1, true));
        SQ_TRY(check_vec(fn, "w_ot", w_ot, 1, true));
    }
    if (!y) return fail(SQ_ERR_INVALID_ARG, "%s: y is NULL", fn);
    if (!aligned16(y)) return fail(SQ_ERR_INVALID_ARG, "%s: y is not 16-byte aligned", fn);
    return hip_result(sqk::launch_gemm_w8a8_outlier(xq, x_scale, wq, w_scale, M, N, K,
                                                    static_cast<const uint16_t*>(x_o),
                                                    static_cast<const uint16_t*>(w_ot), kp, count, y,
                                                    yt == SQ_BF16, stream),
                      fn);
}

const char* sq_gemm_outlier_kernel_name(int64_t M, int64_t N, int64_t K) {
    return sqk::gemm_kernel_name(M, N, K, true);
}

sq_status sq_matmul_f64(const void* x, sq_dtype xt, int64_t M, int64_t K, int64_t ldx, const void* w, sq_dtype wt,
                        int64_t N, int64_t ldw, double* y_ref, hipStream_t stream) {
    const char* fn = "sq_matmul_f64";
    SQ_TRY(check_k(fn, K));
    if (M < 0 || N < 0 || M > kMaxMN || N > sqk::kMatmulF64MaxN)
        return fail(SQ_ERR_INVALID_ARG, "%s: M = %lld, N = %lld out of range (N <= %lld)", fn, (long long)M,
                    (long long)N, (long long)sqk::kMatmulF64MaxN);
    SQ_TRY(check_matrix(fn, "x", x, xt, M, K, ldx, false));
    SQ_TRY(check_matrix(fn, "w", w, wt, K, N, ldw, false));
    if (M == 0 || N == 0) return ok();
    if (!y_ref) return fail(SQ_ERR_INVALID_ARG, "%s: y_ref is NULL", fn);
    if (reinterpret_cast<uintptr_t>(y_ref) & 7u) return fail(SQ_ERR_INVALID_ARG, "%s: y_ref is not 8-byte aligned", fn);
    return hip_result(sqk::launch_matmul_f64(x, xt == SQ_BF16, M, K, ldx, w, wt == SQ_BF16, N, ldw, y_ref, stream),
                      fn);
}

sq_status sq_rel_error(const float* y, const double* y_ref, int64_t M, int64_t N, double* err, void* ws,
                       size_t ws_bytes, hipStream_t stream) {
    const char* fn = "sq_rel_error";
    if (M < 0 || N < 0 || M > kMaxMN || N > kMaxMN)
        return fail(SQ_ERR_INVALID_ARG, "%s: M = %lld, N = %lld out of range", fn, (long long)M, (long long)N);
    SQ_TRY(check_vec(fn, "y", y, M * N));
    if (M * N > 0 && !y_ref) return fail(SQ_ERR_INVALID_ARG, "%s: y_ref is NULL", fn);
    if (reinterpret_cast<uintptr_t>(y_ref) & 7u) return fail(SQ_ERR_INVALID_ARG, "%s: y_ref is not 8-byte aligned", fn);
    if (!err || (reinterpret_cast<uintptr_t>(err) & 7u))
        return fail(SQ_ERR_INVALID_ARG, "%s: err is NULL or not 8-byte aligned", fn);
    const size_t need = sq_workspace_size(SQ_OP_REL_ERROR, M, N, 0, SQ_PER_TOKEN);
    if (!ws || ws_bytes < need || (reinterpret_cast<uintptr_t>(ws) & 7u))
        return fail(SQ_ERR_WORKSPACE, "%s: workspace of %zu bytes at %p, need %zu bytes, 8-byte aligned", fn,
                    ws_bytes, ws, need);
    return hip_result(sqk::launch_rel_error(y, y_ref, M * N, err, static_cast<double*>(ws), stream), fn);
}

}  // extern "C"
