// Internal launchers of the gfx950 kernels (host side).  Each returns the
// HIP error of its launch; argument validation happens in the C ABI layer.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace sqk {

hipError_t launch_fill_u32(uint32_t* out, int64_t n, uint32_t v, hipStream_t st);

// out[c] = max(out[c], max_r |row_scale[r] * x[r, c]|) as fp32 bit patterns.
hipError_t launch_col_absmax(const void* x, bool bf16, int64_t rows, int64_t cols, int64_t ld,
                             const float* row_scale, uint32_t* out, hipStream_t st);

// amax_w[j] = max_k |w[j, k]| (optional output), then s[j], inv_s[j].
hipError_t launch_row_absmax_factors(const void* w, bool bf16, int64_t K, int64_t N, int64_t ld,
                                     const float* amax_x, float alpha, float* s, float* inv_s, float* amax_w,
                                     hipStream_t st);

// Steps 2 + 3a in one read of W (bf16, 16-byte aligned rows, N % 8 == 0,
// N <= 49152): amax_w (optional), s, inv_s and the column maxima of diag(s) W
// into colmax (fp32 bits), through per-block partial maxima
// partial[prep_blocks(K)][N].  hipErrorNotSupported (nothing enqueued) when
// prep_fused_supported() is false.
// For alpha outside {0, 1/2, 1} the powers of s come from tables of
// prep_table_entries(K) doubles at tab (built by the call; tab must not be
// NULL).
int prep_blocks(int64_t K);
int64_t prep_table_entries(int64_t K);
bool prep_fused_supported(const void* w, bool bf16, int64_t N, int64_t ld, float alpha);
hipError_t launch_prepare_weights(const void* w, bool bf16, int64_t K, int64_t N, int64_t ld, const float* amax_x,
                                  float alpha, float* s, float* inv_s, float* amax_w, float* partial,
                                  uint32_t* colmax, double* tab, hipStream_t st);

// out[0] = max_j fl(amax_x[j] * inv_s[j]) (inv_s may be NULL).
hipError_t launch_static_max(const float* amax_x, const float* inv_s, int64_t K, float* out, hipStream_t st);

hipError_t launch_factors(const float* amax_x, const float* amax_w, int64_t K, float alpha, float* s,
                          float* inv_s, hipStream_t st);

// Codes of diag(s) W per output column from the column maxima colmax (fp32
// bits), written transposed to wq[N, K]; w_scale[N].
hipError_t launch_quant_weight(const void* w, bool bf16, int64_t K, int64_t N, int64_t ld, const float* s,
                               const uint32_t* colmax, int8_t* wq, float* w_scale, hipStream_t st);

// Activation quantization.  mode 0: per token.  mode 1: max of |x * inv_s|
// over the tensor into *gmax (no codes).  mode 2: codes with the scale from
// *gmax (x_scale[0]).
// Weight codes (as launch_quant_weight with s) and per-token activation codes
// (as launch_quant_act mode 0 with inv_s) in one launch, for bf16 W and X with
// 16-byte aligned rows and K <= 4096.  hipErrorNotSupported (nothing
// enqueued) for other inputs.
hipError_t launch_codes_both(const void* w, int64_t K, int64_t N, int64_t ldw, const float* s, const uint32_t* colmax,
                             int8_t* wq, float* w_scale, const void* x, int64_t M, int64_t ldx, const float* inv_s,
                             int8_t* xq, float* x_scale, hipStream_t st);
hipError_t launch_quant_act(const void* x, bool bf16, int64_t M, int64_t K, int64_t ld, const float* inv_s,
                            int mode, int8_t* xq, float* x_scale, uint32_t* gmax, hipStream_t st);

// LayerNorm fold: gamma_out = fl(gamma * inv_s), beta_out = fl(beta * inv_s) (beta may be NULL).
hipError_t launch_fold_ln(const float* gamma, const float* beta, const float* inv_s, int64_t K, float* gamma_out,
                          float* beta_out, hipStream_t st);
// LayerNorm (fp64 statistics) of bf16 rows with gamma/beta, then per-token codes; K / 8 <= 2048
// (hipErrorNotSupported beyond).
hipError_t launch_ln_quant(const void* x, int64_t M, int64_t K, int64_t ld, const float* gamma, const float* beta,
                           float eps, int8_t* xq, float* x_scale, hipStream_t st);

// INT8 GEMM + dequant epilogue.
hipError_t launch_gemm_w8a8(const int8_t* xq, const float* x_scale, bool per_tensor, const int8_t* wq,
                            const float* w_scale, int64_t M, int64_t N, int64_t K, void* y, bool y_bf16,
                            int32_t* acc_out, hipStream_t st);

// The same product plus the 16-bit outlier addend of the LLM.int8()-style
// comparator (per-token x_scale): y = fl(y8 + sum_t w_ot[n, t] x_o[m, t]) over
// the *count outlier channels, operands [N, kp] and [M, kp] bf16, zero-padded
// to a multiple of 16 channels.
hipError_t launch_gemm_w8a8_outlier(const int8_t* xq, const float* x_scale, const int8_t* wq, const float* w_scale,
                                    int64_t M, int64_t N, int64_t K, const uint16_t* x_o, const uint16_t* w_ot,
                                    int64_t kp, const int32_t* count, void* y, bool y_bf16, hipStream_t st);

// The static scratch of sq_quant_weight_noalloc: room for noalloc_scratch_cols()
// column maxima; noalloc_scratch() gives its device address on `device`, which
// must be the current device (taken with hipGetSymbolAddress on the first call
// per device, then cached).
int64_t noalloc_scratch_cols();
hipError_t noalloc_scratch(int device, void** out);

// The alpha search's criterion: y[M, N] = x w in fp64 (x [M, K], w [K, N],
// bf16 or fp32, K % 16 == 0, y dense); err[0] = ||y - y_ref||_F / ||y_ref||_F
// over n elements through partial sums in rel_error_workspace_bytes() bytes.
// The product's grid has one y dimension per 128 output columns.
constexpr int64_t kMatmulF64MaxN = (int64_t)65535 * 128;
hipError_t launch_matmul_f64(const void* x, bool x_bf16, int64_t M, int64_t K, int64_t ldx, const void* w,
                             bool w_bf16, int64_t N, int64_t ldw, double* y, hipStream_t st);
int64_t rel_error_workspace_bytes();
hipError_t launch_rel_error(const float* y, const double* y_ref, int64_t n, double* err, double* partial,
                            hipStream_t st);

// Static description of the GEMM kernel launch_gemm_w8a8 (outl: the outlier
// variant) runs for this shape.
const char* gemm_kernel_name(int64_t M, int64_t N, int64_t K, bool outl = false);

// Outlier channels of the comparator: idx[0..*count) ascending with
// amax[j] > thr, keep[j] = 0 there and 1 elsewhere (one block).
hipError_t launch_outlier_columns(const float* amax, int64_t K, float thr, int32_t* idx, int32_t* count, float* keep,
                                  hipStream_t st);
// x_o[i, t] = x[i, idx[t]], w_ot[k, t] = w[idx[t], k] for t < *count, zero up to
// the next multiple of 16 (bf16 patterns; kp % 16 == 0, kp >= that multiple).
hipError_t launch_gather_outliers(const uint16_t* x, int64_t M, int64_t ldx, const uint16_t* w, int64_t N,
                                  int64_t ldw, const int32_t* idx, const int32_t* count, int64_t kp, uint16_t* x_o,
                                  uint16_t* w_ot, hipStream_t st);

}  // namespace sqk
