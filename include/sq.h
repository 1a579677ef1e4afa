/*
 * sq.h -- C ABI of the SmoothQuant W8A8 linear-layer library for AMD Instinct
 * MI355X (gfx950).
 *
 * The method (page "大模型训练、适配与推理" section 3.5; page "4.2 W8A8 量化与
 * SmoothQuant" sections 3, 4 and 7.1; page "量化：只压权重，与训练后量化（PTQ）"
 * section on SmoothQuant W8A8): for a linear layer Y = X W, with X[M,K]
 * (tokens x input channels) and W[K,N] (input channel j = row j), pick one
 * factor s_j per input channel, divide activation channel j by s_j and
 * multiply weight row j by s_j.  The product is unchanged in exact arithmetic,
 * but the activation outlier channels shrink, so both sides quantize well to
 * 8 bits.  Five calls implement the five steps:
 *
 *   1. sq_calib_absmax    per-input-channel max|X| over calibration tokens
 *   2. sq_smooth_factors  s_j = max|X_j|^alpha / max|W_j|^(1-alpha)
 *   3. sq_quant_weight    diag(s) W, one symmetric INT8 scale per output channel
 *   4. sq_quant_act       X diag(s)^-1, one symmetric INT8 scale per token
 *                         (or per tensor), scales computed at run time
 *   5. sq_gemm_w8a8       INT8 x INT8 -> int32 GEMM, then
 *                         y = (acc * x_scale_i) * w_scale_k rounded to bf16
 *
 * Arithmetic contract (what the kernels compute, bit for bit):
 *   - bf16 inputs widen exactly to fp32;
 *   - s_j is evaluated in fp64 from a = max(amax_x_j, 1e-5f) and
 *     b = max(amax_w_j, 1e-5f) as a^alpha / b^(1-alpha) (exponents 0, 1/2 and
 *     1 use the exact forms 1, sqrt, identity; others use fp64 pow) and rounded
 *     once to fp32; inv_s_j = 1/s_j correctly rounded in fp32;
 *   - a quantization group (a weight column, a token row or the whole
 *     activation tensor) with max magnitude m gets scale = fl(m/127) and
 *     multiplier r = fl(127/m) (0 when m = 0); each value v becomes
 *     clamp(round_half_even(fl(v * r)), -127, 127);
 *   - smoothed values are fl(s_j * w) and fl(x * inv_s_j), single roundings;
 *   - the GEMM accumulates exactly in int32 (K <= 131072 keeps
 *     |acc| <= K * 127^2 < 2^31), and the epilogue is
 *     fl(fl(float(acc) * x_scale_i) * w_scale_k), then round-to-nearest-even
 *     to bf16.
 *
 * Conventions for every call:
 *   - Pointers are DEVICE pointers unless stated.  Matrices are row-major; ld*
 *     is the row stride in elements.  Outputs are dense (no stride).
 *   - Every call is asynchronous on `stream` (NULL = the default stream of the
 *     current device) and returns after enqueueing.  Buffers must stay valid
 *     until the stream's work completes.  Calls on one stream are ordered.
 *   - The caller owns all memory.  The library allocates nothing.  Its only
 *     mutable global state is a per-thread error message, a per-device cache
 *     of the compute-unit count (filled on first use, read and written
 *     atomically; the GEMM's launch shape depends on it), and the static
 *     scratch array of sq_quant_weight_noalloc with its per-device address
 *     cache (see there).
 *   - Arguments are validated before anything is enqueued; a failed check
 *     returns a negative sq_status, enqueues nothing and records a message for
 *     sq_last_error().  A launch failure returns SQ_ERR_HIP.
 *   - Requirements checked: non-NULL required pointers; sizes >= 0;
 *     K % 16 == 0 and K <= 131072; ld >= row length; activation inputs (x),
 *     int8 codes, outputs and per-channel vectors read as vectors (inv_s,
 *     w_scale) 16-byte aligned, with activation row strides a multiple of 16
 *     bytes; weight inputs (w) only need element alignment and any row stride
 *     (rows that are not 16-byte aligned are read element by element, slower).
 *     M, N and the token count T may be any non-negative value (ragged tails
 *     are handled).
 *     Empty problems (a zero size) enqueue nothing and return SQ_OK, except
 *     sq_gemm_w8a8 and sq_matmul_f64 with K = 0, which write y = 0 (y_ref = 0),
 *     and sq_rel_error, which always writes its quotient (NaN over no
 *     elements).
 *   - Inputs must be finite; results for NaN or Inf inputs are unspecified.
 */
#ifndef SQ_H
#define SQ_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    SQ_OK = 0,
    SQ_ERR_INVALID_ARG = -1, /* bad pointer, size, stride or alignment */
    SQ_ERR_UNSUPPORTED = -2, /* valid but not implemented (dtype, granularity) */
    SQ_ERR_WORKSPACE = -3,   /* workspace missing or smaller than sq_workspace_size() */
    SQ_ERR_HIP = -4          /* the HIP runtime reported an error at launch */
} sq_status;

typedef enum { SQ_F32 = 0, SQ_BF16 = 1 } sq_dtype;

typedef enum {
    SQ_PER_TOKEN = 0, /* one activation scale per row of X   (x_scale has M entries) */
    SQ_PER_TENSOR = 1 /* one activation scale for all of X   (x_scale has 1 entry)   */
} sq_act_gran;

typedef enum {
    SQ_OP_CALIB_ABSMAX = 0,
    SQ_OP_SMOOTH_FACTORS = 1,
    SQ_OP_QUANT_WEIGHT = 2,
    SQ_OP_QUANT_ACT = 3,
    SQ_OP_GEMM_W8A8 = 4,
    SQ_OP_PREPARE_WEIGHTS = 5,
    SQ_OP_PREPARE_AND_QUANT_ACT = 6,
    SQ_OP_REL_ERROR = 7
} sq_op;

/*
 * Step 1 -- calibration absmax (page "4.2 W8A8 量化与 SmoothQuant" section 7.1:
 * activation statistics come from calibration data, one max|X_j| per input
 * channel; page "量化：只压权重..." SmoothQuant W8A8: X_j is measured on the
 * calibration set).
 *
 *   x     [T, K] row-major, dtype xt (SQ_BF16 or SQ_F32), row stride ldx.
 *   amax  [K] fp32, IN/OUT running maximum: amax[j] = max(amax[j], max_t |x[t,j]|).
 *         Zero it before the first chunk; call again with further chunks to
 *         continue (any chunking gives the same result).  Entries must be
 *         non-negative (0 or a previous result).
 */
sq_status sq_calib_absmax(const void *x, sq_dtype xt, int64_t T, int64_t K, int64_t ldx,
                          float *amax, hipStream_t stream);

/*
 * Start of a calibration: amax[j] = 0 for j < K (K >= 0; amax may be NULL when
 * K is 0).  One small kernel and no memset, so the call may be recorded in a
 * HIP graph; the same as clearing amax any other way before the first
 * sq_calib_absmax.
 */
sq_status sq_calib_reset(float *amax, int64_t K, hipStream_t stream);

/*
 * Step 2 -- smoothing factors (page "大模型训练、适配与推理" section 3.5; page
 * "4.2 W8A8 量化与 SmoothQuant" section 4; W_j is row j of W, the row that
 * multiplies activation channel j).
 *
 *   amax_x  [K] fp32 from step 1.
 *   w       [K, N] row-major, dtype wt, row stride ldw; or NULL.
 *   alpha   migration strength in [0, 1].
 *   s       [K] fp32 out: s_j.
 *   inv_s   [K] fp32 out: 1/s_j (what step 4 multiplies by).
 *   amax_w  [K] fp32: if w != NULL, optional output of max_k |W[j,k]| (may be
 *           NULL); if w == NULL, required INPUT (reuse of a previous result,
 *           e.g. to try several alpha without re-reading W).
 */
sq_status sq_smooth_factors(const float *amax_x, const void *w, sq_dtype wt, int64_t K, int64_t N,
                            int64_t ldw, float alpha, float *s, float *inv_s, float *amax_w,
                            hipStream_t stream);

/*
 * Step 3 -- smoothed weights, per-output-channel symmetric INT8 (page "4.2 W8A8
 * 量化与 SmoothQuant" section 7.1: the weights W' = diag(s) W are quantized
 * statically per channel; the channel is the output column, the reading that
 * reproduces the worked example of page "量化：只压权重...").
 *
 *   w        [K, N] row-major, dtype wt, row stride ldw.
 *   s        [K] fp32, or NULL to quantize W unsmoothed.
 *   wq       [N, K] int8 out, dense: output channel k's K codes are contiguous
 *            (the layout sq_gemm_w8a8 reads).
 *   w_scale  [N] fp32 out: max_j |W'[j,k]| / 127.
 *   ws       device workspace of at least sq_workspace_size(SQ_OP_QUANT_WEIGHT,
 *            0, N, K, 0) bytes, 16-byte aligned; its contents are scratch.
 */
sq_status sq_quant_weight(const void *w, sq_dtype wt, int64_t K, int64_t N, int64_t ldw,
                          const float *s, int8_t *wq, float *w_scale, void *ws, size_t ws_bytes,
                          hipStream_t stream);

/*
 * sq_quant_weight without a workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc): the per-column maxima live in a static scratch array
 * of the library instead of `ws`.  Same arguments (less ws) and the same
 * results as sq_quant_weight.
 *
 *   Limit: N <= 65536 output channels (the scratch holds 65536 maxima, 256 KB
 *   per GPU, kept until the process ends); larger N returns SQ_ERR_WORKSPACE
 *   and enqueues nothing.
 *   The scratch is one array per device, shared by every call on that device
 *   and cleared at the start of each call by a fill kernel (no memset, no
 *   allocation): calls that overlap on one device race, so serialize them (one
 *   stream, or events between streams).  `stream` must belong to the current
 *   device (SQ_ERR_INVALID_ARG otherwise).  The first call on a device looks up
 *   the scratch's device address (hipGetSymbolAddress, no allocation) and
 *   caches it; a failure there returns SQ_ERR_HIP.
 */
sq_status sq_quant_weight_noalloc(const void *w, sq_dtype wt, int64_t K, int64_t N, int64_t ldw, const float *s,
                                  int8_t *wq, float *w_scale, hipStream_t stream);

/*
 * Steps 2 and 3 in one call -- the offline weight preparation (page "4.2 W8A8
 * 量化与 SmoothQuant" section 7.1: factors from the calibration statistics,
 * then the smoothed weights quantized statically per channel).
 *
 * Computes exactly what sq_smooth_factors(amax_x, w, ..., alpha, s, inv_s,
 * amax_w) followed by sq_quant_weight(w, ..., s, wq, w_scale, ...) compute,
 * with the same arguments and results.  For a bf16 W with 16-byte aligned
 * rows, N % 8 == 0 and N <= 49152, it reads W once less: one pass over W
 * yields the row maxima, the factors and the column maxima of diag(s) W, and
 * a second pass writes the codes.  Other inputs take the two-call sequence
 * internally.
 *
 *   amax_x, w, wt, K, N, ldw, alpha, s, inv_s, amax_w   as sq_smooth_factors
 *                   (w is required; amax_w is an optional output);
 *   wq, w_scale     as sq_quant_weight;
 *   ws              workspace of sq_workspace_size(SQ_OP_PREPARE_WEIGHTS, 0, N,
 *                   K, 0) bytes, 16-byte aligned (column maxima and per-block
 *                   partial maxima, about 1 KB per output channel, then
 *                   (32769 + K) doubles: for alpha outside {0, 1/2, 1} the
 *                   fp64 powers of the factor rule are tabulated first, per
 *                   row of W and per bf16 value of a row maximum).
 */
sq_status sq_prepare_weights(const float *amax_x, const void *w, sq_dtype wt, int64_t K, int64_t N, int64_t ldw,
                             float alpha, float *s, float *inv_s, float *amax_w, int8_t *wq, float *w_scale,
                             void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * Step 4 -- fused smoothing and activation quantization (page "大模型训练、适配
 * 与推理" section 3.5: X'_ij = X_ij / s_j; page "4.2 W8A8 量化与 SmoothQuant"
 * section 7.1: per-token scales computed at run time; page "量化：只压权重..."
 * worked example: per-tensor and per-token activation scales).
 *
 *   x        [M, K] row-major, dtype xt, row stride ldx.
 *   inv_s    [K] fp32 from step 2, or NULL to quantize X unsmoothed.
 *   g        SQ_PER_TOKEN (x_scale[M]) or SQ_PER_TENSOR (x_scale[1]).
 *   xq       [M, K] int8 out, dense.
 *   x_scale  fp32 out (see g).
 *   ws       workspace of sq_workspace_size(SQ_OP_QUANT_ACT, M, 0, K, g) bytes
 *            (0 for SQ_PER_TOKEN, where ws may be NULL).
 */
sq_status sq_quant_act(const void *x, sq_dtype xt, int64_t M, int64_t K, int64_t ldx,
                       const float *inv_s, sq_act_gran g, int8_t *xq, float *x_scale, void *ws,
                       size_t ws_bytes, hipStream_t stream);

/*
 * Steps 2, 3 and 4 in one call -- the factors, the weight codes and the
 * activation codes of one batch (page "4.2 W8A8 量化与 SmoothQuant" section
 * 7.1; page "大模型训练、适配与推理" section 3.5).
 *
 * Computes exactly what sq_prepare_weights(amax_x, w, ..., alpha, s, inv_s,
 * amax_w, wq, w_scale, ...) followed by sq_quant_act(x, ..., inv_s, g, xq,
 * x_scale, ...) compute, with the same arguments and results; it rejects
 * what either of them rejects.  For bf16 W and X with 16-byte aligned rows, W
 * as the one-read pass of sq_prepare_weights takes it, K <= 4096 and
 * SQ_PER_TOKEN, the weight codes and the activation codes are written by one
 * launch (each alone leaves the memory system idle during its start and tail
 * at these sizes).  Other inputs take the two calls internally.
 *
 *   amax_x, w, wt, K, N, ldw, alpha, s, inv_s, amax_w, wq, w_scale
 *                   as sq_prepare_weights;
 *   x, xt, M, ldx, g, xq, x_scale   as sq_quant_act (x is [M, K]);
 *   ws              workspace of sq_workspace_size(SQ_OP_PREPARE_AND_QUANT_ACT,
 *                   M, N, K, g) bytes, 16-byte aligned: the workspace of
 *                   sq_prepare_weights, then (rounded to 256 bytes) that of
 *                   sq_quant_act.
 */
sq_status sq_prepare_and_quant_act(const float *amax_x, const void *w, sq_dtype wt, int64_t K, int64_t N,
                                   int64_t ldw, float alpha, float *s, float *inv_s, float *amax_w, int8_t *wq,
                                   float *w_scale, const void *x, sq_dtype xt, int64_t M, int64_t ldx,
                                   sq_act_gran g, int8_t *xq, float *x_scale, void *ws, size_t ws_bytes,
                                   hipStream_t stream);

/*
 * LayerNorm fold (page "4.2 W8A8 量化与 SmoothQuant" section 6: the factor
 * 1/s_j folds into the LayerNorm in front of the layer,
 * LN(x)_j / s_j = (x_j - mu) / sigma * gamma_j / s_j + beta_j / s_j, so the
 * runtime needs no separate smoothing multiply).
 *
 * sq_fold_layernorm: offline, gamma_out[j] = fl(gamma[j] * inv_s[j]) and
 *   beta_out[j] = fl(beta[j] * inv_s[j]) (beta may be NULL: no bias, beta_out
 *   unused).  All [K] fp32 device vectors; outputs may alias the inputs.
 * sq_layernorm_quant: at run time, LayerNorm of each bf16 token row of
 *   x [M, K] with the folded gamma/beta, then per-token INT8 codes (step 4
 *   with the smoothing already inside gamma/beta).  The page gives the
 *   formula, not its arithmetic; the library computes, per row:
 *     A = max_j |x_j|, with 2^(E-1) <= A < 2^E (E = 0 when A = 0);
 *     S1 = sum_j trunc(x_j * 2^(39-E)) and S2 = sum_j trunc(x_j^2 * 2^(39-2E))
 *       (truncation toward zero; integers below 2^39, summed exactly, so the
 *       statistics do not depend on the order of summation);
 *     mu = S1 * 2^(E-39) / K and var = max(S2 * 2^(2E-39) / K - mu^2, 0),
 *       each in fp64 with single roundings (mu = var = 0 when A = 0);
 *     mu32 = (float)mu, rstd32 = (float)(1 / sqrt(var + (double)eps))
 *       (fp64 sqrt and divide, then one rounding to fp32);
 *     n_j = fl(fl(x_j - mu32) * rstd32), z_j = fl(fl(n_j * gamma_j) + beta_j)
 *       (z_j = fl(n_j * gamma_j) when beta is NULL);
 *     m_i = max_j |z_j|, x_scale[i] = fl(m_i / 127) and
 *       codes clamp(rne(fl(z_j * fl(127 / m_i))), -127, 127) (0 when m_i = 0).
 *   The truncation moves mu by less than 2^(E-39) and the mean square by less
 *   than 2^(2E-39) from the exact row statistics (biased variance, eps inside
 *   the root).  x: bf16 only (SQ_ERR_UNSUPPORTED otherwise), 16-byte aligned
 *   rows; K <= 16384; eps >= 0; gamma (and beta) 16-byte aligned; xq [M, K]
 *   and x_scale [M] as sq_quant_act per token.
 */
sq_status sq_fold_layernorm(const float *gamma, const float *beta, const float *inv_s, int64_t K, float *gamma_out,
                            float *beta_out, hipStream_t stream);
sq_status sq_layernorm_quant(const void *x, sq_dtype xt, int64_t M, int64_t K, int64_t ldx, const float *gamma,
                             const float *beta, float eps, int8_t *xq, float *x_scale, hipStream_t stream);

/*
 * Static per-tensor activation scale (page "4.2 W8A8 量化与 SmoothQuant"
 * section 7.1, export step: activation scales may come from the calibration
 * statistics instead of being computed at run time).
 *
 * sq_static_act_max: a_static[0] = max_j fl(amax_x[j] * inv_s[j]), the
 *   largest |X'| over the calibration tokens (amax_x from step 1, inv_s from
 *   step 2, or NULL for unsmoothed activations).  K may be 0 (a = 0).
 * sq_quant_act_static: step 4 with that fixed maximum: x_scale[0] =
 *   fl(a/127), codes clamp(rne(fl(fl(x * inv_s_j) * fl(127/a))), -127, 127).
 *   Run-time values beyond the calibrated range saturate at +-127; no
 *   reduction over X runs, so the call is one pass and needs no workspace.
 *   x, inv_s, xq as sq_quant_act; a_static is a device pointer to one float
 *   (a >= 0).  The GEMM then takes x_scale with SQ_PER_TENSOR.
 */
sq_status sq_static_act_max(const float *amax_x, const float *inv_s, int64_t K, float *a_static,
                            hipStream_t stream);
sq_status sq_quant_act_static(const void *x, sq_dtype xt, int64_t M, int64_t K, int64_t ldx, const float *inv_s,
                              const float *a_static, int8_t *xq, float *x_scale, hipStream_t stream);

/*
 * Step 5 -- INT8 GEMM with int32 accumulation and the dequantization epilogue
 * (page "4.2 W8A8 量化与 SmoothQuant" section 6: the runtime kernel is a plain
 * INT8 GEMM; page "量化：只压权重..." SmoothQuant W8A8: the activation scale
 * must be constant along the reduction so it can be applied after the GEMM;
 * page "GBDQ权重与平滑激活量化": the product is dequantized to BF16).
 *
 *   xq, x_scale, g  from step 4 (xq [M, K] dense).
 *   wq, w_scale     from step 3 (wq [N, K] dense).
 *                   Steps 3 and 4 write codes in [-127, 127].  Codes of -128
 *                   from elsewhere are multiplied as they are; the int32 sum
 *                   is then still exact except at K = 131072 with every
 *                   product equal to 128 * 128, whose sum 2^31 does not fit
 *                   int32 (the result is then undefined).
 *   y               [M, N] out, dense, dtype yt: SQ_BF16 (the deployed output)
 *                   or SQ_F32 (the fp32 value before the bf16 rounding).
 *   acc_out         [M, N] int32 out, or NULL: the exact accumulators (for
 *                   verification; costs an extra 4 bytes per output).
 *   ws              workspace of sq_workspace_size(SQ_OP_GEMM_W8A8, M, N, K, g)
 *                   bytes (may be 0).
 */
sq_status sq_gemm_w8a8(const int8_t *xq, const float *x_scale, sq_act_gran g, const int8_t *wq,
                       const float *w_scale, int64_t M, int64_t N, int64_t K, void *y, sq_dtype yt,
                       int32_t *acc_out, void *ws, size_t ws_bytes, hipStream_t stream);

/*
 * LLM.int8()-style mixed-precision product, the route the pages set
 * SmoothQuant against (page "4.2 W8A8 量化与 SmoothQuant" section 2; page
 * "量化：只压权重，与训练后量化（PTQ）", SmoothQuant W8A8 results paragraph,
 * which gives the threshold 6): the input channels whose activation magnitude
 * exceeds a threshold are taken out of the INT8 product and multiplied in
 * 16 bits, and the two results are added.  Provided as a comparator on the
 * same data.  One runtime pass (the outlier count never leaves the device):
 *   sq_calib_absmax(x)        amax_x of the activation being multiplied
 *                             (amax zeroed first)
 *   sq_outlier_columns        idx, count, keep
 *   sq_quant_act(x, inv_s = keep, SQ_PER_TOKEN)
 *                             xq (0 on outlier channels), x_scale over the
 *                             regular channels
 *   sq_gather_outliers        x_o, w_ot
 *   sq_gemm_w8a8_outlier      y
 * with the weight codes of W itself (sq_quant_weight with s = NULL), made
 * once offline.
 *
 * sq_outlier_columns: amax_x [K] in.  idx [K] int32 out: the channels with
 *   amax_x[j] > threshold (strictly), ascending, in idx[0 .. *count).
 *   count: one int32 out.  keep [K] fp32 out (16-byte aligned): 0 on outlier
 *   channels, 1 elsewhere (fl(x * 1) = x and fl(x * 0) = 0 for finite x, so
 *   sq_quant_act with inv_s = keep quantizes only the regular channels).
 *   threshold must not be NaN.  One workgroup; K as everywhere (K % 16 == 0).
 * sq_gather_outliers: x [M, K] (ldx) and w [K, N] (ldw), both bf16 (else
 *   SQ_ERR_UNSUPPORTED; element alignment suffices); idx, count from
 *   sq_outlier_columns.  kp: row stride of the outputs, a multiple of 16 and at
 *   least K rounded up to 16 (room for every channel).  x_o [M, kp] and
 *   w_ot [N, kp] bf16 out, 16-byte aligned: x_o[i, t] = x[i, idx[t]] and
 *   w_ot[k, t] = w[idx[t], k] for t < count, 0 from count up to the next
 *   multiple of 16; entries beyond are not written.
 * sq_gemm_w8a8_outlier: the product of sq_gemm_w8a8 with a per-token x_scale
 *   (y8 = fl(fl(float(acc) * x_scale_i) * w_scale_k)) plus
 *   y16[m, n] = sum over t < count of x_o[m, t] * w_ot[n, t]: bf16 products,
 *   exact in fp32, summed in fp32 by the bf16 matrix cores (v_mfma 32x32x16,
 *   in the hardware's order of addition, so y16 is within
 *   count * 2^-23 * sum_t |x_o[m, t] w_ot[n, t]| of the exact sum, not bit
 *   defined); y = fl(y8 + y16), stored as bf16 (round to nearest even) or fp32
 *   per yt.  Arguments as sq_gemm_w8a8, plus x_o, w_ot, kp, count from the
 *   calls above.  M <= 16 runs the tile kernels too (the weight-streaming
 *   decode kernels have no 16-bit half).
 */
sq_status sq_outlier_columns(const float *amax_x, int64_t K, float threshold, int32_t *idx, int32_t *count,
                             float *keep, hipStream_t stream);
sq_status sq_gather_outliers(const void *x, sq_dtype xt, int64_t M, int64_t K, int64_t ldx, const void *w,
                             sq_dtype wt, int64_t N, int64_t ldw, const int32_t *idx, const int32_t *count,
                             int64_t kp, void *x_o, void *w_ot, hipStream_t stream);
sq_status sq_gemm_w8a8_outlier(const int8_t *xq, const float *x_scale, const int8_t *wq, const float *w_scale,
                               int64_t M, int64_t N, int64_t K, const void *x_o, const void *w_ot, int64_t kp,
                               const int32_t *count, void *y, sq_dtype yt, hipStream_t stream);

/*
 * Criterion of the offline migration-strength search (page "4.2 W8A8 量化与
 * SmoothQuant" section 5.2: a one-time grid search over alpha on calibration
 * data; section 4 of the same page: 0.5 is the usual value, up to 0.75 for
 * models with severe activation outliers).  The pages score each alpha by
 * validation perplexity; without a model, the layer-level reading scores it by
 * the error of the quantized layer's output: for each alpha the caller runs
 * steps 2-5 with an fp32 y and compares it with the same product in fp64:
 *
 * sq_matmul_f64: y_ref[m, n] = sum_k x[m, k] w[k, n], every product and sum
 *   in fp64 (bf16 and fp32 inputs widen exactly; the order of the sum over k
 *   is ascending within chunks of 16 and the chunks ascending, so y_ref is
 *   within K * 2^-53 * sum_k |x w| of the exact sum).  x [M, K] row-major,
 *   dtype xt, row stride ldx; w [K, N] row-major, dtype wt, row stride ldw
 *   (element alignment suffices for both); y_ref [M, N] fp64 out, dense,
 *   8-byte aligned, owned by the caller.  K % 16 == 0 as everywhere;
 *   N <= 65535 * 128.  Plain CUDA-core fp64 FMAs: an offline helper, not part
 *   of the runtime path.
 * sq_rel_error: err[0] = ||y - y_ref||_F / ||y_ref||_F in fp64 over the M * N
 *   elements of y [M, N] fp32 (dense, 4-byte aligned) and y_ref [M, N] fp64
 *   (dense, 8-byte aligned).  err: one fp64 out, device memory.  ws: device
 *   workspace of sq_workspace_size(SQ_OP_REL_ERROR, M, N, 0, 0) bytes, 8-byte
 *   aligned, scratch.  The partial sums are added in a fixed order, so the
 *   result does not depend on scheduling.  A y_ref of all zeros gives the
 *   quotient's IEEE value (NaN or infinity); M * N == 0 gives NaN.
 */
sq_status sq_matmul_f64(const void *x, sq_dtype xt, int64_t M, int64_t K, int64_t ldx, const void *w,
                        sq_dtype wt, int64_t N, int64_t ldw, double *y_ref, hipStream_t stream);
sq_status sq_rel_error(const float *y, const double *y_ref, int64_t M, int64_t N, double *err, void *ws,
                       size_t ws_bytes, hipStream_t stream);

/* Bytes of device workspace the call `op` needs for these sizes (0 if none).
 * Sizes the call does not use are ignored. */
size_t sq_workspace_size(sq_op op, int64_t M, int64_t N, int64_t K, sq_act_gran g);

/* Static English name of a status code. */
const char *sq_status_str(sq_status status);

/* Message of the last failed call on this host thread ("" if none).  Valid
 * until the next library call on the same thread. */
const char *sq_last_error(void);

/* Library version, "major.minor.patch". */
const char *sq_version(void);

/* Static description of the kernel sq_gemm_w8a8 launches for an M x N x K
 * product (tile shape and wavefront layout), for profiling and reports.
 * Host function: enqueues nothing; it may query the current device's compute
 * unit count (the decode kernel's grid depends on it).  Never fails. */
const char *sq_gemm_kernel_name(int64_t M, int64_t N, int64_t K);
/* The same for sq_gemm_w8a8_outlier. */
const char *sq_gemm_outlier_kernel_name(int64_t M, int64_t N, int64_t K);

#ifdef __cplusplus
}
#endif

#endif /* SQ_H */
