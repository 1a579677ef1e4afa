/*
 * CPU oracle for the SmoothQuant W8A8 linear layer.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the plain, slow, obviously correct
 * statement of what the GPU library must compute.  Only the test suite, the
 * smoke check and the CPU-baseline leg of the benchmark load it.  It shares no
 * code, header, table or helper with the HIP library and includes nothing from
 * it.
 *
 * Build: gcc -O2 -ffp-contract=off -fno-fast-math -fPIC -shared -pthread.
 * Contraction is off so every fp32 product below is rounded once, in the order
 * written; the default rounding mode (round to nearest, ties to even) is kept.
 *
 * Notation follows the pages: Y = X W with X[M,K] (tokens x input channels)
 * and W[K,N] (input channel j = row j, output channel k = column k).
 *
 * Sources (page title, section):
 *  [P1] "大模型训练、适配与推理", section 3.5 (SmoothQuant): the equivalence
 *       X' = X diag(s)^-1, W' = diag(s) W and the alpha-weighted scale formula.
 *  [P2] "SmoothQuant大模型平滑量化技术", sections on the scale derivation and the
 *       Python demo: absmax over each channel, symmetric INT8 with scale
 *       max|.|/127, numpy rounding (half to even) and clipping to [-127, 127].
 *  [P3] "4.2 W8A8 量化与 SmoothQuant", section 4 (the formula and its alpha = 0
 *       and alpha = 1 limits), section 7.1 (calibration flow: per-channel
 *       activation maxima, static per-channel weights, per-token dynamic
 *       activation scales).
 *  [P4] "量化：只压权重，与训练后量化（PTQ）", section on SmoothQuant W8A8 and
 *       its worked 3x3 example (per-tensor / per-token activations, per-channel
 *       weights, relative output error).
 *  [P5] "GBDQ权重与平滑激活量化", outlier-visualisation section: the 4-bit
 *       symmetric scale max/7.
 *
 * Readings taken where the pages leave a step open (each is also listed with
 * its reason in the design notes of the repository):
 *  - both maxima are floored at 1e-5f before the scale formula (the pages
 *    mention a stability term without giving it);
 *  - the scale is evaluated in fp64 and rounded once to fp32; exponents 0,
 *    1/2 and 1 use the exact forms 1, sqrt and identity;
 *  - division by a scale is realised as a multiply by its fp32 reciprocal:
 *    x' = fl(x * fl(1/s)), code = rne(fl(x' * fl(127/a)));
 *  - weights are quantized per output channel (column k of W');
 *  - all-zero rows/columns get scale 0 and codes 0.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { SQO_F32 = 0, SQO_BF16 = 1 };
enum { SQO_PER_TOKEN = 0, SQO_PER_TENSOR = 1 };

/* ---- element access ---------------------------------------------------- */

/* A bf16 value is the upper half of the fp32 with the same sign, exponent
 * and leading 7 mantissa bits, so widening is a 16-bit shift (exact). */
static float bf16_bits_to_float(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

static float load_elem(const void *p, int dtype, int64_t idx)
{
    if (dtype == SQO_BF16)
        return bf16_bits_to_float(((const uint16_t *)p)[idx]);
    return ((const float *)p)[idx];
}

/* fp32 -> bf16 with round to nearest, ties to even, on the 16 bits that are
 * dropped.  Adding 0x7FFF plus the lowest kept bit carries into the kept part
 * exactly when the dropped part is above one half, or equal to one half with
 * an odd kept part.  NaN keeps a quiet NaN. */
uint16_t sqo_float_to_bf16(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu) != 0)
        return (uint16_t)((u >> 16) | 0x0040u);
    uint32_t keep_lsb = (u >> 16) & 1u;
    u += 0x7FFFu + keep_lsb;
    return (uint16_t)(u >> 16);
}

void sqo_floats_to_bf16(const float *x, int64_t n, uint16_t *out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = sqo_float_to_bf16(x[i]);
}

/* ---- symmetric absmax quantizer ([P2] demo, [P5] 4-bit row) ------------- */

/* From the largest magnitude m of a group: scale = m / qmax (stored for the
 * dequantization) and the multiplier r = qmax / m applied to each element.
 * A group whose maximum is 0 gets scale 0 and multiplier 0, so its codes are 0. */
static void sym_scale(float m, float qmax, float *scale, float *r)
{
    *scale = m / qmax;
    *r = (m > 0.0f) ? qmax / m : 0.0f;
}

/* code = clip(round_half_even(v * r), -qmax, qmax).  When the group max m is
 * so small that qmax / m overflows to +inf (m below about 3.7e-37), v * r is
 * +-inf for v != 0 (clipped to +-qmax) and 0 * inf = NaN for v == 0, which is
 * taken as code 0. */
static int sym_code(float v, float r, float qmax)
{
    float t = rintf(v * r);
    if (t != t)
        t = 0.0f;
    if (t > qmax)
        t = qmax;
    if (t < -qmax)
        t = -qmax;
    return (int)t;
}

/* Generic symmetric quantizer of one group of n values to a signed code range
 * [-(2^(bits-1)-1), 2^(bits-1)-1].  Used for the 4-bit pin; the 8-bit paths
 * below use the same two helpers with qmax = 127. */
int sqo_quant_sym(const float *x, int64_t n, int bits, int8_t *codes, float *scale)
{
    if (bits < 2 || bits > 8 || n < 0)
        return -1;
    float qmax = (float)((1 << (bits - 1)) - 1);
    float m = 0.0f;
    for (int64_t i = 0; i < n; ++i) {
        float a = fabsf(x[i]);
        if (a > m)
            m = a;
    }
    float r;
    sym_scale(m, qmax, scale, &r);
    for (int64_t i = 0; i < n; ++i)
        codes[i] = (int8_t)sym_code(x[i], r, qmax);
    return 0;
}

/* ---- step 1: calibration absmax ([P3] 7.1, [P4] SmoothQuant W8A8) ------- */

/* Running per-input-channel maximum of |X| over calibration tokens:
 * amax[j] = max(amax[j], max_t |x[t, j]|).  The caller sets amax to 0 before
 * the first chunk; later chunks continue the same running maximum. */
int sqo_calib_absmax(const void *x, int dtype, int64_t T, int64_t K, int64_t ldx,
                     float *amax)
{
    if (T < 0 || K < 0 || ldx < K)
        return -1;
    for (int64_t t = 0; t < T; ++t)
        for (int64_t j = 0; j < K; ++j) {
            float a = fabsf(load_elem(x, dtype, t * ldx + j));
            if (a > amax[j])
                amax[j] = a;
        }
    return 0;
}

/* ---- step 2: weight row maxima and smoothing factors -------------------- */

/* amax_w[j] = max_k |W[j, k]|: row j of W is the row that multiplies input
 * channel j ([P4] defines W_j as the j-th row; [P1] takes the max over k). */
int sqo_weight_rowmax(const void *w, int dtype, int64_t K, int64_t N, int64_t ldw,
                      float *amax_w)
{
    if (K < 0 || N < 0 || ldw < N)
        return -1;
    for (int64_t j = 0; j < K; ++j) {
        float m = 0.0f;
        for (int64_t k = 0; k < N; ++k) {
            float a = fabsf(load_elem(w, dtype, j * ldw + k));
            if (a > m)
                m = a;
        }
        amax_w[j] = m;
    }
    return 0;
}

/* x^e in fp64 with the exact forms for the exponents the pages single out. */
static double pow_exact_cases(double x, double e)
{
    if (e == 0.0)
        return 1.0;
    if (e == 1.0)
        return x;
    if (e == 0.5)
        return sqrt(x);
    return pow(x, e);
}

/* s_j = max|X_j|^alpha / max|W_j|^(1 - alpha)  ([P1] 3.5, [P3] section 4,
 * [P4] SmoothQuant W8A8), evaluated in fp64 and rounded once to fp32;
 * inv_s_j = fl32(1 / s_j).  alpha = 0 gives 1/max|W_j|, alpha = 1 gives
 * max|X_j| ([P3] section 4). */
int sqo_smooth_factors(const float *amax_x, const float *amax_w, int64_t K, float alpha,
                       float *s, float *inv_s)
{
    if (K < 0 || !(alpha >= 0.0f && alpha <= 1.0f))
        return -1;
    const float floor_ = 1e-5f;
    double ea = (double)alpha;
    double eb = 1.0 - ea;
    for (int64_t j = 0; j < K; ++j) {
        float a = amax_x[j] > floor_ ? amax_x[j] : floor_;
        float b = amax_w[j] > floor_ ? amax_w[j] : floor_;
        double num = pow_exact_cases((double)a, ea);
        double den = pow_exact_cases((double)b, eb);
        float sj = (float)(num / den);
        s[j] = sj;
        inv_s[j] = 1.0f / sj;
    }
    return 0;
}

/* ---- step 3: smoothed weights, per-output-channel INT8 ------------------ */

/* W'[j, k] = fl(s_j * W[j, k]) ([P1] 3.5: the weight row j grows by s_j);
 * one symmetric scale per output channel k, i.e. per column of W' ([P3] 7.1
 * static per-channel weights; the column reading is the one that reproduces
 * [P4]'s printed errors).  Codes are written transposed, wq[k * ldq + j], so
 * each output channel's codes are contiguous along the reduction axis.
 * s == NULL quantizes W itself (the unsmoothed baseline). */
int sqo_quant_weight(const void *w, int dtype, int64_t K, int64_t N, int64_t ldw,
                     const float *s, int8_t *wq, int64_t ldq, float *w_scale)
{
    if (K < 0 || N < 0 || ldw < N || ldq < K)
        return -1;
    for (int64_t k = 0; k < N; ++k) {
        float m = 0.0f;
        for (int64_t j = 0; j < K; ++j) {
            float v = load_elem(w, dtype, j * ldw + k);
            float wp = s ? s[j] * v : v;
            float a = fabsf(wp);
            if (a > m)
                m = a;
        }
        float r;
        sym_scale(m, 127.0f, &w_scale[k], &r);
        for (int64_t j = 0; j < K; ++j) {
            float v = load_elem(w, dtype, j * ldw + k);
            float wp = s ? s[j] * v : v;
            wq[k * ldq + j] = (int8_t)sym_code(wp, r, 127.0f);
        }
    }
    return 0;
}

/* ---- step 4: smoothed activations, per-token / per-tensor INT8 ---------- */

/* X'[i, j] = fl(X[i, j] * inv_s_j) ([P1] 3.5: channel j shrinks by s_j).
 * Per token: one scale per row, from that row's max|X'| computed at run time
 * ([P3] 7.1, [P4] worked example).  Per tensor: one scale from the max over
 * the whole X' ([P3] 1.2, [P4] worked example).  inv_s == NULL quantizes X
 * itself.  x_scale has M entries (per token) or 1 (per tensor). */
int sqo_quant_act(const void *x, int dtype, int64_t M, int64_t K, int64_t ldx,
                  const float *inv_s, int gran, int8_t *xq, int64_t ldq, float *x_scale)
{
    if (M < 0 || K < 0 || ldx < K || ldq < K)
        return -1;
    if (gran != SQO_PER_TOKEN && gran != SQO_PER_TENSOR)
        return -1;
    float *row = (float *)malloc((size_t)(K > 0 ? K : 1) * sizeof(float));
    if (!row)
        return -2;
    float tensor_max = 0.0f;
    if (gran == SQO_PER_TENSOR) {
        for (int64_t i = 0; i < M; ++i)
            for (int64_t j = 0; j < K; ++j) {
                float v = load_elem(x, dtype, i * ldx + j);
                float a = fabsf(inv_s ? v * inv_s[j] : v);
                if (a > tensor_max)
                    tensor_max = a;
            }
    }
    float t_scale = 0.0f, t_r = 0.0f;
    if (gran == SQO_PER_TENSOR) {
        sym_scale(tensor_max, 127.0f, &t_scale, &t_r);
        x_scale[0] = t_scale;
    }
    for (int64_t i = 0; i < M; ++i) {
        float m = 0.0f;
        for (int64_t j = 0; j < K; ++j) {
            float v = load_elem(x, dtype, i * ldx + j);
            row[j] = inv_s ? v * inv_s[j] : v;
            float a = fabsf(row[j]);
            if (a > m)
                m = a;
        }
        float r = t_r;
        if (gran == SQO_PER_TOKEN)
            sym_scale(m, 127.0f, &x_scale[i], &r);
        for (int64_t j = 0; j < K; ++j)
            xq[i * ldq + j] = (int8_t)sym_code(row[j], r, 127.0f);
    }
    free(row);
    return 0;
}

/* ---- static per-tensor activation scale ([P3] 7.1 export step) ---------- */

/* The calibrated maximum of the smoothed activations: the largest |X'| =
 * |fl(x * inv_s_j)| over all calibration tokens t and channels j ([P3] 7.1:
 * activation scales may come from calibration statistics instead of being
 * computed at run time).  inv_s == NULL takes X itself. */
float sqo_static_act_max(const void *x, int dtype, int64_t T, int64_t K, int64_t ldx, const float *inv_s)
{
    float a = 0.0f;
    for (int64_t t = 0; t < T; ++t)
        for (int64_t j = 0; j < K; ++j) {
            float v = load_elem(x, dtype, t * ldx + j);
            float m = fabsf(inv_s ? v * inv_s[j] : v);
            if (m > a)
                a = m;
        }
    return a;
}

/* Per-tensor codes with that fixed maximum a: x_scale[0] = fl(a / 127) and
 * r = fl(127 / a) (0 if a = 0) as for a dynamic per-tensor scale, but a does
 * not depend on x, so run-time values beyond the calibrated range saturate
 * at +-127. */
int sqo_quant_act_static(const void *x, int dtype, int64_t M, int64_t K, int64_t ldx, const float *inv_s,
                         float a, int8_t *xq, int64_t ldq, float *x_scale)
{
    if (M < 0 || K < 0 || ldx < K || ldq < K || !(a >= 0.0f))
        return -1;
    float r;
    sym_scale(a, 127.0f, x_scale, &r);
    for (int64_t i = 0; i < M; ++i)
        for (int64_t j = 0; j < K; ++j) {
            float v = load_elem(x, dtype, i * ldx + j);
            xq[i * ldq + j] = (int8_t)sym_code(inv_s ? v * inv_s[j] : v, r, 127.0f);
        }
    return 0;
}

/* ---- LayerNorm fold ([P3] section 6) ------------------------------------ */

/* The smoothing folded into the LayerNorm in front of the linear layer:
 * LN(x)_j / s_j = (x_j - mu) / sigma * (gamma_j / s_j) + beta_j / s_j, so
 * gamma'_j = fl(gamma_j * inv_s_j) and beta'_j = fl(beta_j * inv_s_j) (division
 * by s_j realised as the multiply by inv_s_j, as everywhere else).  beta may
 * be NULL (no bias): beta_out is then left alone. */
int sqo_fold_layernorm(const float *gamma, const float *beta, const float *inv_s, int64_t K, float *gamma_out,
                       float *beta_out)
{
    if (K < 0 || !gamma || !inv_s || !gamma_out)
        return -1;
    for (int64_t j = 0; j < K; ++j) {
        gamma_out[j] = gamma[j] * inv_s[j];
        if (beta)
            beta_out[j] = beta[j] * inv_s[j];
    }
    return 0;
}

/* LayerNorm of one bf16 token row followed by per-token symmetric INT8 codes
 * (the runtime half of the fold: the row that reaches the GEMM is
 * LN(x) diag(s)^-1).  The pages give the LayerNorm formula but not its
 * arithmetic; the statistics are taken on a fixed-point grid so that they do
 * not depend on the order of summation: with 2^E the power of two just above
 * the row's largest magnitude (frexp), each x_j is truncated toward zero to a
 * multiple of 2^(E - 39) and each x_j^2 to a multiple of 2^(2E - 39), and the
 * integers are summed exactly (|sum| < K 2^39 <= 2^53 for K <= 16384, so the
 * sums are exact even in fp64):
 *   mu = S1 2^(E-39) / K,  var = max(S2 2^(2E-39) / K - mu^2, 0)  (biased),
 *   rstd = 1 / sqrt(var + eps), all in fp64 with single roundings; then
 * mu32 = (float)mu and rstd32 = (float)rstd.  Element j, in fp32 as a fp32
 * LayerNorm computes it: n_j = fl(fl(x_j - mu32) * rstd32),
 * z_j = fl(fl(n_j * gamma_j) + beta_j).  The row's codes and scale are those
 * of step 4 per token.  beta NULL: no bias term. */
int sqo_layernorm_quant(const uint16_t *x, int64_t M, int64_t K, int64_t ldx, const float *gamma,
                        const float *beta, float eps, int8_t *xq, int64_t ldq, float *x_scale)
{
    if (M < 0 || K <= 0 || K > 16384 || ldx < K || ldq < K || !gamma)
        return -1;
    float *z = (float *)malloc((size_t)K * sizeof(float));
    if (!z)
        return -2;
    for (int64_t i = 0; i < M; ++i) {
        const uint16_t *row = x + i * ldx;
        float xmax = 0.0f;
        for (int64_t j = 0; j < K; ++j) {
            float a = fabsf(bf16_bits_to_float(row[j]));
            if (a > xmax)
                xmax = a;
        }
        double mu = 0.0, var = 0.0;
        if (xmax > 0.0f) {
            int E;
            frexpf(xmax, &E);
            const double c1 = ldexp(1.0, 39 - E), c2 = ldexp(1.0, 39 - 2 * E);
            int64_t s1 = 0, s2 = 0;
            for (int64_t j = 0; j < K; ++j) {
                double v = (double)bf16_bits_to_float(row[j]);
                s1 += (int64_t)(v * c1);
                s2 += (int64_t)(v * v * c2);
            }
            mu = ldexp((double)s1, E - 39) / (double)K;
            var = ldexp((double)s2, 2 * E - 39) / (double)K - mu * mu;
            if (var < 0.0)
                var = 0.0;
        }
        const float mu32 = (float)mu, rstd32 = (float)(1.0 / sqrt(var + (double)eps));
        float m = 0.0f;
        for (int64_t j = 0; j < K; ++j) {
            float n = (bf16_bits_to_float(row[j]) - mu32) * rstd32;
            float t = n * gamma[j];
            z[j] = beta ? t + beta[j] : t;
            float a = fabsf(z[j]);
            if (a > m)
                m = a;
        }
        float r;
        sym_scale(m, 127.0f, &x_scale[i], &r);
        for (int64_t j = 0; j < K; ++j)
            xq[i * ldq + j] = (int8_t)sym_code(z[j], r, 127.0f);
    }
    free(z);
    return 0;
}

/* ---- step 5: INT8 x INT8 -> int32 GEMM and dequantization --------------- */

/* acc[i, k] = sum_j Xq[i, j] * Wq[k, j] in int32.  |acc| <= K * 127^2, which
 * stays below 2^31 for K up to 133,143, so the sum is exact in any order.
 * ([P3] section 6 and [P4]: the runtime is a standard INT8 GEMM.)  Rows are
 * split over threads; each output is one plain dot product. */
struct gemm_job {
    const int8_t *xq, *wq;
    int32_t *acc;
    int64_t i0, i1, N, K, ldx, ldw, ldc;
};

static void *gemm_rows(void *p)
{
    const struct gemm_job *g = (const struct gemm_job *)p;
    for (int64_t i = g->i0; i < g->i1; ++i) {
        const int8_t *xr = g->xq + i * g->ldx;
        for (int64_t k = 0; k < g->N; ++k) {
            const int8_t *wr = g->wq + k * g->ldw;
            int32_t sum = 0;
            for (int64_t j = 0; j < g->K; ++j)
                sum += (int32_t)xr[j] * (int32_t)wr[j];
            g->acc[i * g->ldc + k] = sum;
        }
    }
    return NULL;
}

int sqo_gemm_i8(const int8_t *xq, int64_t ldx, const int8_t *wq, int64_t ldw, int64_t M,
                int64_t N, int64_t K, int32_t *acc, int64_t ldc, int nthreads)
{
    if (M < 0 || N < 0 || K < 0 || ldx < K || ldw < K || ldc < N)
        return -1;
    if (nthreads < 1)
        nthreads = 1;
    if (nthreads > 256)
        nthreads = 256;
    if ((int64_t)nthreads > M)
        nthreads = M > 0 ? (int)M : 1;
    pthread_t tid[256];
    struct gemm_job jobs[256];
    int64_t per = (M + nthreads - 1) / nthreads;
    int started = 0;
    for (int t = 0; t < nthreads; ++t) {
        int64_t i0 = t * per, i1 = i0 + per < M ? i0 + per : M;
        jobs[t] = (struct gemm_job){xq, wq, acc, i0, i1 > i0 ? i1 : i0, N, K, ldx, ldw, ldc};
        if (nthreads == 1) {
            gemm_rows(&jobs[t]);
        } else if (pthread_create(&tid[t], NULL, gemm_rows, &jobs[t]) == 0) {
            ++started;
        } else {
            gemm_rows(&jobs[t]);
            tid[t] = 0;
        }
    }
    if (nthreads > 1)
        for (int t = 0; t < nthreads; ++t)
            if (tid[t])
                pthread_join(tid[t], NULL);
    (void)started;
    return 0;
}

/* y[i, k] = fl(fl(float(acc[i, k]) * x_scale_i) * w_scale_k): the per-token
 * activation scale is constant along the reduction, so it factors out of the
 * integer sum together with the per-output-channel weight scale ([P4]: a
 * per-input-channel activation scale could not).  The int -> fp32 conversion
 * rounds to nearest even.  y32 and/or ybf16 (bf16 bit patterns, round to
 * nearest even) may be NULL. */
int sqo_dequant(const int32_t *acc, int64_t ldc, const float *x_scale, int gran,
                const float *w_scale, int64_t M, int64_t N, float *y32, uint16_t *ybf16,
                int64_t ldy)
{
    if (M < 0 || N < 0 || ldc < N || ldy < N)
        return -1;
    for (int64_t i = 0; i < M; ++i) {
        float xs = gran == SQO_PER_TENSOR ? x_scale[0] : x_scale[i];
        for (int64_t k = 0; k < N; ++k) {
            float y = ((float)acc[i * ldc + k] * xs) * w_scale[k];
            if (y32)
                y32[i * ldy + k] = y;
            if (ybf16)
                ybf16[i * ldy + k] = sqo_float_to_bf16(y);
        }
    }
    return 0;
}

/* ---- LLM.int8()-style mixed-precision decomposition (comparator) --------- */

/* The earlier route the pages set SmoothQuant against ([P3] section 2, the
 * mixed-precision route; [P4] SmoothQuant W8A8, its results paragraph): the
 * input channels of X are split at run time.  Channel j is an outlier when
 * some |x[i, j]| of the activation being multiplied exceeds a threshold (the
 * pages give 6); outlier channels are multiplied in 16 bits, the others in
 * INT8, and the two products are added.
 *
 * Outlier selection from the per-channel maxima amax_x (of the whole X, as
 * step 1 computes them): idx receives the outlier channels in ascending
 * order, keep[j] = 0 for an outlier channel and 1 otherwise.  "Exceeds" is
 * read as strictly greater.  Returns the number of outlier channels, or -1. */
int sqo_outlier_columns(const float *amax_x, int64_t K, float threshold, int32_t *idx, float *keep)
{
    if (K < 0 || K > 2147483647LL)
        return -1;
    int32_t n = 0;
    for (int64_t j = 0; j < K; ++j) {
        int out = amax_x[j] > threshold;
        if (out)
            idx[n++] = (int32_t)j;
        if (keep)
            keep[j] = out ? 0.0f : 1.0f;
    }
    return n;
}

/* The decomposed product for the token rows x[0..R) (bf16 patterns, row
 * stride ldx) with a given outlier set idx[0..n_out) (ascending):
 *  - INT8 part: per token i, a_i = max over regular channels of |x[i, j]|,
 *    x_scale_i = fl(a_i / 127), codes rne(fl(x[i, j] * fl(127 / a_i))) clipped
 *    to +-127 on the regular channels and 0 on the outlier channels (they are
 *    taken out of this product); acc[i, k] = sum over regular j of
 *    xq[i, j] * wq[k, j] (exact), y8 = fl(fl(float(acc) * x_scale_i) * w_scale_k)
 *    with the offline per-output-channel weight codes wq, w_scale of W itself
 *    (no smoothing);
 *  - 16-bit part: the bf16 values as given, y16[i, k] = the sum over outlier
 *    j of x[i, j] * w[j, k], products exact, summed in fp64 and rounded once
 *    to fp32 (the pages fix no precision for this sum beyond 16-bit operands);
 *  - y = fl(y8 + y16), stored as fp32 (y32) and/or bf16 (ybf16, RNE).
 * bound (may be NULL) receives sum over outlier j of |x[i, j] * w[j, k]|, the
 * scale of the rounding error any fp32 evaluation of y16 may make.  xq
 * (may be NULL) receives the codes, x_scale the per-token scales. */
int sqo_llm_int8(const uint16_t *x, int64_t R, int64_t K, int64_t ldx, const uint16_t *w, int64_t N,
                 int64_t ldw, const int8_t *wq, const float *w_scale, const int32_t *idx, int64_t n_out,
                 int8_t *xq, float *x_scale, float *y32, uint16_t *ybf16, double *bound)
{
    if (R < 0 || K < 0 || N < 0 || ldx < K || ldw < N || n_out < 0 || n_out > K)
        return -1;
    for (int64_t t = 0; t < n_out; ++t)
        if (idx[t] < 0 || idx[t] >= K || (t > 0 && idx[t] <= idx[t - 1]))
            return -1;
    char *is_out = (char *)calloc((size_t)(K > 0 ? K : 1), 1);
    int8_t *codes = (int8_t *)malloc((size_t)(K > 0 ? K : 1));
    if (!is_out || !codes) {
        free(is_out);
        free(codes);
        return -2;
    }
    for (int64_t t = 0; t < n_out; ++t)
        is_out[idx[t]] = 1;
    for (int64_t i = 0; i < R; ++i) {
        const uint16_t *xr = x + i * ldx;
        float m = 0.0f;
        for (int64_t j = 0; j < K; ++j) {
            if (is_out[j])
                continue;
            float a = fabsf(bf16_bits_to_float(xr[j]));
            if (a > m)
                m = a;
        }
        float xs, r;
        sym_scale(m, 127.0f, &xs, &r);
        for (int64_t j = 0; j < K; ++j)
            codes[j] = is_out[j] ? 0 : (int8_t)sym_code(bf16_bits_to_float(xr[j]), r, 127.0f);
        if (xq)
            memcpy(xq + i * K, codes, (size_t)K);
        if (x_scale)
            x_scale[i] = xs;
        for (int64_t k = 0; k < N; ++k) {
            const int8_t *wr = wq + k * K;
            int32_t acc = 0;
            for (int64_t j = 0; j < K; ++j)
                if (!is_out[j])
                    acc += (int32_t)codes[j] * (int32_t)wr[j];
            float y8 = ((float)acc * xs) * w_scale[k];
            double s16 = 0.0, b16 = 0.0;
            for (int64_t t = 0; t < n_out; ++t) {
                int64_t j = idx[t];
                double p = (double)bf16_bits_to_float(xr[j]) * (double)bf16_bits_to_float(w[j * ldw + k]);
                s16 += p;
                b16 += fabs(p);
            }
            float y = y8 + (float)s16;
            if (y32)
                y32[i * N + k] = y;
            if (ybf16)
                ybf16[i * N + k] = sqo_float_to_bf16(y);
            if (bound)
                bound[i * N + k] = b16;
        }
    }
    free(is_out);
    free(codes);
    return 0;
}
