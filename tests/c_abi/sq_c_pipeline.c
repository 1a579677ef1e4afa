/*
 * The five steps through the C ABI alone (no Python, no torch): plain device
 * buffers from hipMalloc, every call of include/sq.h, results copied back and
 * compared bit for bit with the CPU oracle's C functions on the same inputs.
 *
 * Test infrastructure: links libsq.so (the product) and liboracle.so (the
 * checker); neither library knows the other.
 *
 *   sq_c_pipeline host   argument checks and utilities only (no GPU call)
 *   sq_c_pipeline gpu    the five steps on device 0 against the oracle
 *
 * Exit status 0 on success; the first failure is printed.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "sq.h"

/* the oracle's entry points (oracle/sq_oracle.c) */
int sqo_calib_absmax(const void *x, int dtype, int64_t T, int64_t K, int64_t ldx, float *amax);
int sqo_weight_rowmax(const void *w, int dtype, int64_t K, int64_t N, int64_t ldw, float *amax_w);
int sqo_smooth_factors(const float *amax_x, const float *amax_w, int64_t K, float alpha, float *s,
                       float *inv_s);
int sqo_quant_weight(const void *w, int dtype, int64_t K, int64_t N, int64_t ldw, const float *s, int8_t *wq,
                     int64_t ldq, float *w_scale);
int sqo_quant_act(const void *x, int dtype, int64_t M, int64_t K, int64_t ldx, const float *inv_s, int gran,
                  int8_t *xq, int64_t ldq, float *x_scale);
int sqo_gemm_i8(const int8_t *xq, int64_t ldx, const int8_t *wq, int64_t ldw, int64_t M, int64_t N, int64_t K,
                int32_t *acc, int64_t ldc, int nthreads);
int sqo_dequant(const int32_t *acc, int64_t ldc, const float *x_scale, int gran, const float *w_scale, int64_t M,
                int64_t N, float *y32, uint16_t *ybf16, int64_t ldy);

#define FAIL(...)                             \
    do {                                      \
        fprintf(stderr, "FAIL: " __VA_ARGS__); \
        fprintf(stderr, "\n");                \
        exit(1);                              \
    } while (0)
#define HIP(call)                                                                         \
    do {                                                                                  \
        hipError_t e_ = (call);                                                           \
        if (e_ != hipSuccess) FAIL("%s: %s", #call, hipGetErrorString(e_));               \
    } while (0)
#define SQ(call)                                                                          \
    do {                                                                                  \
        sq_status st_ = (call);                                                           \
        if (st_ != SQ_OK) FAIL("%s: %s (%s)", #call, sq_status_str(st_), sq_last_error()); \
    } while (0)

/* ---- seeded inputs: a 64-bit LCG, Box-Muller normals, fp32 -> bf16 (nearest even) ---- */

static uint64_t rng_state;
static double uniform01(void) {
    rng_state = rng_state * 6364136223846793005ull + 1442695040888963407ull;
    return ((double)(rng_state >> 11) + 0.5) / 9007199254740992.0;
}
static float normal(void) {
    const double u = uniform01(), v = uniform01();
    return (float)(sqrt(-2.0 * log(u)) * cos(6.283185307179586 * v));
}
static uint16_t to_bf16(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}
/* rows x cols bf16, N(0, sd^2), channels j % every == 3 scaled by `outlier` */
static uint16_t *make_bf16(int64_t rows, int64_t cols, float sd, int every, float outlier) {
    uint16_t *p = (uint16_t *)malloc((size_t)(rows * cols) * 2);
    for (int64_t i = 0; i < rows * cols; ++i) {
        const int64_t j = i % cols;
        float v = normal() * sd;
        if (every > 0 && j % every == 3) v *= outlier;
        p[i] = to_bf16(v);
    }
    return p;
}

static void *dev_copy(const void *h, size_t bytes) {
    void *d = NULL;
    HIP(hipMalloc(&d, bytes ? bytes : 16));
    if (bytes) HIP(hipMemcpy(d, h, bytes, hipMemcpyHostToDevice));
    return d;
}
static void *dev_alloc(size_t bytes) {
    void *d = NULL;
    HIP(hipMalloc(&d, bytes ? bytes : 16));
    return d;
}
static void same(const char *what, const void *dev, const void *host, size_t bytes) {
    void *h = malloc(bytes);
    HIP(hipMemcpy(h, dev, bytes, hipMemcpyDeviceToHost));
    if (memcmp(h, host, bytes) != 0) {
        size_t i = 0;
        while (((const unsigned char *)h)[i] == ((const unsigned char *)host)[i]) ++i;
        FAIL("%s differs from the oracle (first differing byte %zu of %zu)", what, i, bytes);
    }
    free(h);
}

static int host_checks(void) {
    printf("libsq %s\n", sq_version());
    if (strcmp(sq_status_str(SQ_ERR_WORKSPACE), "SQ_ERR_WORKSPACE") != 0) FAIL("sq_status_str");
    if (sq_workspace_size(SQ_OP_QUANT_WEIGHT, 0, 4096, 4096, SQ_PER_TOKEN) < 4096 * 4) FAIL("workspace size");
    if (sq_workspace_size(SQ_OP_REL_ERROR, 8, 24, 0, SQ_PER_TOKEN) == 0) FAIL("rel_error workspace size");
    /* rejected before any device work: fake pointers are never dereferenced */
    void *fake = (void *)(uintptr_t)0x10000;
    if (sq_calib_absmax(fake, SQ_BF16, 8, 20, 20, (float *)fake, NULL) != SQ_ERR_INVALID_ARG ||
        !strstr(sq_last_error(), "multiple of 16"))
        FAIL("K = 20 accepted (%s)", sq_last_error());
    if (sq_gemm_w8a8((const int8_t *)fake, (const float *)fake, SQ_PER_TOKEN, (const int8_t *)fake,
                     (const float *)fake, 4, 8, 32, NULL, SQ_BF16, NULL, NULL, 0, NULL) != SQ_ERR_INVALID_ARG)
        FAIL("NULL y accepted");
    if (sq_quant_weight(fake, SQ_BF16, 32, 64, 64, NULL, (int8_t *)fake, (float *)fake, fake, 4, NULL) !=
        SQ_ERR_WORKSPACE)
        FAIL("short workspace accepted (%s)", sq_last_error());
    printf("host checks ok\n");
    return 0;
}

/* one pass of the five steps at (M, K, N, T, alpha, gran) against the oracle */
static void pipeline_case(int64_t M, int64_t K, int64_t N, int64_t T, float alpha, sq_act_gran gran) {
    printf("case M=%lld K=%lld N=%lld T=%lld alpha=%g %s\n", (long long)M, (long long)K, (long long)N, (long long)T,
           alpha, gran == SQ_PER_TOKEN ? "per-token" : "per-tensor");
    fflush(stdout);
    uint16_t *x = make_bf16(M, K, 1.0f, 37, 60.0f);
    uint16_t *calib = make_bf16(T, K, 1.0f, 37, 60.0f);
    uint16_t *w = make_bf16(K, N, 0.02f, 0, 1.0f);
    const int64_t ns = gran == SQ_PER_TOKEN ? M : 1;

    /* the library, on device buffers */
    void *d_x = dev_copy(x, (size_t)(M * K) * 2), *d_calib = dev_copy(calib, (size_t)(T * K) * 2);
    void *d_w = dev_copy(w, (size_t)(K * N) * 2);
    float *d_amax = (float *)dev_alloc((size_t)K * 4), *d_s = (float *)dev_alloc((size_t)K * 4);
    float *d_inv_s = (float *)dev_alloc((size_t)K * 4), *d_amax_w = (float *)dev_alloc((size_t)K * 4);
    int8_t *d_wq = (int8_t *)dev_alloc((size_t)(N * K)), *d_xq = (int8_t *)dev_alloc((size_t)(M * K));
    float *d_ws = (float *)dev_alloc((size_t)N * 4), *d_xs = (float *)dev_alloc((size_t)ns * 4);
    uint16_t *d_y = (uint16_t *)dev_alloc((size_t)(M * N) * 2);
    int32_t *d_acc = (int32_t *)dev_alloc((size_t)(M * N) * 4);
    const size_t nw = sq_workspace_size(SQ_OP_QUANT_WEIGHT, M, N, K, gran);
    const size_t na = sq_workspace_size(SQ_OP_QUANT_ACT, M, N, K, gran);
    const size_t ng = sq_workspace_size(SQ_OP_GEMM_W8A8, M, N, K, gran);
    void *d_wkw = dev_alloc(nw), *d_wka = dev_alloc(na), *d_wkg = dev_alloc(ng);

    SQ(sq_calib_reset(d_amax, K, NULL));
    SQ(sq_calib_absmax(d_calib, SQ_BF16, T, K, K, d_amax, NULL));
    SQ(sq_smooth_factors(d_amax, d_w, SQ_BF16, K, N, N, alpha, d_s, d_inv_s, d_amax_w, NULL));
    SQ(sq_quant_weight(d_w, SQ_BF16, K, N, N, d_s, d_wq, d_ws, d_wkw, nw, NULL));
    SQ(sq_quant_act(d_x, SQ_BF16, M, K, K, d_inv_s, gran, d_xq, d_xs, d_wka, na, NULL));
    SQ(sq_gemm_w8a8(d_xq, d_xs, gran, d_wq, d_ws, M, N, K, d_y, SQ_BF16, d_acc, d_wkg, ng, NULL));
    HIP(hipDeviceSynchronize());

    /* the oracle, on the same host inputs */
    float *amax = (float *)calloc((size_t)K, 4), *amax_w = (float *)malloc((size_t)K * 4);
    float *s = (float *)malloc((size_t)K * 4), *inv_s = (float *)malloc((size_t)K * 4);
    int8_t *wq = (int8_t *)malloc((size_t)(N * K)), *xq = (int8_t *)malloc((size_t)(M * K));
    float *ws = (float *)malloc((size_t)N * 4), *xs = (float *)malloc((size_t)ns * 4);
    int32_t *acc = (int32_t *)malloc((size_t)(M * N) * 4);
    float *y32 = (float *)malloc((size_t)(M * N) * 4);
    uint16_t *y = (uint16_t *)malloc((size_t)(M * N) * 2);
    if (sqo_calib_absmax(calib, 1, T, K, K, amax) || sqo_weight_rowmax(w, 1, K, N, N, amax_w) ||
        sqo_smooth_factors(amax, amax_w, K, alpha, s, inv_s) ||
        sqo_quant_weight(w, 1, K, N, N, s, wq, K, ws) ||
        sqo_quant_act(x, 1, M, K, K, inv_s, gran == SQ_PER_TOKEN ? 0 : 1, xq, K, xs) ||
        sqo_gemm_i8(xq, K, wq, K, M, N, K, acc, N, 8) ||
        sqo_dequant(acc, N, xs, gran == SQ_PER_TOKEN ? 0 : 1, ws, M, N, y32, y, N))
        FAIL("the oracle rejected its arguments");

    same("amax_x", d_amax, amax, (size_t)K * 4);
    same("amax_w", d_amax_w, amax_w, (size_t)K * 4);
    same("s", d_s, s, (size_t)K * 4);
    same("inv_s", d_inv_s, inv_s, (size_t)K * 4);
    same("wq", d_wq, wq, (size_t)(N * K));
    same("w_scale", d_ws, ws, (size_t)N * 4);
    same("xq", d_xq, xq, (size_t)(M * K));
    same("x_scale", d_xs, xs, (size_t)ns * 4);
    same("acc", d_acc, acc, (size_t)(M * N) * 4);
    same("y (bf16)", d_y, y, (size_t)(M * N) * 2);

    void *dev[] = {d_x, d_calib, d_w, d_amax, d_s, d_inv_s, d_amax_w, d_wq, d_xq, d_ws, d_xs, d_y, d_acc,
                   d_wkw, d_wka, d_wkg};
    for (size_t i = 0; i < sizeof(dev) / sizeof(dev[0]); ++i) HIP(hipFree(dev[i]));
    void *host[] = {x, calib, w, amax, amax_w, s, inv_s, wq, xq, ws, xs, acc, y32, y};
    for (size_t i = 0; i < sizeof(host) / sizeof(host[0]); ++i) free(host[i]);
    printf("  bit-exact\n");
}

int main(int argc, char **argv) {
    if (argc < 2) FAIL("usage: %s host|gpu", argv[0]);
    rng_state = 20261203u;
    if (strcmp(argv[1], "host") == 0) return host_checks();
    if (strcmp(argv[1], "gpu") != 0) FAIL("unknown mode %s", argv[1]);
    HIP(hipSetDevice(0));
    pipeline_case(300, 512, 392, 777, 0.5f, SQ_PER_TOKEN);   /* ragged M and N, two calibration chunks' worth */
    pipeline_case(64, 1024, 256, 64, 0.75f, SQ_PER_TENSOR);  /* general alpha, one scale for the tensor */
    pipeline_case(2100, 4096, 3000, 4096, 0.4f, SQ_PER_TOKEN);  /* several tiles of the 256-row GEMMs */
    printf("c pipeline ok\n");
    return 0;
}
