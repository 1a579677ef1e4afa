// The criterion of the offline migration-strength search (page "4.2 W8A8 量化与
// SmoothQuant" section 5.2: alpha chosen by a grid search on calibration data):
// the W8A8 output of a token sample against X W in fp64, by relative
// Frobenius error.  Neither kernel is on the runtime path; both keep the
// search inside the library.
#include "sq_device.h"
#include "sq_internal.h"

namespace sqk {

// y[m, n] = sum_k x[m, k] w[k, n] in fp64 (bf16 and fp32 inputs widen
// exactly).  Block tile 64 x 128 with 256 threads; a wavefront's 64 lanes
// are 8 row lanes x 8 column lanes over a 32 x 64 tile, each lane 4 rows x 8
// columns, so the lanes of a wavefront read only 8 distinct row slices of
// the X tile and 8 distinct column slices of the W tile per k from LDS
// (broadcast reads), and the fp64 FMAs set the pace.  k in chunks of 16,
// staged in LDS as fp64 (X transposed, [k][m]).  Elements past M or N read
// as zero and are not stored; K % 16 == 0.
constexpr int kF64BM = 64, kF64BN = 128, kF64KC = 16;
static_assert(kF64BN == 128, "kMatmulF64MaxN counts 128 columns per grid row");

template <typename TX, typename TW>
__global__ __launch_bounds__(256) void k_matmul_f64(const TX* __restrict__ x, int64_t M, int64_t K, int64_t ldx,
                                                    const TW* __restrict__ w, int64_t N, int64_t ldw,
                                                    double* __restrict__ y) {
    __shared__ double xs[kF64KC][kF64BM];
    __shared__ double wsh[kF64KC][kF64BN];
    const int t = threadIdx.x, wave = t / kWave, lane = t % kWave;
    // the row tiles of one column tile are consecutive blocks, so W's tile is
    // read from HBM once and then hit in L2
    const int64_t m0 = (int64_t)blockIdx.x * kF64BM, n0 = (int64_t)blockIdx.y * kF64BN;
    // wavefront (wm, wn) of 2 x 2 covers rows 32 wm .., columns 64 wn ..;
    // lane (lm, ln) of 8 x 8 its rows 4 lm .. 4 lm + 3, columns 8 ln .. 8 ln + 7
    const int wm = wave / 2, wn = wave % 2, lm = lane / 8, ln = lane % 8;
    const int rm = 32 * wm + 4 * lm, cn = 64 * wn + 8 * ln;
    double acc[4][8];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = 0.0;

    auto widen = [](auto v) -> double {
        if constexpr (sizeof(v) == 2) return (double)__uint_as_float((uint32_t)v.bits << 16);
        else return (double)v;
    };
    for (int64_t k0 = 0; k0 < K; k0 += kF64KC) {
        // X tile: 64 rows x 16 k, 4 consecutive k per thread
        {
            const int r = t / 4, kk = 4 * (t % 4);
            const int64_t m = m0 + r;
#pragma unroll
            for (int e = 0; e < 4; ++e) xs[kk + e][r] = m < M ? widen(x[m * ldx + k0 + kk + e]) : 0.0;
        }
        // W tile: 16 k x 128 columns, 8 consecutive columns per thread
        {
            const int kk = t / 16, c = 8 * (t % 16);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int64_t n = n0 + c + e;
                wsh[kk][c + e] = n < N ? widen(w[(k0 + kk) * ldw + n]) : 0.0;
            }
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < kF64KC; ++kk) {
            double a[4], b[8];
#pragma unroll
            for (int i = 0; i < 4; ++i) a[i] = xs[kk][rm + i];
#pragma unroll
            for (int j = 0; j < 8; ++j) b[j] = wsh[kk][cn + j];
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 8; ++j) acc[i][j] = fma(a[i], b[j], acc[i][j]);
        }
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int64_t m = m0 + rm + i;
        if (m >= M) continue;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int64_t n = n0 + cn + j;
            if (n < N) y[m * N + n] = acc[i][j];
        }
    }
}

hipError_t launch_matmul_f64(const void* x, bool x_bf16, int64_t M, int64_t K, int64_t ldx, const void* w,
                             bool w_bf16, int64_t N, int64_t ldw, double* y, hipStream_t st) {
    if (M <= 0 || N <= 0) return hipSuccess;
    const int64_t tn = (N + kF64BN - 1) / kF64BN, tm = (M + kF64BM - 1) / kF64BM;
    if (N > kMatmulF64MaxN || tm > 0x7FFFFFFF) return hipErrorInvalidValue;
    const dim3 grid((unsigned)tm, (unsigned)tn);
    auto go = [&](auto tx, auto tw) {
        using TX = decltype(tx);
        using TW = decltype(tw);
        hipLaunchKernelGGL((k_matmul_f64<TX, TW>), grid, dim3(256), 0, st, static_cast<const TX*>(x), M, K, ldx,
                           static_cast<const TW*>(w), N, ldw, y);
    };
    if (x_bf16) {
        if (w_bf16) go(bf16_t{}, bf16_t{});
        else go(bf16_t{}, float{});
    } else {
        if (w_bf16) go(float{}, bf16_t{});
        else go(float{}, float{});
    }
    return hipGetLastError();
}

// Relative Frobenius error ||y - y_ref||_F / ||y_ref||_F of y [M, N] fp32
// against y_ref [M, N] fp64, both dense.  Pass 1: kRelErrBlocks blocks walk
// the elements with a grid stride and write their two fp64 partial sums
// (sum (y - y_ref)^2, sum y_ref^2) to partial[2][kRelErrBlocks]; pass 2: one
// block adds the partials in a fixed order and divides, so the result does not
// depend on the order in which blocks finish.
constexpr int kRelErrBlocks = 512;

__device__ __forceinline__ double block_sum_f64(double v, double* red) {
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
    if (lane == 0) red[wave] = v;
    __syncthreads();
    double s = 0.0;
    if (threadIdx.x == 0)
        for (int i = 0; i < (int)(blockDim.x / kWave); ++i) s += red[i];
    __syncthreads();
    return s;  // valid in thread 0
}

__global__ __launch_bounds__(256) void k_rel_error_partials(const float* __restrict__ y,
                                                            const double* __restrict__ y_ref, int64_t n,
                                                            double* __restrict__ partial) {
    __shared__ double red[4];
    double e = 0.0, r = 0.0;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
        const double ref = y_ref[i];
        const double d = (double)y[i] - ref;
        e = fma(d, d, e);
        r = fma(ref, ref, r);
    }
    e = block_sum_f64(e, red);
    r = block_sum_f64(r, red);
    if (threadIdx.x == 0) {
        partial[blockIdx.x] = e;
        partial[kRelErrBlocks + blockIdx.x] = r;
    }
}

__global__ __launch_bounds__(256) void k_rel_error_final(const double* __restrict__ partial,
                                                         double* __restrict__ err) {
    __shared__ double red[4];
    double e = 0.0, r = 0.0;
    for (int i = threadIdx.x; i < kRelErrBlocks; i += 256) {
        e += partial[i];
        r += partial[kRelErrBlocks + i];
    }
    e = block_sum_f64(e, red);
    r = block_sum_f64(r, red);
    if (threadIdx.x == 0) err[0] = sqrt(e) / sqrt(r);
}

int64_t rel_error_workspace_bytes() { return 2 * kRelErrBlocks * (int64_t)sizeof(double); }

hipError_t launch_rel_error(const float* y, const double* y_ref, int64_t n, double* err, double* partial,
                            hipStream_t st) {
    hipLaunchKernelGGL(k_rel_error_partials, dim3(kRelErrBlocks), dim3(256), 0, st, y, y_ref, n, partial);
    hipLaunchKernelGGL(k_rel_error_final, dim3(1), dim3(256), 0, st, partial, err);
    return hipGetLastError();
}

}  // namespace sqk
