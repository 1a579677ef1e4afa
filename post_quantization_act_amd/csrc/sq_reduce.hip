// Reductions of the SmoothQuant path on gfx950: channel maxima and the
// smoothing factors.  All of them are HBM-bound streams over a matrix; the
// loads are 16-byte vectors along the contiguous axis and each wavefront
// covers whole 128-byte lines.
#include <type_traits>

#include "sq_device.h"
#include "sq_internal.h"

namespace sqk {

// out[i] = v for i < n (used to clear atomic-max targets without
// hipMemsetAsync, so the calls stay safe to capture in a HIP graph).
__global__ __launch_bounds__(256) void k_fill_u32(uint32_t* __restrict__ out, int64_t n, uint32_t v) {
    int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n) out[i] = v;
}

// Column max of |row_scale[r] * x[r, c]| (row_scale optional) over a block of
// rows, merged into out[c] by atomicMax on the fp32 bit pattern (non-negative
// floats order like their unsigned bit patterns).
//
// Block = 256 threads = 32 column lanes x 8 row lanes; a column lane owns 8
// consecutive columns (one 16-byte load for bf16), so a block spans 256
// columns and each wavefront reads 2 rows x 512 contiguous bytes per load.
// Row lanes stride over the block's rows; the 8 partial maxima per column are
// combined through LDS and each column then costs one atomic per block.
constexpr int kColLanes = 32;
constexpr int kRowLanes = 8;
constexpr int kColsPerBlock = kColLanes * 8;

template <typename T, bool kScaled, bool kVec>
__global__ __launch_bounds__(256) void k_col_absmax(const T* __restrict__ x, int64_t rows, int64_t cols,
                                                    int64_t ld, const float* __restrict__ row_scale,
                                                    uint32_t* __restrict__ out, int64_t rows_per_block) {
    const int cl = threadIdx.x % kColLanes;
    const int rl = threadIdx.x / kColLanes;
    const int64_t c0 = (int64_t)blockIdx.x * kColsPerBlock + cl * 8;
    const int64_t r_begin = (int64_t)blockIdx.y * rows_per_block;
    const int64_t r_end = min(rows, r_begin + rows_per_block);
    float m[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) m[i] = 0.0f;

    if (c0 < cols) {
        const int64_t ncol = cols - c0;
        const T* base = x + c0;
        int64_t r = r_begin + rl;
        constexpr int U = 4;
        for (; r + (U - 1) * kRowLanes < r_end; r += U * kRowLanes) {
            float v[U][8];
#pragma unroll
            for (int u = 0; u < U; ++u) load8_any<kVec>(base + (r + u * kRowLanes) * ld, ncol, v[u]);
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const float sc = kScaled ? row_scale[r + u * kRowLanes] : 1.0f;
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const float t = kScaled ? sc * v[u][i] : v[u][i];
                    m[i] = fmaxf(m[i], fabsf(t));
                }
            }
        }
        for (; r < r_end; r += kRowLanes) {
            float v[8];
            load8_any<kVec>(base + r * ld, ncol, v);
            const float sc = kScaled ? row_scale[r] : 1.0f;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float t = kScaled ? sc * v[i] : v[i];
                m[i] = fmaxf(m[i], fabsf(t));
            }
        }
    }

    __shared__ float red[kRowLanes][kColsPerBlock];
#pragma unroll
    for (int i = 0; i < 8; ++i) red[rl][cl * 8 + i] = m[i];
    __syncthreads();
    const int col = threadIdx.x;  // 256 threads, 256 columns
    float mm = 0.0f;
#pragma unroll
    for (int q = 0; q < kRowLanes; ++q) mm = fmaxf(mm, red[q][col]);
    const int64_t gc = (int64_t)blockIdx.x * kColsPerBlock + col;
    if (gc < cols && mm > 0.0f) atomicMax(out + gc, __float_as_uint(mm));
}

// x^e in fp64 with the exact forms for e = 0, 1/2, 1.
__device__ __forceinline__ double pow_cases(double x, double e) {
    if (e == 0.0) return 1.0;
    if (e == 1.0) return x;
    if (e == 0.5) return sqrt(x);
    return pow(x, e);
}

// s = a^alpha / b^(1-alpha) with both maxima floored at 1e-5f, in fp64 and
// rounded once; inv_s = correctly rounded fp32 reciprocal.
__device__ __forceinline__ void smooth_factor(float ax, float aw, float alpha, float& s, float& inv_s) {
    const float fl = 1e-5f;
    const float a = ax > fl ? ax : fl;
    const float b = aw > fl ? aw : fl;
    const double ea = (double)alpha;
    const double eb = 1.0 - ea;
    s = (float)(pow_cases((double)a, ea) / pow_cases((double)b, eb));
    inv_s = 1.0f / s;
}

// One wavefront per weight row j: amax_w[j] = max_k |W[j, k]|, then s_j and
// inv_s_j right away (the row max is the only per-row input the factor
// needs besides amax_x[j]).  Lanes stride along the row with 16-byte loads,
// 4 loads in flight per lane, and reduce with cross-lane shuffles.
template <typename T, bool kVec>
__global__ __launch_bounds__(256) void k_row_absmax_factors(const T* __restrict__ w, int64_t K, int64_t N,
                                                            int64_t ld, const float* __restrict__ amax_x,
                                                            float alpha, float* __restrict__ s,
                                                            float* __restrict__ inv_s,
                                                            float* __restrict__ amax_w) {
    const int lane = threadIdx.x % kWave;
    const int64_t j = (int64_t)blockIdx.x * 4 + threadIdx.x / kWave;
    if (j >= K) return;  // whole wavefront leaves together; no block barrier below
    const T* row = w + j * ld;
    float m = 0.0f;
    constexpr int U = 4;
    constexpr int step = kWave * 8;
    int64_t c = (int64_t)lane * 8;
    for (; kVec && c + (U - 1) * step + 8 <= N; c += U * step) {
        float v[U][8];
#pragma unroll
        for (int u = 0; u < U; ++u) load8(row + c + u * step, v[u]);
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(v[u][i]));
    }
    for (; c < N; c += step) {
        float v[8];
        load8_any<kVec>(row + c, N - c, v);
#pragma unroll
        for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(v[i]));
    }
    m = wave_max(m);
    if (lane == 0) {
        float sj, ij;
        smooth_factor(amax_x[j], m, alpha, sj, ij);
        s[j] = sj;
        inv_s[j] = ij;
        if (amax_w) amax_w[j] = m;
    }
}

// s and inv_s from both maxima already known (reuse of amax_w across alphas).
__global__ __launch_bounds__(256) void k_factors(const float* __restrict__ amax_x,
                                                 const float* __restrict__ amax_w, int64_t K, float alpha,
                                                 float* __restrict__ s, float* __restrict__ inv_s) {
    const int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (j >= K) return;
    float sj, ij;
    smooth_factor(amax_x[j], amax_w[j], alpha, sj, ij);
    s[j] = sj;
    inv_s[j] = ij;
}

}  // namespace sqk

// ---- launchers -------------------------------------------------------------

namespace sqk {

hipError_t launch_fill_u32(uint32_t* out, int64_t n, uint32_t v, hipStream_t st) {
    if (n <= 0) return hipSuccess;
    const int64_t blocks = (n + 255) / 256;
    hipLaunchKernelGGL(k_fill_u32, dim3((unsigned)blocks), dim3(256), 0, st, out, n, v);
    return hipGetLastError();
}

// Rows per block chosen so the grid has about `target` blocks in total but
// each block still reads at least 64 rows (bounds the atomics per element).
static int64_t rows_per_block_for(int64_t rows, int64_t col_blocks, int64_t target) {
    int64_t row_blocks = target / (col_blocks > 0 ? col_blocks : 1);
    if (row_blocks < 1) row_blocks = 1;
    int64_t rpb = (rows + row_blocks - 1) / row_blocks;
    if (rpb < 64) rpb = 64;
    rpb = (rpb + kRowLanes - 1) / kRowLanes * kRowLanes;
    return rpb;
}

hipError_t launch_col_absmax(const void* x, bool bf16, int64_t rows, int64_t cols, int64_t ld,
                             const float* row_scale, uint32_t* out, hipStream_t st) {
    if (rows <= 0 || cols <= 0) return hipSuccess;
    const int64_t col_blocks = (cols + kColsPerBlock - 1) / kColsPerBlock;
    const int64_t rpb = rows_per_block_for(rows, col_blocks, 2048);
    const int64_t row_blocks = (rows + rpb - 1) / rpb;
    dim3 grid((unsigned)col_blocks, (unsigned)row_blocks);
    const bool vec = rows_aligned16(x, ld, bf16 ? 2 : 4);
    auto go = [&](auto tag, auto scaled, auto vecc) {
        using T = decltype(tag);
        hipLaunchKernelGGL((k_col_absmax<T, decltype(scaled)::value, decltype(vecc)::value>), grid, dim3(256), 0, st,
                           static_cast<const T*>(x), rows, cols, ld, row_scale, out, rpb);
    };
    using TT = std::true_type;
    using FF = std::false_type;
    if (bf16) {
        if (row_scale) { if (vec) go(bf16_t{}, TT{}, TT{}); else go(bf16_t{}, TT{}, FF{}); }
        else { if (vec) go(bf16_t{}, FF{}, TT{}); else go(bf16_t{}, FF{}, FF{}); }
    } else {
        if (row_scale) { if (vec) go(float{}, TT{}, TT{}); else go(float{}, TT{}, FF{}); }
        else { if (vec) go(float{}, FF{}, TT{}); else go(float{}, FF{}, FF{}); }
    }
    return hipGetLastError();
}

hipError_t launch_row_absmax_factors(const void* w, bool bf16, int64_t K, int64_t N, int64_t ld,
                                     const float* amax_x, float alpha, float* s, float* inv_s, float* amax_w,
                                     hipStream_t st) {
    if (K <= 0) return hipSuccess;
    const int64_t blocks = (K + 3) / 4;
    const bool vec = rows_aligned16(w, ld, bf16 ? 2 : 4);
    auto go = [&](auto tag, auto vecc) {
        using T = decltype(tag);
        hipLaunchKernelGGL((k_row_absmax_factors<T, decltype(vecc)::value>), dim3((unsigned)blocks), dim3(256), 0, st,
                           static_cast<const T*>(w), K, N, ld, amax_x, alpha, s, inv_s, amax_w);
    };
    if (bf16) { if (vec) go(bf16_t{}, std::true_type{}); else go(bf16_t{}, std::false_type{}); }
    else { if (vec) go(float{}, std::true_type{}); else go(float{}, std::false_type{}); }
    return hipGetLastError();
}

hipError_t launch_factors(const float* amax_x, const float* amax_w, int64_t K, float alpha, float* s,
                          float* inv_s, hipStream_t st) {
    if (K <= 0) return hipSuccess;
    const int64_t blocks = (K + 255) / 256;
    hipLaunchKernelGGL(k_factors, dim3((unsigned)blocks), dim3(256), 0, st, amax_x, amax_w, K, alpha, s, inv_s);
    return hipGetLastError();
}

}  // namespace sqk
