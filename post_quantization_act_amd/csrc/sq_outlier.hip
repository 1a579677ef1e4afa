// Kernels of the LLM.int8()-style comparator (page "4.2 W8A8 量化与 SmoothQuant"
// section 2; page "量化：只压权重，与训练后量化（PTQ）", SmoothQuant W8A8 results
// paragraph): the input channels whose activation maximum exceeds a
// threshold are taken out of the INT8 product and multiplied in 16 bits.
//
//  - k_outlier_columns: one block compacts the outlier channels in ascending
//    order (wavefront ballots + an LDS scan over the 16 wavefronts) and writes
//    the 0/1 keep mask the INT8 quantizer multiplies the activations by.
//  - k_gather_x / k_gather_w: copy the outlier channels of X (columns) and W
//    (rows) into two small k-contiguous bf16 operands [M, kp] and [N, kp],
//    zero-padded to a multiple of 16 channels, which the GEMM epilogue feeds
//    to the bf16 matrix cores.
// The outlier count stays on the device: every kernel reads it from memory,
// so the pass needs no host synchronization.
#include "sq_device.h"
#include "sq_internal.h"

namespace sqk {

constexpr int kSelThreads = 1024;

__global__ __launch_bounds__(kSelThreads) void k_outlier_columns(const float* __restrict__ amax, int K, float thr,
                                                                 int32_t* __restrict__ idx, int32_t* __restrict__ count,
                                                                 float* __restrict__ keep) {
    constexpr int NW = kSelThreads / kWave;
    __shared__ int wtot[NW];
    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));  // lanes under this one
    int base = 0;
    for (int j0 = 0; j0 < K; j0 += kSelThreads) {
        const int j = j0 + tid;
        const bool out = j < K && amax[j] > thr;
        if (j < K) keep[j] = out ? 0.0f : 1.0f;
        const uint64_t m = __ballot(out);
        if (lane == 0) wtot[wave] = __popcll(m);
        __syncthreads();
        int before = 0, total = 0;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            const int c = wtot[w];
            before += w < wave ? c : 0;
            total += c;
        }
        if (out) idx[base + before + __popcll(m & below)] = j;
        base += total;
        __syncthreads();  // wtot is rewritten by the next chunk
    }
    if (tid == 0) count[0] = base;
}

// One wavefront per token row: x_o[i, t] = x[i, idx[t]] for t < n, 0 up to
// the next multiple of 16.
__global__ __launch_bounds__(256) void k_gather_x(const uint16_t* __restrict__ x, int64_t M, int64_t ldx,
                                                  const int32_t* __restrict__ idx, const int32_t* __restrict__ count,
                                                  int64_t kp, uint16_t* __restrict__ x_o) {
    const int lane = threadIdx.x % kWave;
    const int64_t i = (int64_t)blockIdx.x * 4 + threadIdx.x / kWave;
    if (i >= M) return;
    const int n = __builtin_amdgcn_readfirstlane(count[0]);
    const int n16 = (n + 15) & ~15;
    const uint16_t* xr = x + i * ldx;
    uint16_t* o = x_o + i * kp;
    for (int t = lane; t < n16; t += kWave) o[t] = t < n ? xr[idx[t]] : (uint16_t)0;
}

// One thread per output channel k and slice of outlier channels:
// w_ot[k, t] = w[idx[t], k], eight channels t per 16-byte store, the octets of
// t dealt round-robin over gridDim.y slices; loads of consecutive k are
// coalesced.
__global__ __launch_bounds__(256) void k_gather_w(const uint16_t* __restrict__ w, int64_t N, int64_t ldw,
                                                  const int32_t* __restrict__ idx, const int32_t* __restrict__ count,
                                                  int64_t kp, uint16_t* __restrict__ w_ot) {
    const int64_t k = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (k >= N) return;
    const int n = __builtin_amdgcn_readfirstlane(count[0]);
    const int n16 = (n + 15) & ~15;
    uint16_t* o = w_ot + k * kp;
    for (int t0 = 8 * (int)blockIdx.y; t0 < n16; t0 += 8 * (int)gridDim.y) {
        uint32_t v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int t = t0 + 2 * e;
            const uint32_t lo = t < n ? w[(int64_t)idx[t] * ldw + k] : 0u;
            const uint32_t hi = t + 1 < n ? w[(int64_t)idx[t + 1] * ldw + k] : 0u;
            v[e] = lo | (hi << 16);
        }
        *reinterpret_cast<uint4*>(o + t0) = make_uint4(v[0], v[1], v[2], v[3]);
    }
}

constexpr int kGatherSlices = 8;

hipError_t launch_outlier_columns(const float* amax, int64_t K, float thr, int32_t* idx, int32_t* count, float* keep,
                                  hipStream_t st) {
    hipLaunchKernelGGL(k_outlier_columns, dim3(1), dim3(kSelThreads), 0, st, amax, (int)K, thr, idx, count, keep);
    return hipGetLastError();
}

hipError_t launch_gather_outliers(const uint16_t* x, int64_t M, int64_t ldx, const uint16_t* w, int64_t N,
                                  int64_t ldw, const int32_t* idx, const int32_t* count, int64_t kp, uint16_t* x_o,
                                  uint16_t* w_ot, hipStream_t st) {
    if (M > 0) hipLaunchKernelGGL(k_gather_x, dim3((unsigned)((M + 3) / 4)), dim3(256), 0, st, x, M, ldx, idx, count,
                                  kp, x_o);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (N > 0) hipLaunchKernelGGL(k_gather_w, dim3((unsigned)((N + 255) / 256), kGatherSlices), dim3(256), 0, st, w,
                                  N, ldw, idx, count, kp, w_ot);
    return hipGetLastError();
}

}  // namespace sqk
