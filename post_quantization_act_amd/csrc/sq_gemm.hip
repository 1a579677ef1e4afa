// INT8 x INT8 -> int32 GEMM with the SmoothQuant dequantization epilogue on
// gfx950 matrix cores (v_mfma_i32_32x32x32_i8).
//
//   acc[m, n] = sum_k Xq[m, k] * Wq[n, k]        (exact int32)
//   y[m, n]   = bf16_rne(fl(fl(float(acc) * x_scale[m]) * w_scale[n]))
//
// Both operands are K-contiguous (Xq [M, K], Wq [N, K]).  The kernel computes
// the transposed product D = Wq . Xq^T so that each lane's accumulator
// registers run along n, which is the contiguous axis of y: four consecutive
// outputs leave as one 8-byte bf16 store.
//
// Block tile BN (n) x BM (m) x 128 (k), 256 threads = 2 x 2 wavefronts, each
// wavefront owning a (BN/2) x (BM/2) sub-tile of 32 x 32 MFMA blocks.
// Operand tiles are staged through LDS, double-buffered: while the matrix
// cores work on stage k, the next stage's 16-byte global loads are in flight
// in registers and are written to the other LDS buffer afterwards.  LDS rows
// are 128 bytes (8 chunks of 16 B); chunk c of row r lives at slot
// c ^ ((r >> 1) & 7), which makes both the 16-byte LDS writes and the
// fragment reads (16 rows x one chunk per quarter-wave) bank-conflict free.
#include "sq_device.h"
#include "sq_internal.h"

namespace sqk {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int kBK = 128;  // bytes of k per stage (one 128-byte line per row)

__device__ __forceinline__ int swz(int r, int c) { return r * 8 + (c ^ ((r >> 1) & 7)); }

template <int BN, int BM, int kOut /*0: bf16, 1: fp32*/, bool kAcc>
__global__ __launch_bounds__(256) void k_gemm_w8a8(const int8_t* __restrict__ xq, const float* __restrict__ x_scale,
                                                   int per_tensor, const int8_t* __restrict__ wq,
                                                   const float* __restrict__ w_scale, int M, int N, int K,
                                                   void* __restrict__ y, int32_t* __restrict__ acc_out,
                                                   int tiles_n) {
    constexpr int WN = BN / 2, WM = BM / 2;
    constexpr int TN = WN / 32, TM = WM / 32;
    constexpr int A_CHUNKS = BN * 8 / 256;  // 16-byte chunks per thread per stage
    constexpr int B_CHUNKS = BM * 8 / 256;
    constexpr int STAGE = (BN + BM) * 8;    // uint4 slots per stage

    __shared__ uint4 lds[2 * STAGE];

    const int tid = threadIdx.x;
    const int wave = tid / kWave, lane = tid % kWave;
    const int wn = wave % 2, wm = wave / 2;

    const int tile = blockIdx.x;
    const int tn = tile % tiles_n, tm = tile / tiles_n;
    const int n0 = tn * BN, m0 = tm * BM;

    // Global source rows of this thread's chunks (clamped into the matrix so
    // ragged edges read valid memory; their results are never stored).
    const int8_t* a_src[A_CHUNKS];
    const int8_t* b_src[B_CHUNKS];
    int a_slot[A_CHUNKS], b_slot[B_CHUNKS], a_kc[A_CHUNKS], b_kc[B_CHUNKS];
#pragma unroll
    for (int i = 0; i < A_CHUNKS; ++i) {
        const int q = tid + i * 256;
        const int r = q / 8, c = q % 8;
        const int n = min(n0 + r, N - 1);
        a_src[i] = wq + (int64_t)n * K + c * 16;
        a_kc[i] = c * 16;
        a_slot[i] = swz(r, c);
    }
#pragma unroll
    for (int i = 0; i < B_CHUNKS; ++i) {
        const int q = tid + i * 256;
        const int r = q / 8, c = q % 8;
        const int m = min(m0 + r, M - 1);
        b_src[i] = xq + (int64_t)m * K + c * 16;
        b_kc[i] = c * 16;
        b_slot[i] = BN * 8 + swz(r, c);
    }

    v16i acc[TN][TM];
#pragma unroll
    for (int a = 0; a < TN; ++a)
#pragma unroll
        for (int b = 0; b < TM; ++b)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[a][b][e] = 0;

    uint4 ra[A_CHUNKS], rb[B_CHUNKS];
    const int nk = (K + kBK - 1) / kBK;

    auto gload = [&](int kt) {
        const int k0 = kt * kBK;
        const bool full = k0 + kBK <= K;
#pragma unroll
        for (int i = 0; i < A_CHUNKS; ++i)
            ra[i] = (full || k0 + a_kc[i] < K) ? ld16(a_src[i] + k0) : make_uint4(0, 0, 0, 0);
#pragma unroll
        for (int i = 0; i < B_CHUNKS; ++i)
            rb[i] = (full || k0 + b_kc[i] < K) ? ld16(b_src[i] + k0) : make_uint4(0, 0, 0, 0);
    };
    auto lstore = [&](int buf) {
        uint4* base = lds + buf * STAGE;
#pragma unroll
        for (int i = 0; i < A_CHUNKS; ++i) base[a_slot[i]] = ra[i];
#pragma unroll
        for (int i = 0; i < B_CHUNKS; ++i) base[b_slot[i]] = rb[i];
    };

    // Fragment rows of this lane: row (lane % 32) of each 32-row block, chunk
    // (2 * kstep + lane / 32) within the 128-byte row.
    const int fr = lane % 32, fh = lane / 32;

    if (nk > 0) {
        gload(0);
        lstore(0);
    }
    __syncthreads();

    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < nk) gload(kt + 1);
        const uint4* base = lds + cur * STAGE;
#pragma unroll
        for (int ks = 0; ks < kBK / 32; ++ks) {
            const int c = 2 * ks + fh;
            v4i af[TN], bfr[TM];
#pragma unroll
            for (int a = 0; a < TN; ++a) {
                const uint4 u = base[swz(wn * WN + a * 32 + fr, c)];
                af[a] = v4i{(int)u.x, (int)u.y, (int)u.z, (int)u.w};
            }
#pragma unroll
            for (int b = 0; b < TM; ++b) {
                const uint4 u = base[BN * 8 + swz(wm * WM + b * 32 + fr, c)];
                bfr[b] = v4i{(int)u.x, (int)u.y, (int)u.z, (int)u.w};
            }
#pragma unroll
            for (int a = 0; a < TN; ++a)
#pragma unroll
                for (int b = 0; b < TM; ++b)
                    acc[a][b] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[a], bfr[b], acc[a][b], 0, 0, 0);
        }
        if (kt + 1 < nk) lstore(cur ^ 1);
        __syncthreads();
    }

    // Epilogue.  32x32 accumulator layout: lane holds column (lane % 32) of
    // the block (here: m) and rows 8*g + 4*(lane/32) + e, e = 0..3, in
    // registers 4*g + e (here: n).
    const bool n_vec = (N % 4) == 0;
    const float xs_t = per_tensor ? x_scale[0] : 0.0f;
#pragma unroll
    for (int b = 0; b < TM; ++b) {
        const int m = m0 + wm * WM + b * 32 + fr;
        if (m >= M) continue;
        const float xs = per_tensor ? xs_t : x_scale[m];
#pragma unroll
        for (int a = 0; a < TN; ++a) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int n = n0 + wn * WN + a * 32 + 8 * g + 4 * fh;
                if (n >= N) continue;
                int32_t av[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) av[e] = acc[a][b][4 * g + e];
                float yv[4];
                if (n_vec) {
                    const float4 ws = *reinterpret_cast<const float4*>(w_scale + n);
                    yv[0] = ((float)av[0] * xs) * ws.x;
                    yv[1] = ((float)av[1] * xs) * ws.y;
                    yv[2] = ((float)av[2] * xs) * ws.z;
                    yv[3] = ((float)av[3] * xs) * ws.w;
                    const int64_t off = (int64_t)m * N + n;
                    if constexpr (kOut == 0) {
                        uint2 pk = make_uint2(pack_bf16x2(yv[0], yv[1]), pack_bf16x2(yv[2], yv[3]));
                        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(y) + off) = pk;
                    } else {
                        *reinterpret_cast<float4*>(static_cast<float*>(y) + off) = make_float4(yv[0], yv[1], yv[2], yv[3]);
                    }
                    if constexpr (kAcc) *reinterpret_cast<int4*>(acc_out + off) = make_int4(av[0], av[1], av[2], av[3]);
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        if (n + e >= N) break;
                        const float v = ((float)av[e] * xs) * w_scale[n + e];
                        const int64_t off = (int64_t)m * N + n + e;
                        if constexpr (kOut == 0) {
                            static_cast<uint16_t*>(y)[off] = (uint16_t)(pack_bf16x2(v, 0.0f) & 0xFFFFu);
                        } else {
                            static_cast<float*>(y)[off] = v;
                        }
                        if constexpr (kAcc) acc_out[off] = av[e];
                    }
                }
            }
        }
    }
}

template <int BN, int BM>
static void launch_tiles(const int8_t* xq, const float* x_scale, bool per_tensor, const int8_t* wq,
                         const float* w_scale, int M, int N, int K, void* y, bool y_bf16, int32_t* acc_out,
                         hipStream_t st) {
    const int tiles_n = (N + BN - 1) / BN;
    const int tiles_m = (M + BM - 1) / BM;
    dim3 grid((unsigned)(tiles_n * tiles_m));
    const int pt = per_tensor ? 1 : 0;
    if (y_bf16) {
        if (acc_out)
            hipLaunchKernelGGL((k_gemm_w8a8<BN, BM, 0, true>), grid, dim3(256), 0, st, xq, x_scale, pt, wq, w_scale, M, N, K, y, acc_out, tiles_n);
        else
            hipLaunchKernelGGL((k_gemm_w8a8<BN, BM, 0, false>), grid, dim3(256), 0, st, xq, x_scale, pt, wq, w_scale, M, N, K, y, acc_out, tiles_n);
    } else {
        if (acc_out)
            hipLaunchKernelGGL((k_gemm_w8a8<BN, BM, 1, true>), grid, dim3(256), 0, st, xq, x_scale, pt, wq, w_scale, M, N, K, y, acc_out, tiles_n);
        else
            hipLaunchKernelGGL((k_gemm_w8a8<BN, BM, 1, false>), grid, dim3(256), 0, st, xq, x_scale, pt, wq, w_scale, M, N, K, y, acc_out, tiles_n);
    }
}

hipError_t launch_gemm_w8a8(const int8_t* xq, const float* x_scale, bool per_tensor, const int8_t* wq,
                            const float* w_scale, int64_t M, int64_t N, int64_t K, void* y, bool y_bf16,
                            int32_t* acc_out, hipStream_t st) {
    if (M <= 0 || N <= 0) return hipSuccess;
    launch_tiles<256, 128>(xq, x_scale, per_tensor, wq, w_scale, (int)M, (int)N, (int)K, y, y_bf16, acc_out, st);
    return hipGetLastError();
}

}  // namespace sqk
