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
template <bool kGeneral = true>
__device__ __forceinline__ double pow_cases(double x, double e) {
    if (e == 0.0) return 1.0;
    if (e == 1.0) return x;
    if (e == 0.5 || !kGeneral) return sqrt(x);  // !kGeneral: the caller guarantees e is 0, 1/2 or 1
    return pow(x, e);
}

// s = a^alpha / b^(1-alpha) with both maxima floored at 1e-5f, in fp64 and
// rounded once; inv_s = correctly rounded fp32 reciprocal.
template <bool kGeneral = true>
__device__ __forceinline__ void smooth_factor(float ax, float aw, float alpha, float& s, float& inv_s) {
    const float fl = 1e-5f;
    const float a = ax > fl ? ax : fl;
    const float b = aw > fl ? aw : fl;
    const double ea = (double)alpha;
    const double eb = 1.0 - ea;
    s = (float)(pow_cases<kGeneral>((double)a, ea) / pow_cases<kGeneral>((double)b, eb));
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

// ---- steps 2 + 3a fused: one read of W gives amax_w, s, inv_s and the
// column maxima of diag(s) W ------------------------------------------------
//
// A block of NT threads (1024 on rows of more than 256 8-column groups, else
// 512) streams the rows [r0, r1) of W (bf16, 16-byte aligned rows,
// N % 8 == 0, N <= 49152).
// Each iteration takes RB rows: row slot t / TPR (TPR = NT / RB threads per
// row); thread t % TPR of a slot owns the 8-column groups q = t % TPR + TPR i,
// i < GPT, and keeps their running column maxima in registers (GR groups) or
// LDS (GL more).  Per row: max |w| over the slot (shuffles, then LDS across
// its wavefronts behind one barrier), s_j by the same fp64 rule as
// k_row_absmax_factors, then the running maxima take |fl(s_j w)|.  For alpha
// in {0, 1/2, 1} the two powers are exact forms computed in place; for any
// other alpha (kTab) they come from tables of pow_cases built before the pass
// (k_pow_tables): the numerator per row of W, the denominator per bf16 value
// of the row maximum, which is always one of the row's bf16 elements.  The
// tables hold the fp64 values the in-place rule would compute, so s_j is the
// same; the pass keeps the registers of the exact-alpha form instead of the
// fp64 pow's.  The next
// row's loads are issued at the top of the iteration and stay in flight
// through the reduction, the factor and the update; the barrier waits on LDS
// only, and nothing else touches global memory in the loop: amax_x is staged
// in LDS before, the per-row results are written after it.  The block's
// column maxima (its RB slots combined through LDS) leave as plain stores to
// partial[blockIdx.x][N]; k_colmax_reduce takes the maximum over blocks.
// kKeep: plain loads instead of nontemporal ones, for a W that the weight
// codes read again right after this pass.
constexpr int kPrepThreads = 512;
constexpr int kPrepMaxRows = 256;  // rows per block (LDS staging of per-row values)
constexpr int kPowTabB = 32768;    // denominator table: bf16 patterns 0 .. 0x7FFF, then the floor

// tab[i] = pow_cases(bf16 value of pattern i, 1 - alpha) for i < kPowTabB,
// tab[kPowTabB] = pow_cases(1e-5f, 1 - alpha), then
// tab[kPowTabB + 1 + j] = pow_cases(max(amax_x[j], 1e-5f), alpha), j < K.
__global__ __launch_bounds__(256) void k_pow_tables(const float* __restrict__ amax_x, int64_t K, float alpha,
                                                    double* __restrict__ tab) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const float fl = 1e-5f;
    const double ea = (double)alpha, eb = 1.0 - ea;
    if (i < kPowTabB) {
        tab[i] = pow_cases((double)__uint_as_float((uint32_t)i << 16), eb);
    } else if (i == kPowTabB) {
        tab[i] = pow_cases((double)fl, eb);
    } else if (i <= kPowTabB + K) {
        const float a = amax_x[i - kPowTabB - 1];
        tab[i] = pow_cases((double)(a > fl ? a : fl), ea);
    }
}

__device__ __forceinline__ void lds_only_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

template <int RB, int GR, int GL, bool kTab, int NT = kPrepThreads, bool kKeep = false>
__global__ __launch_bounds__(NT) void k_prep_rows(const bf16_t* __restrict__ w, int64_t K, int64_t N,
                                                            int64_t ld, const float* __restrict__ amax_x,
                                                            float alpha, const double* __restrict__ tab,
                                                            float* __restrict__ s, float* __restrict__ inv_s,
                                                            float* __restrict__ amax_w, float* __restrict__ partial,
                                                            int rows_per_block) {
    // GR groups keep their running maxima in registers, GL more in LDS
    // (thread-major, so each access is conflict-free)
    constexpr int GPT = GR + GL;
    constexpr int TPR = NT / RB, WPR = TPR / kWave;
    static_assert(RB == 1 || GL == 0, "LDS-held maxima only with one row per iteration");
    __shared__ float red[2][NT / kWave];
    __shared__ float axl[kPrepMaxRows], srow[kPrepMaxRows], irow[kPrepMaxRows], arow[kPrepMaxRows];
    __shared__ double pal[kTab ? kPrepMaxRows : 1];  // numerators of the rows (kTab)
    __shared__ float comb[RB > 1 ? (RB - 1) * TPR * 8 * GPT : 1];
    __shared__ float cml[GL > 0 ? GL * 8 * NT : 1];
    const int t = threadIdx.x, slot = t / TPR, ts = t % TPR, wave = t / kWave, lane = t % kWave;
    const int64_t r0 = (int64_t)blockIdx.x * rows_per_block;
    const int nrows = (int)min((int64_t)rows_per_block, K - r0);
    for (int i = t; i < nrows; i += NT) {
        if constexpr (kTab) pal[i] = tab[kPowTabB + 1 + r0 + i];
        else axl[i] = amax_x[r0 + i];
    }
#pragma unroll
    for (int i = 0; i < GL * 8; ++i) cml[i * NT + t] = 0.0f;
    const int iters = (nrows + RB - 1) / RB;

    float cm[GR][8];
#pragma unroll
    for (int i = 0; i < GR; ++i)
#pragma unroll
        for (int e = 0; e < 8; ++e) cm[i][e] = 0.0f;
    uint4 cur[GPT], nxt[GPT];
    auto load_rows = [&](int it, uint4 (&dst)[GPT]) {
        const int rl = it * RB + slot;
        const bf16_t* row = w + (r0 + rl) * ld;
#pragma unroll
        for (int i = 0; i < GPT; ++i) {
            const int64_t q = ts + (int64_t)TPR * i;
            const bool in = rl < nrows && 8 * q < N;
            dst[i] = in ? (kKeep ? ld16(row + 8 * q) : ld16_stream(row + 8 * q)) : make_uint4(0, 0, 0, 0);
        }
    };
    if (iters > 0) load_rows(0, cur);
    for (int it = 0; it < iters; ++it) {
        const int rl = it * RB + slot;
        // the next rows' loads go out first, so they are in flight during this
        // row's reduction, factor and column update
        if (it + 1 < iters) load_rows(it + 1, nxt);
        float m = 0.0f;
#pragma unroll
        for (int i = 0; i < GPT; ++i) {
            const uint32_t u[4] = {cur[i].x, cur[i].y, cur[i].z, cur[i].w};
#pragma unroll
            for (int h = 0; h < 4; ++h) m = fmaxf(m, fmaxf(fabsf(bf16_lo(u[h])), fabsf(bf16_hi(u[h]))));
        }
        m = wave_max(m);
        if (lane == 0) red[it & 1][wave] = m;
        lds_only_barrier();
        // the row stays packed across the barrier and the factor: unpack it
        // again below instead of keeping 8 floats per group alive
#pragma unroll
        for (int i = 0; i < GPT; ++i)
            asm volatile("" : "+v"(cur[i].x), "+v"(cur[i].y), "+v"(cur[i].z), "+v"(cur[i].w));
        if (rl < nrows) {  // uniform over the slot's wavefronts
            float rm = 0.0f;
#pragma unroll
            for (int v = 0; v < WPR; ++v) rm = fmaxf(rm, red[it & 1][slot * WPR + v]);
            float sj = 0.0f, ij = 0.0f;
            if (lane == 0) {
                if constexpr (kTab) {
                    // the floored maximum rm > 1e-5f is a bf16 value: its pattern indexes the table
                    const float fl = 1e-5f;
                    const double pb = tab[rm > fl ? (int)(__float_as_uint(rm) >> 16) : kPowTabB];
                    sj = (float)(pal[rl] / pb);
                    ij = 1.0f / sj;
                } else {
                    smooth_factor<false>(axl[rl], rm, alpha, sj, ij);
                }
            }
            sj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(sj), 0));  // lane 0 to the wavefront
            if (ts == 0) {
                srow[rl] = sj;
                irow[rl] = ij;
                arow[rl] = rm;
            }
#pragma unroll
            for (int i = 0; i < GPT; ++i) {
                const uint32_t u[4] = {cur[i].x, cur[i].y, cur[i].z, cur[i].w};
#pragma unroll
                for (int h = 0; h < 4; ++h) {
                    const float a0 = fabsf(sj * bf16_lo(u[h])), a1 = fabsf(sj * bf16_hi(u[h]));
                    if (i < GR) {
                        cm[i < GR ? i : 0][2 * h] = fmaxf(cm[i < GR ? i : 0][2 * h], a0);
                        cm[i < GR ? i : 0][2 * h + 1] = fmaxf(cm[i < GR ? i : 0][2 * h + 1], a1);
                    } else {
                        float* c = cml + ((i - GR) * 8 + 2 * h) * NT + t;
                        c[0] = fmaxf(c[0], a0);
                        c[NT] = fmaxf(c[NT], a1);
                    }
                }
            }
        }
#pragma unroll
        for (int i = 0; i < GPT; ++i) cur[i] = nxt[i];
    }
    if constexpr (RB > 1) {
        if (slot > 0) {
#pragma unroll
            for (int i = 0; i < GPT; ++i)
#pragma unroll
                for (int e = 0; e < 8; ++e) comb[(((slot - 1) * GPT + i) * TPR + ts) * 8 + e] = cm[i][e];
        }
    }
    lds_only_barrier();
    if (slot == 0) {
#pragma unroll
        for (int i = 0; i < GPT; ++i) {
            const int64_t q = ts + (int64_t)TPR * i;
            if (8 * q >= N) continue;
            float o[8];
#pragma unroll
            for (int e = 0; e < 8; ++e)
                o[e] = i < GR ? cm[i < GR ? i : 0][e] : cml[((i - GR) * 8 + e) * NT + t];
            if constexpr (RB > 1) {
                for (int sl = 1; sl < RB; ++sl)
#pragma unroll
                    for (int e = 0; e < 8; ++e) o[e] = fmaxf(o[e], comb[(((sl - 1) * GPT + i) * TPR + ts) * 8 + e]);
            }
            float* dst = partial + (int64_t)blockIdx.x * N + 8 * q;
            *reinterpret_cast<float4*>(dst) = make_float4(o[0], o[1], o[2], o[3]);
            *reinterpret_cast<float4*>(dst + 4) = make_float4(o[4], o[5], o[6], o[7]);
        }
    }
    for (int i = t; i < nrows; i += NT) {
        s[r0 + i] = srow[i];
        inv_s[r0 + i] = irow[i];
        if (amax_w) amax_w[r0 + i] = arow[i];
    }
}

// colmax[k] = max over blocks b of partial[b][k], as fp32 bit patterns.
// A block of 1024 threads takes 64 columns: 16 column lanes of 4 floats
// (16-byte loads; N % 8 == 0 on this path) x 64 row lanes striding over the
// nb partial rows with four loads in flight, then the 64 row lanes are
// combined through LDS.
constexpr int kRedCols = 64, kRedRowLanes = 64;
__global__ __launch_bounds__(1024) void k_colmax_reduce(const float* __restrict__ partial, int nb, int64_t N,
                                                        uint32_t* __restrict__ colmax) {
    const int cl = threadIdx.x % 16, rl = threadIdx.x / 16;
    const int64_t c = (int64_t)blockIdx.x * kRedCols + cl * 4;
    float m[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    if (c < N) {
        auto take = [&](const float4 v) {
            m[0] = fmaxf(m[0], v.x);
            m[1] = fmaxf(m[1], v.y);
            m[2] = fmaxf(m[2], v.z);
            m[3] = fmaxf(m[3], v.w);
        };
        int b = rl;
        for (; b + 3 * kRedRowLanes < nb; b += 4 * kRedRowLanes) {
            float4 v[4];
#pragma unroll
            for (int u = 0; u < 4; ++u)
                v[u] = *reinterpret_cast<const float4*>(partial + (int64_t)(b + u * kRedRowLanes) * N + c);
#pragma unroll
            for (int u = 0; u < 4; ++u) take(v[u]);
        }
        for (; b < nb; b += kRedRowLanes) take(*reinterpret_cast<const float4*>(partial + (int64_t)b * N + c));
    }
    __shared__ float red[kRedRowLanes][kRedCols];
#pragma unroll
    for (int e = 0; e < 4; ++e) red[rl][cl * 4 + e] = m[e];
    __syncthreads();
    if (threadIdx.x < kRedCols) {
        float r = 0.0f;
#pragma unroll 8
        for (int q = 0; q < kRedRowLanes; ++q) r = fmaxf(r, red[q][threadIdx.x]);
        const int64_t gc = (int64_t)blockIdx.x * kRedCols + threadIdx.x;
        if (gc < N) colmax[gc] = __float_as_uint(r);
    }
}

// Static per-tensor activation maximum from the calibration statistics:
// a = max_j fl(amax_x[j] * inv_s[j]) (inv_s NULL: max_j amax_x[j]).  Rounding
// is monotonic, so this is the largest |fl(x * inv_s_j)| of the calibration
// tokens.  One block; out[0] is written, not accumulated.
__global__ __launch_bounds__(1024) void k_static_max(const float* __restrict__ amax_x,
                                                     const float* __restrict__ inv_s, int64_t K,
                                                     float* __restrict__ out) {
    __shared__ float red[16];
    float m = 0.0f;
    for (int64_t j = threadIdx.x; j < K; j += 1024) m = fmaxf(m, inv_s ? amax_x[j] * inv_s[j] : amax_x[j]);
    m = wave_max(m);
    if (threadIdx.x % kWave == 0) red[threadIdx.x / kWave] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
        float r = red[0];
        for (int i = 1; i < 16; ++i) r = fmaxf(r, red[i]);
        out[0] = r;
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


// About 256 blocks (one per CU), at most kPrepMaxRows rows each, none empty.
int prep_blocks(int64_t K) {
    if (K <= 0) return 0;
    int64_t rpb = (K + 255) / 256;
    if (rpb > kPrepMaxRows) rpb = kPrepMaxRows;
    return (int)((K + rpb - 1) / rpb);
}

bool prep_fused_supported(const void* w, bool bf16, int64_t N, int64_t ld, float alpha) {
    (void)alpha;  // every alpha takes the one-read pass up to 6144 groups of 8 columns
    return bf16 && N > 0 && N % 8 == 0 && N / 8 <= 6144 && rows_aligned16(w, ld, 2);
}

int64_t prep_table_entries(int64_t K) { return K > 0 ? kPowTabB + 1 + K : 0; }

hipError_t launch_prepare_weights(const void* w, bool bf16, int64_t K, int64_t N, int64_t ld, const float* amax_x,
                                  float alpha, float* s, float* inv_s, float* amax_w, float* partial,
                                  uint32_t* colmax, double* tab, hipStream_t st) {
    if (K <= 0 || N <= 0) return hipSuccess;
    if (!prep_fused_supported(w, bf16, N, ld, alpha) || !tab) return hipErrorNotSupported;
    const int nb = prep_blocks(K);
    const int rpb = (int)((K + nb - 1) / nb);
    const int64_t groups = N / 8;
    const bf16_t* wb = static_cast<const bf16_t*>(w);
    // W of up to 128 MB is read without the nontemporal hint, so the caches
    // (the 256 MB memory-side cache above all) still hold much of it when the
    // weight codes read it again right after: 1.8 us off steps 2-4 at
    // 4096x4096.  Larger W streams.
    const bool keep = (uint64_t)K * (uint64_t)ld * 2u <= (128ull << 20);
#define SQ_PREP_KEEP(RB, GR, GL, G, NT, KEEP)                                                                     \
    hipLaunchKernelGGL((k_prep_rows<RB, GR, GL, G, NT, KEEP>), dim3((unsigned)nb), dim3(NT), 0, st, wb, K, N, ld,     \
                       amax_x, alpha, tab, s, inv_s, amax_w, partial, rpb)
#define SQ_PREP_NT(RB, GR, GL, G, NT)                                                                             \
    do {                                                                                                          \
        if (keep) SQ_PREP_KEEP(RB, GR, GL, G, NT, true);                                                          \
        else SQ_PREP_KEEP(RB, GR, GL, G, NT, false);                                                              \
    } while (0)
#define SQ_PREP(RB, GR, GL, G) SQ_PREP_NT(RB, GR, GL, G, kPrepThreads)
    // Rows per iteration so that each thread has 4-8 loads of 16 bytes in
    // flight per row set (several rows at once for narrow W: with one row per
    // iteration a 4096-column row is one 16-byte load per thread).  alpha
    // outside {0, 1/2, 1}: the powers from tables built first.
    const bool general = !(alpha == 0.0f || alpha == 0.5f || alpha == 1.0f);
    if (general) {
        const int64_t n = prep_table_entries(K);
        hipLaunchKernelGGL(k_pow_tables, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, amax_x, K, alpha, tab);
    }
    auto go = [&](auto g) {
        constexpr bool G = decltype(g)::value;
        // beyond 256 groups: 1024 threads (16 wavefronts per CU stream the
        // rows 3-8 % faster than 8), half the groups per thread
        if (groups <= 128) SQ_PREP(4, 1, 0, G);
        else if (groups <= 256) SQ_PREP(4, 2, 0, G);
        else if (groups <= 512) SQ_PREP_NT(4, 2, 0, G, 1024);
        else if (groups <= 1024) SQ_PREP_NT(4, 4, 0, G, 1024);
        else if (groups <= 2048) SQ_PREP_NT(2, 4, 0, G, 1024);
        else if (groups <= 3072) SQ_PREP_NT(1, 3, 0, G, 1024);
        else if (groups <= 4096) SQ_PREP_NT(1, 4, 0, G, 1024);
        else SQ_PREP_NT(1, 5, 1, G, 1024);  // up to 6144 groups: 5 in registers, 1 in LDS
    };
    if (general) go(std::true_type{});
    else go(std::false_type{});
#undef SQ_PREP
#undef SQ_PREP_NT
#undef SQ_PREP_KEEP
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_colmax_reduce, dim3((unsigned)((N + kRedCols - 1) / kRedCols)), dim3(1024), 0, st, partial, nb,
                       N, colmax);
    return hipGetLastError();
}

hipError_t launch_static_max(const float* amax_x, const float* inv_s, int64_t K, float* out, hipStream_t st) {
    hipLaunchKernelGGL(k_static_max, dim3(1), dim3(1024), 0, st, amax_x, inv_s, K, out);
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
