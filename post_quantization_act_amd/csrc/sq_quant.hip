// Quantization kernels of the SmoothQuant path on gfx950:
//  - smoothed weights to per-output-channel INT8, transposed to [N, K];
//  - smoothed activations to per-token (or per-tensor) INT8.
// Both are HBM-bound: read the bf16/fp32 source once, write one byte per
// element.
#include <type_traits>

#include "sq_device.h"
#include "sq_internal.h"

namespace sqk {

// ---- weights -----------------------------------------------------------------
//
// Tile of 128 input channels (j) x 128 output channels (k) per block of 256
// threads.  Thread (rg, cg) reads an 8 x 8 sub-block: 8 rows j, 8 consecutive
// k (one 16-byte load per row for bf16).  A wavefront holds 8 row groups x 8
// column groups, so each load instruction reads 8 full 128-byte lines.
// Codes are transposed through LDS: the thread writes, for each of its 8
// columns, the 8 codes along j as one 8-byte word; rows of the LDS tile are
// padded to 136 bytes so a wavefront's 8-byte writes spread over all banks.
// The tile then leaves as 16-byte stores of 16 consecutive j of one output
// channel (wq is [N, K], K contiguous), nontemporal when stream_out is set.
constexpr int kQwTile = 128;
constexpr int kQwStride = kQwTile + 8;
constexpr int kQwGroup = 16;

template <typename T, bool kScaled, bool kVec>
__device__ __forceinline__ void quant_weight_tile(int64_t bid, const T* __restrict__ w, int64_t K, int64_t N,
                                                  int64_t ld, const float* __restrict__ s,
                                                  const uint32_t* __restrict__ colmax, int8_t* __restrict__ wq,
                                                  float* __restrict__ w_scale, bool stream_out) {
    __shared__ float r_s[kQwTile];
    __shared__ __align__(16) uint8_t tile[kQwTile * kQwStride];

    // 1-D grid over the tiles in groups of kQwGroup output-channel tiles,
    // input-channel tiles fastest inside a group: the blocks in flight together
    // write whole rows of wq (contiguous) and read kQwGroup * 256-byte runs of
    // each row of W.
    const int64_t tj = (K + kQwTile - 1) / kQwTile;
    const int64_t per = (int64_t)kQwGroup * tj;
    const int64_t grp = bid / per, rem = bid % per;
    const int64_t k0 = (grp * kQwGroup + rem / tj) * kQwTile;
    const int64_t j0 = (rem % tj) * kQwTile;
    const int t = threadIdx.x;
    const int wave = t / kWave, lane = t % kWave;
    const int cg = (lane % 8) + 8 * (wave % 2);
    const int rg = (lane / 8) + 8 * (wave / 2);
    const int64_t kc = k0 + cg * 8;
    const int64_t ncol = N - kc;

    // The thread's 8 rows (and their s) are loaded before anything waits: with
    // 16-byte rows (kVec) as buffer loads over the tile's rows below K, so
    // rows past K, and groups of a lane whose 8 columns are not all inside N,
    // read zeros without a branch (the latter then load element-wise).
    float v[8][8];
    float sv[8];
    if constexpr (kVec) {
        const int rows = (int)min<int64_t>(kQwTile, K - j0);
        const __amdgpu_buffer_rsrc_t rs = row_rsrc(w + j0 * ld, (int)(rows * ld * (int64_t)sizeof(T)));
        const bool full = ncol >= 8;
        constexpr int kLd = 8 * (int)sizeof(T) / 16;  // 16-byte loads per row
        uint4 raw[8][kLd];
#pragma unroll
        for (int rr = 0; rr < 8; ++rr)
#pragma unroll
            for (int h = 0; h < kLd; ++h) {
                const int off = (int)(((rg * 8 + rr) * ld + kc) * (int64_t)sizeof(T)) + 16 * h;
                raw[rr][h] = ld16_buf_stream(rs, full ? off : 0x7FFFFFF0);
            }
        if constexpr (kScaled) {
            const __amdgpu_buffer_rsrc_t rsj = row_rsrc(s + j0, rows * 4);
#pragma unroll
            for (int rr = 0; rr < 8; ++rr) sv[rr] = ld4_buf(rsj, (rg * 8 + rr) * 4);
        }
#pragma unroll
        for (int rr = 0; rr < 8; ++rr) {
            if constexpr (sizeof(T) == 2) {
                const uint32_t u[4] = {raw[rr][0].x, raw[rr][0].y, raw[rr][0].z, raw[rr][0].w};
#pragma unroll
                for (int h = 0; h < 4; ++h) {
                    v[rr][2 * h] = bf16_lo(u[h]);
                    v[rr][2 * h + 1] = bf16_hi(u[h]);
                }
            } else {
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    v[rr][4 * h] = __uint_as_float(raw[rr][h].x);
                    v[rr][4 * h + 1] = __uint_as_float(raw[rr][h].y);
                    v[rr][4 * h + 2] = __uint_as_float(raw[rr][h].z);
                    v[rr][4 * h + 3] = __uint_as_float(raw[rr][h].w);
                }
            }
        }
        if (!full && ncol > 0) {
#pragma unroll
            for (int rr = 0; rr < 8; ++rr) {
                const int64_t j = j0 + rg * 8 + rr;
                if (j < K) load8_tail(w + j * ld + kc, ncol, v[rr]);
            }
        }
    } else {
        if (ncol > 0) {
#pragma unroll
            for (int rr = 0; rr < 8; ++rr) {
                const int64_t j = j0 + rg * 8 + rr;
                if (j < K) {
                    load8_tail(w + j * ld + kc, ncol, v[rr]);
                } else {
#pragma unroll
                    for (int i = 0; i < 8; ++i) v[rr][i] = 0.0f;
                }
            }
        }
#pragma unroll
        for (int rr = 0; rr < 8; ++rr) {
            const int64_t j = j0 + rg * 8 + rr;
            sv[rr] = (kScaled && j < K) ? s[j] : 1.0f;
        }
    }

    if (t < kQwTile) {
        const int64_t k = k0 + t;
        float scale = 0.0f, r = 0.0f;
        if (k < N) {
            group_scale(__uint_as_float(colmax[k]), scale, r);
            if (j0 == 0) w_scale[k] = scale;
        }
        r_s[t] = r;
    }
    __syncthreads();

    uint32_t lo[8], hi[8];  // per column cc: codes of rows 0..3 (lo) and 4..7 (hi)
#pragma unroll
    for (int cc = 0; cc < 8; ++cc) lo[cc] = hi[cc] = 0u;

    if (ncol > 0) {
        float rr_[8];
        bool finite = true;
#pragma unroll
        for (int cc = 0; cc < 8; ++cc) {
            rr_[cc] = r_s[cg * 8 + cc];
            finite = finite && (rr_[cc] <= 3.402823466e38f);
        }
        auto code_all = [&](auto fast) {
#pragma unroll
            for (int cc = 0; cc < 8; ++cc) {
                if constexpr (decltype(fast)::value) {
                    // the column's max (taken over these same fl(s_j w) values)
                    // bounds each of them: no clamp
                    uint32_t c[8];
#pragma unroll
                    for (int rr = 0; rr < 8; ++rr)
                        c[rr] = code8_bounded_bits(kScaled ? sv[rr] * v[rr][cc] : v[rr][cc], rr_[cc]);
                    lo[cc] = pack4_low(c[0], c[1], c[2], c[3]);
                    hi[cc] = pack4_low(c[4], c[5], c[6], c[7]);
                } else {
#pragma unroll
                    for (int rr = 0; rr < 8; ++rr) {
                        const float wp = kScaled ? sv[rr] * v[rr][cc] : v[rr][cc];
                        const uint32_t c = uint32_t(code8(wp, rr_[cc])) & 0xFFu;
                        if (rr < 4) lo[cc] |= c << (8 * rr);
                        else hi[cc] |= c << (8 * (rr - 4));
                    }
                }
            }
        };
        if (finite) code_all(std::true_type{});
        else code_all(std::false_type{});
    }
#pragma unroll
    for (int cc = 0; cc < 8; ++cc) {
        uint2 word = make_uint2(lo[cc], hi[cc]);
        *reinterpret_cast<uint2*>(tile + (cg * 8 + cc) * kQwStride + rg * 8) = word;
    }
    __syncthreads();

#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int c = t + q * 256;  // 1024 chunks of 16 bytes
        const int kl = c / 8, jc = c % 8;
        const int64_t k = k0 + kl;
        const int64_t j = j0 + jc * 16;
        if (k < N && j < K) {
            const uint8_t* src = tile + kl * kQwStride + jc * 16;
            uint2 a = *reinterpret_cast<const uint2*>(src);
            uint2 b = *reinterpret_cast<const uint2*>(src + 8);
            const uint4 v = make_uint4(a.x, a.y, b.x, b.y);
            if (stream_out) st16_stream(wq + k * K + j, v);  // uniform over the grid
            else *reinterpret_cast<uint4*>(wq + k * K + j) = v;
        }
    }
}

template <typename T, bool kScaled, bool kVec>
__global__ __launch_bounds__(256) void k_quant_weight(const T* __restrict__ w, int64_t K, int64_t N, int64_t ld,
                                                      const float* __restrict__ s,
                                                      const uint32_t* __restrict__ colmax,
                                                      int8_t* __restrict__ wq, float* __restrict__ w_scale,
                                                      int stream_out) {
    quant_weight_tile<T, kScaled, kVec>(blockIdx.x, w, K, N, ld, s, colmax, wq, w_scale, stream_out != 0);
}

// ---- activations -------------------------------------------------------------
//
// WPR wavefronts per token row (1 or 4); blocks of 256 threads hold 4 / WPR
// rows.  The row is kept in registers: a thread owns NV groups of 8
// consecutive channels (16-byte loads for bf16), smooths them with inv_s,
// reduces max|x'| across the wavefront with shuffles (and across the row's
// wavefronts through LDS), then codes and stores 8 bytes per group.
template <typename T, int NV, int WPR>
__global__ __launch_bounds__(256) void k_quant_act(const T* __restrict__ x, int64_t M, int64_t K, int64_t ld,
                                                   const float* __restrict__ inv_s, int mode,
                                                   int8_t* __restrict__ xq, float* __restrict__ x_scale,
                                                   uint32_t* __restrict__ gmax) {
    constexpr int kRowsPerBlock = 4 / WPR;
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    const int row_in_block = wave / WPR;
    const int t = (wave % WPR) * kWave + lane;
    const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + row_in_block;
    const bool valid = row < M;
    const int64_t groups = K / 8;

    float v[NV][8];
    float m = 0.0f;
#pragma unroll
    for (int q = 0; q < NV; ++q) {
        const int64_t g = t + (int64_t)q * (WPR * kWave);
        if (valid && g < groups) {
            load8(x + row * ld + g * 8, v[q]);
            if (inv_s) {
                const float4 a = *reinterpret_cast<const float4*>(inv_s + g * 8);
                const float4 b = *reinterpret_cast<const float4*>(inv_s + g * 8 + 4);
                v[q][0] = v[q][0] * a.x; v[q][1] = v[q][1] * a.y;
                v[q][2] = v[q][2] * a.z; v[q][3] = v[q][3] * a.w;
                v[q][4] = v[q][4] * b.x; v[q][5] = v[q][5] * b.y;
                v[q][6] = v[q][6] * b.z; v[q][7] = v[q][7] * b.w;
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(v[q][i]));
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) v[q][i] = 0.0f;
        }
    }

    __shared__ float red[4];
    if (mode == 1) {
        // Tensor-wide maximum: one atomic per block.
        m = wave_max(m);
        if (lane == 0) red[wave] = m;
        __syncthreads();
        if (threadIdx.x == 0) {
            const float bm = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
            // the running maximum only grows: when it already reaches bm the
            // atomic would change nothing (and thousands of blocks would queue
            // on one address)
            if (bm > 0.0f && __uint_as_float(__atomic_load_n(gmax, __ATOMIC_RELAXED)) < bm)
                atomicMax(gmax, __float_as_uint(bm));
        }
        return;
    }

    float a;
    if (mode == 2) {
        a = __uint_as_float(*gmax);
    } else {
        m = wave_max(m);
        if constexpr (WPR > 1) {
            if (lane == 0) red[wave] = m;
            __syncthreads();
            const int w0 = row_in_block * WPR;
            m = red[w0];
#pragma unroll
            for (int i = 1; i < WPR; ++i) m = fmaxf(m, red[w0 + i]);
        }
        a = m;
    }
    float scale, r;
    group_scale(a, scale, r);
    if (mode == 0) {
        if (valid && t == 0) x_scale[row] = scale;
    } else if (blockIdx.x == 0 && threadIdx.x == 0) {
        x_scale[0] = scale;
    }
    if (!valid) return;
    auto code_row = [&](auto fast) {
#pragma unroll
        for (int q = 0; q < NV; ++q) {
            const int64_t g = t + (int64_t)q * (WPR * kWave);
            if (g < groups) {
                int c[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) c[i] = decltype(fast)::value ? code8_finite(v[q][i], r) : code8(v[q][i], r);
                st8_stream(xq + row * K + g * 8, make_uint2(pack4(c[0], c[1], c[2], c[3]), pack4(c[4], c[5], c[6], c[7])));
            }
        }
    };
    if (r <= 3.402823466e38f) code_row(std::true_type{});
    else code_row(std::false_type{});
}

// One row's groups g = t + TPB q (q < NV) of bf16 x, 16 bytes each, as
// buffer loads over a descriptor of the row: offsets at or past the row's
// groups * 16 bytes (groups past the row end) and every offset of a row at or
// past M (the descriptor then holds 0 bytes) read as zero without touching
// memory.  So the loads carry no branch, and the compiler can wait for the
// current row alone (vmcnt(NV)) while the next row's loads stay in flight;
// loads under a per-lane branch would each end in a full wait.
template <int NV, int TPB>
__device__ __forceinline__ void load_row_groups(const bf16_t* __restrict__ x, int64_t row, int64_t M, int64_t ld,
                                                int groups, int t, uint4 (&d)[NV]) {
    const bool in = row < M;
    const __amdgpu_buffer_rsrc_t rs = row_rsrc(x + (in ? row : 0) * ld, in ? groups * 16 : 0);
#pragma unroll
    for (int q = 0; q < NV; ++q) d[q] = ld16_buf_stream(rs, (t + q * TPB) * 16);
}

// bf16 rows with per-token scales (mode 0) or a fixed per-tensor maximum
// (mode 2), K <= 16384: a block of 4 wavefronts walks rows blockIdx.x,
// blockIdx.x + gridDim.x, ...  Each thread owns the NV 8-channel groups
// t + 256 q of every row and keeps their inv_s in registers for all its rows
// (loaded once, instead of once per row); the next row's 16-byte loads are in
// flight while the current row is reduced (one barrier per row, LDS slots
// alternating between rows) and coded.  Codes and scales as k_quant_act.
template <int NV, bool kStatic, bool kKeepOut = false>
__device__ __forceinline__ void quant_act_stream_rows(int64_t bid, int64_t nblk, const bf16_t* __restrict__ x,
                                                     int64_t M, int64_t K, int64_t ld,
                                                     const float* __restrict__ inv_s, int8_t* __restrict__ xq,
                                                     float* __restrict__ x_scale,
                                                     const uint32_t* __restrict__ gmax) {
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave, t = threadIdx.x;
    const int64_t groups = K / 8;
    float is[NV][8];
#pragma unroll
    for (int q = 0; q < NV; ++q) {
        const int64_t g = t + (int64_t)q * 256;
        if (inv_s && g < groups) {
            const float4 a = *reinterpret_cast<const float4*>(inv_s + g * 8);
            const float4 b = *reinterpret_cast<const float4*>(inv_s + g * 8 + 4);
            is[q][0] = a.x; is[q][1] = a.y; is[q][2] = a.z; is[q][3] = a.w;
            is[q][4] = b.x; is[q][5] = b.y; is[q][6] = b.z; is[q][7] = b.w;
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) is[q][i] = 1.0f;  // fl(x * 1) = x
        }
    }
    float scale = 0.0f, r = 0.0f;
    if constexpr (kStatic) {
        group_scale(__uint_as_float(*gmax), scale, r);
        if (bid == 0 && t == 0) x_scale[0] = scale;
    }
    __shared__ float red[2][4];
    // one row of codes from its loaded groups d; `slot` picks the LDS slots
    // (alternating between consecutive rows of the block)
    auto row_codes = [&](int64_t row, const uint4 (&d)[NV], int slot) {
        float v[NV][8];
        float m = 0.0f;
#pragma unroll
        for (int q = 0; q < NV; ++q) {
            const uint32_t u[4] = {d[q].x, d[q].y, d[q].z, d[q].w};
#pragma unroll
            for (int h = 0; h < 4; ++h) {
                v[q][2 * h] = bf16_lo(u[h]) * is[q][2 * h];
                v[q][2 * h + 1] = bf16_hi(u[h]) * is[q][2 * h + 1];
            }
            if constexpr (!kStatic) {
#pragma unroll
                for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(v[q][i]));
            }
        }
        if constexpr (!kStatic) {
            m = wave_max(m);
            if (lane == 0) red[slot][wave] = m;
            __syncthreads();
            m = fmaxf(fmaxf(red[slot][0], red[slot][1]), fmaxf(red[slot][2], red[slot][3]));
            group_scale(m, scale, r);
            if (t == 0) x_scale[row] = scale;
        }
        auto code_row = [&](auto fast) {
#pragma unroll
            for (int q = 0; q < NV; ++q) {
                const int64_t g = t + (int64_t)q * 256;
                if (g < groups) {
                    uint2 pk;
                    if constexpr (!kStatic && decltype(fast)::value) {
                        // the row's own max bounds every value: no clamp
                        uint32_t c[8];
#pragma unroll
                        for (int i = 0; i < 8; ++i) c[i] = code8_bounded_bits(v[q][i], r);
                        pk = make_uint2(pack4_low(c[0], c[1], c[2], c[3]), pack4_low(c[4], c[5], c[6], c[7]));
                    } else {
                        int c[8];
#pragma unroll
                        for (int i = 0; i < 8; ++i)
                            c[i] = decltype(fast)::value ? code8_finite(v[q][i], r) : code8(v[q][i], r);
                        pk = make_uint2(pack4(c[0], c[1], c[2], c[3]), pack4(c[4], c[5], c[6], c[7]));
                    }
                    if constexpr (kKeepOut) *reinterpret_cast<uint2*>(xq + row * K + g * 8) = pk;
                    else st8_stream(xq + row * K + g * 8, pk);
                }
            }
        };
        if (r <= 3.402823466e38f) code_row(std::true_type{});
        else code_row(std::false_type{});
    };
    // two rows per iteration with two load buffers: the loads of one row are
    // in flight while the other is coded, and no register copy between
    // iterations waits for them
    uint4 da[NV], db[NV];
    int64_t row = bid;
    if (row < M) load_row_groups<NV, 256>(x, row, M, ld, (int)groups, t, da);
    for (; row < M; row += 2 * nblk) {
        load_row_groups<NV, 256>(x, row + nblk, M, ld, (int)groups, t, db);
        row_codes(row, da, 0);
        if (row + nblk >= M) break;
        load_row_groups<NV, 256>(x, row + 2 * nblk, M, ld, (int)groups, t, da);
        row_codes(row + nblk, db, 1);
    }
}

template <int NV, bool kStatic>
__global__ __launch_bounds__(256) void k_quant_act_stream(const bf16_t* __restrict__ x, int64_t M, int64_t K,
                                                          int64_t ld, const float* __restrict__ inv_s,
                                                          int8_t* __restrict__ xq, float* __restrict__ x_scale,
                                                          const uint32_t* __restrict__ gmax) {
    quant_act_stream_rows<NV, kStatic>(blockIdx.x, gridDim.x, x, M, K, ld, inv_s, xq, x_scale, gmax);
}

// Step 3's codes and step 4's per-token codes in one launch: both need only
// s / inv_s and the column maxima, and each alone leaves the memory system
// idle during its start and tail at attention-projection sizes.  Blocks
// [0, tiles) code 128 x 128 weight tiles (bf16, 16-byte aligned rows), the
// others walk token rows with the block count as their stride.  kKeepOut:
// the activation codes leave as plain stores, so the GEMM that reads them
// next finds them in the caches (nontemporal stores otherwise).
template <int NV, bool kKeepOut>
__global__ __launch_bounds__(256) void k_codes_both(const bf16_t* __restrict__ w, int64_t K, int64_t N, int64_t ldw,
                                                    const float* __restrict__ s,
                                                    const uint32_t* __restrict__ colmax, int8_t* __restrict__ wq,
                                                    float* __restrict__ w_scale, int64_t tiles,
                                                    const bf16_t* __restrict__ x, int64_t M, int64_t ldx,
                                                    const float* __restrict__ inv_s, int8_t* __restrict__ xq,
                                                    float* __restrict__ x_scale, int w_stream) {
    if ((int64_t)blockIdx.x < tiles)
        quant_weight_tile<bf16_t, true, true>(blockIdx.x, w, K, N, ldw, s, colmax, wq, w_scale, w_stream != 0);
    else
        quant_act_stream_rows<NV, false, kKeepOut>((int64_t)blockIdx.x - tiles, (int64_t)gridDim.x - tiles, x, M, K,
                                                   ldx, inv_s, xq, x_scale, nullptr);
}

// The per-tensor maximum a = max_ij |fl(x_ij inv_s_j)| (the first of the two
// passes of dynamic per-tensor step 4): blocks walk token rows with a grid
// stride, two rows' loads in flight, each thread keeps the inv_s of its
// channel groups in registers and one running maximum; one atomicMax per
// block on the fp32 bit pattern (*gmax starts at 0).  keep: plain loads, so
// the codes pass that reads x again finds much of it in the caches (the
// 256 MB memory-side cache above all); nontemporal loads otherwise.
template <int NV>
__global__ __launch_bounds__(256) void k_act_absmax_stream(const bf16_t* __restrict__ x, int64_t M, int64_t K,
                                                           int64_t ld, const float* __restrict__ inv_s,
                                                           uint32_t* __restrict__ gmax, int keep) {
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave, t = threadIdx.x;
    const int64_t groups = K / 8;
    float is[NV][8];
#pragma unroll
    for (int q = 0; q < NV; ++q) {
        const int64_t g = t + (int64_t)q * 256;
        if (inv_s && g < groups) {
            const float4 a = *reinterpret_cast<const float4*>(inv_s + g * 8);
            const float4 b = *reinterpret_cast<const float4*>(inv_s + g * 8 + 4);
            is[q][0] = a.x; is[q][1] = a.y; is[q][2] = a.z; is[q][3] = a.w;
            is[q][4] = b.x; is[q][5] = b.y; is[q][6] = b.z; is[q][7] = b.w;
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) is[q][i] = 1.0f;
        }
    }
    float m = 0.0f;
    const int64_t stride = gridDim.x;
    for (int64_t row = blockIdx.x; row < M; row += 2 * stride) {
        uint4 u[2][NV];
#pragma unroll
        for (int r = 0; r < 2; ++r)
#pragma unroll
            for (int q = 0; q < NV; ++q) {
                const int64_t rr = row + r * stride, g = t + (int64_t)q * 256;
                const bf16_t* p = x + rr * ld + g * 8;
                u[r][q] = (rr < M && g < groups) ? (keep ? ld16(p) : ld16_stream(p)) : make_uint4(0, 0, 0, 0);
            }
#pragma unroll
        for (int r = 0; r < 2; ++r)
#pragma unroll
            for (int q = 0; q < NV; ++q) {
                const uint32_t w[4] = {u[r][q].x, u[r][q].y, u[r][q].z, u[r][q].w};
#pragma unroll
                for (int h = 0; h < 4; ++h) {
                    m = fmaxf(m, fabsf(bf16_lo(w[h]) * is[q][2 * h]));
                    m = fmaxf(m, fabsf(bf16_hi(w[h]) * is[q][2 * h + 1]));
                }
            }
    }
    __shared__ float red[4];
    m = wave_max(m);
    if (lane == 0) red[wave] = m;
    __syncthreads();
    if (t == 0) {
        m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
        if (m > 0.0f) atomicMax(gmax, __float_as_uint(m));
    }
}

// Rows longer than the register-resident variants hold (K > 16384): four
// wavefronts per row loop over it twice, once for the max, once for codes
// (the second pass re-reads the row, mostly from L2).
template <typename T>
__global__ __launch_bounds__(256) void k_quant_act_long(const T* __restrict__ x, int64_t M, int64_t K,
                                                        int64_t ld, const float* __restrict__ inv_s, int mode,
                                                        int8_t* __restrict__ xq, float* __restrict__ x_scale,
                                                        uint32_t* __restrict__ gmax) {
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    const int64_t row = blockIdx.x;
    const int64_t groups = K / 8;
    const T* xr = x + row * ld;
    __shared__ float red[4];
    float m = 0.0f;
    if (mode != 2) {
        for (int64_t g = threadIdx.x; g < groups; g += 256) {
            float v[8];
            load8(xr + g * 8, v);
#pragma unroll
            for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(inv_s ? v[i] * inv_s[g * 8 + i] : v[i]));
        }
        m = wave_max(m);
        if (lane == 0) red[wave] = m;
        __syncthreads();
        m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
        if (mode == 1) {
            if (threadIdx.x == 0 && m > 0.0f && __uint_as_float(__atomic_load_n(gmax, __ATOMIC_RELAXED)) < m)
                atomicMax(gmax, __float_as_uint(m));
            return;
        }
    }
    const float a = mode == 2 ? __uint_as_float(*gmax) : m;
    float scale, r;
    group_scale(a, scale, r);
    if (threadIdx.x == 0) {
        if (mode == 0) x_scale[row] = scale;
        else if (row == 0) x_scale[0] = scale;
    }
    for (int64_t g = threadIdx.x; g < groups; g += 256) {
        float v[8];
        load8(xr + g * 8, v);
        if (inv_s) {
#pragma unroll
            for (int i = 0; i < 8; ++i) v[i] = v[i] * inv_s[g * 8 + i];
        }
        uint2 word;
        word.x = pack4(code8(v[0], r), code8(v[1], r), code8(v[2], r), code8(v[3], r));
        word.y = pack4(code8(v[4], r), code8(v[5], r), code8(v[6], r), code8(v[7], r));
        *reinterpret_cast<uint2*>(xq + row * K + g * 8) = word;
    }
}

// ---- launchers -----------------------------------------------------------------

// A weight tile's 128 rows of stride ld fit the 31-bit byte range of one
// buffer descriptor.
static bool qw_rows_addressable(int64_t ld, int64_t elem_bytes) {
    return ld > 0 && (int64_t)kQwTile * ld * elem_bytes < ((int64_t)1 << 31) - 64;
}

// Weight codes beyond 64 MB leave as nontemporal stores; smaller ones stay
// cacheable for the GEMM that reads them next.
static int weight_codes_stream(int64_t K, int64_t N) { return (uint64_t)K * (uint64_t)N > (64ull << 20) ? 1 : 0; }

hipError_t launch_quant_weight(const void* w, bool bf16, int64_t K, int64_t N, int64_t ld, const float* s,
                               const uint32_t* colmax, int8_t* wq, float* w_scale, hipStream_t st) {
    if (K <= 0 || N <= 0) return hipSuccess;
    const int64_t tiles = ((N + kQwTile - 1) / kQwTile) * ((K + kQwTile - 1) / kQwTile);
    if (tiles > 0x7FFFFFFF) return hipErrorInvalidValue;  // beyond 2^45 weights: not addressable in one grid
    dim3 grid((unsigned)tiles);
    const int w_stream = weight_codes_stream(K, N);
    // the 16-byte path addresses a tile's 128 rows through one buffer
    // descriptor (32-bit byte offsets)
    const bool vec = rows_aligned16(w, ld, bf16 ? 2 : 4) && qw_rows_addressable(ld, bf16 ? 2 : 4);
    auto go = [&](auto tag, auto scaled, auto vecc) {
        using T = decltype(tag);
        hipLaunchKernelGGL((k_quant_weight<T, decltype(scaled)::value, decltype(vecc)::value>), grid, dim3(256), 0,
                           st, static_cast<const T*>(w), K, N, ld, s, colmax, wq, w_scale, w_stream);
    };
    using TT = std::true_type;
    using FF = std::false_type;
    if (bf16) {
        if (s) { if (vec) go(bf16_t{}, TT{}, TT{}); else go(bf16_t{}, TT{}, FF{}); }
        else { if (vec) go(bf16_t{}, FF{}, TT{}); else go(bf16_t{}, FF{}, FF{}); }
    } else {
        if (s) { if (vec) go(float{}, TT{}, TT{}); else go(float{}, TT{}, FF{}); }
        else { if (vec) go(float{}, FF{}, TT{}); else go(float{}, FF{}, FF{}); }
    }
    return hipGetLastError();
}

// ---- fused LayerNorm + per-token codes (the runtime half of the LN fold) ----------
//
// The statistics use a fixed-point grid so no reduction order can change
// them: with 2^E the power of two just above the row's largest magnitude,
// x_j is truncated toward zero to a multiple of 2^(E-39) and x_j^2 to a
// multiple of 2^(2E-39); the truncated values are integers in units of the
// grid, and with K <= 16384 every partial sum stays below 2^53, so fp64 adds
// them exactly in any order.  Then mu = S1 2^(E-39) / K,
// var = max(S2 2^(2E-39) / K - mu^2, 0), rstd = 1 / sqrt(var + eps) in fp64,
// each rounded once to fp32; element j in fp32: n = fl(fl(x_j - mu) rstd),
// z = fl(fl(n g_j) + b_j) with the folded LayerNorm weight g and bias b; then
// the row's max |z|, scale and codes as in step 4.
//
// The grid terms are formed in fp32: a = x 2^(39-E) is exact, and so is
// p = a (x 2^-E) = x^2 2^(39-2E) whenever p >= 1 (both factors are then
// normal and the product has at most 16 significant bits); a smaller p
// truncates to 0 whatever its rounding.  Only the sums run in fp64.

// One token row per TPB threads (TPB / 64 wavefronts), rows walked with a
// grid stride; TEAMS teams of TPB threads per block each take their own rows
// (the team's first row is blockIdx.x * TEAMS + team, its stride
// gridDim.x * TEAMS).  Thread t of a team owns the 8-channel groups
// t + TPB q (q < NV) of every row.  The folded gamma (and beta) of those
// groups stay in the thread's registers for all its rows when TEAMS == 1;
// with TEAMS > 1 they sit in LDS once for the whole block (two planes of
// float4 per group, channels 0-3 then 4-7, so a wavefront's reads of
// consecutive groups are consecutive 16-byte slots) and the registers they
// free let more wavefronts per SIMD hide each other's latency.  Rows go
// through two load buffers, so one row's loads are in flight while the other
// is reduced, normalised and coded.  Three reductions per row (max |x|, the
// two grid sums, max |z|) cross the team's wavefronts through LDS slots that
// alternate between rows, one barrier each; the teams take those barriers
// together, so every team runs the same number of rows and a team whose row
// lies past M computes on zeros and stores nothing.
template <int NV, int TPB, int TEAMS, bool kBeta>
__global__ __launch_bounds__(TPB * TEAMS) void k_ln_quant(const bf16_t* __restrict__ x, int64_t M, int64_t K,
                                                          int64_t ld, const float* __restrict__ gamma,
                                                          const float* __restrict__ beta, float eps,
                                                          int8_t* __restrict__ xq, float* __restrict__ x_scale) {
    constexpr int W = TPB / kWave, NT = TPB * TEAMS;
    constexpr bool kLdsGB = TEAMS > 1;
    constexpr int CAP = NV * TPB;  // groups the LDS planes hold
    const int team = TEAMS > 1 ? (int)threadIdx.x / TPB : 0;
    const int t = TEAMS > 1 ? (int)threadIdx.x % TPB : (int)threadIdx.x;
    const int wave = t / kWave, lane = t % kWave, w0 = team * W;
    const int groups = (int)(K / 8);
    __shared__ float4 gl[kLdsGB ? 2 * CAP : 1];
    __shared__ float4 bl[kLdsGB && kBeta ? 2 * CAP : 1];
    __shared__ float red_x[2][TEAMS * W], red_z[2][TEAMS * W];
    __shared__ double red_1[2][TEAMS * W], red_2[2][TEAMS * W];
    // groups past the row end (last q only) take the last group's gamma/beta;
    // their x is zero and they are left out of the max and the stores
    float gr[kLdsGB ? 1 : NV][8], br[kLdsGB ? 1 : NV][8];
    if constexpr (kLdsGB) {
        for (int i = threadIdx.x; i < 2 * groups; i += NT) {
            gl[(i & 1) * CAP + (i >> 1)] = reinterpret_cast<const float4*>(gamma)[i];  // channels 8g + 4h .. + 3
            if constexpr (kBeta) bl[(i & 1) * CAP + (i >> 1)] = reinterpret_cast<const float4*>(beta)[i];
        }
        __syncthreads();
    } else {
#pragma unroll
        for (int q = 0; q < NV; ++q) {
            const int g = t + q * TPB;
            const int64_t gc = (q < NV - 1 || g < groups) ? g : groups - 1;
            const float4 a = *reinterpret_cast<const float4*>(gamma + gc * 8);
            const float4 b = *reinterpret_cast<const float4*>(gamma + gc * 8 + 4);
            gr[q][0] = a.x; gr[q][1] = a.y; gr[q][2] = a.z; gr[q][3] = a.w;
            gr[q][4] = b.x; gr[q][5] = b.y; gr[q][6] = b.z; gr[q][7] = b.w;
            if constexpr (kBeta) {
                const float4 c = *reinterpret_cast<const float4*>(beta + gc * 8);
                const float4 d = *reinterpret_cast<const float4*>(beta + gc * 8 + 4);
                br[q][0] = c.x; br[q][1] = c.y; br[q][2] = c.z; br[q][3] = c.w;
                br[q][4] = d.x; br[q][5] = d.y; br[q][6] = d.z; br[q][7] = d.w;
            }
        }
    }
    auto row_codes = [&](int64_t row, const uint4 (&cur)[NV], int b) {
        float v[NV][8];
        float xm = 0.0f;
#pragma unroll
        for (int q = 0; q < NV; ++q) {
            const uint32_t u[4] = {cur[q].x, cur[q].y, cur[q].z, cur[q].w};
#pragma unroll
            for (int h = 0; h < 4; ++h) {
                v[q][2 * h] = bf16_lo(u[h]);
                v[q][2 * h + 1] = bf16_hi(u[h]);
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) xm = fmaxf(xm, fabsf(v[q][i]));
        }
        xm = wave_max(xm);
        if constexpr (W > 1 || TEAMS > 1) {
            if (lane == 0) red_x[b][w0 + wave] = xm;
            __syncthreads();
            xm = red_x[b][w0];
#pragma unroll
            for (int i = 1; i < W; ++i) xm = fmaxf(xm, red_x[b][w0 + i]);
        }
        int E = 0;
        frexpf(xm, &E);
        // ldexpf scales exactly over the whole range (a constant 2^(39-E) could overflow)
        double s1 = 0.0, s2 = 0.0;
#pragma unroll
        for (int q = 0; q < NV; ++q)
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float a = ldexpf(v[q][i], 39 - E);
                s1 += (double)truncf(a);
                s2 += (double)truncf(a * ldexpf(v[q][i], -E));
            }
        s1 = wave_sum_f64(s1);
        s2 = wave_sum_f64(s2);
        if constexpr (W > 1 || TEAMS > 1) {
            if (lane == 0) {
                red_1[b][w0 + wave] = s1;
                red_2[b][w0 + wave] = s2;
            }
            __syncthreads();
            s1 = red_1[b][w0];
            s2 = red_2[b][w0];
#pragma unroll
            for (int i = 1; i < W; ++i) {
                s1 += red_1[b][w0 + i];
                s2 += red_2[b][w0 + i];
            }
        }
        double mu = 0.0, var = 0.0;
        if (xm > 0.0f) {
            mu = ldexp(s1, E - 39) / (double)K;
            var = ldexp(s2, 2 * E - 39) / (double)K - mu * mu;
            if (var < 0.0) var = 0.0;
        }
        const float mu32 = (float)mu, rstd32 = (float)(1.0 / sqrt(var + (double)eps));
        float m = 0.0f;
#pragma unroll
        for (int q = 0; q < NV; ++q) {
            const int g = t + q * TPB;
            const bool in = q < NV - 1 || g < groups;
            float gw[8] = {0, 0, 0, 0, 0, 0, 0, 0}, bw[8] = {0, 0, 0, 0, 0, 0, 0, 0};
            if constexpr (kLdsGB) {
                const int gc = in ? g : groups - 1;
                const float4 ga = gl[gc], gb = gl[CAP + gc];
                gw[0] = ga.x; gw[1] = ga.y; gw[2] = ga.z; gw[3] = ga.w;
                gw[4] = gb.x; gw[5] = gb.y; gw[6] = gb.z; gw[7] = gb.w;
                if constexpr (kBeta) {
                    const float4 ba = bl[gc], bb = bl[CAP + gc];
                    bw[0] = ba.x; bw[1] = ba.y; bw[2] = ba.z; bw[3] = ba.w;
                    bw[4] = bb.x; bw[5] = bb.y; bw[6] = bb.z; bw[7] = bb.w;
                }
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float n = (v[q][i] - mu32) * rstd32;
                const float tt = n * (kLdsGB ? gw[i] : gr[kLdsGB ? 0 : q][i]);
                v[q][i] = kBeta ? tt + (kLdsGB ? bw[i] : br[kLdsGB ? 0 : q][i]) : tt;
                m = fmaxf(m, in ? fabsf(v[q][i]) : 0.0f);
            }
        }
        m = wave_max(m);
        if constexpr (W > 1 || TEAMS > 1) {
            if (lane == 0) red_z[b][w0 + wave] = m;
            __syncthreads();
            m = red_z[b][w0];
#pragma unroll
            for (int i = 1; i < W; ++i) m = fmaxf(m, red_z[b][w0 + i]);
        }
        if (TEAMS > 1 && row >= M) return;  // a team past the last row: nothing to store
        float scale, r;
        group_scale(m, scale, r);
        if (t == 0) x_scale[row] = scale;
        auto code_row = [&](auto fast) {
#pragma unroll
            for (int q = 0; q < NV; ++q) {
                const int g = t + q * TPB;
                if (q < NV - 1 || g < groups) {
                    uint2 pk;
                    if constexpr (decltype(fast)::value) {
                        // m is the max of these values: no clamp
                        uint32_t c[8];
#pragma unroll
                        for (int i = 0; i < 8; ++i) c[i] = code8_bounded_bits(v[q][i], r);
                        pk = make_uint2(pack4_low(c[0], c[1], c[2], c[3]), pack4_low(c[4], c[5], c[6], c[7]));
                    } else {
                        int c[8];
#pragma unroll
                        for (int i = 0; i < 8; ++i) c[i] = code8(v[q][i], r);
                        pk = make_uint2(pack4(c[0], c[1], c[2], c[3]), pack4(c[4], c[5], c[6], c[7]));
                    }
                    st8_stream(xq + row * K + (int64_t)g * 8, pk);
                }
            }
        };
        if (r <= 3.402823466e38f) code_row(std::true_type{});
        else code_row(std::false_type{});
    };
    // rows base + team, base stepping by the grid's share; two rows per
    // iteration with two load buffers (no register copy between iterations
    // that would wait for the loads in flight); the loop bounds are the same
    // for every team
    const int64_t stride = (int64_t)gridDim.x * TEAMS;
    uint4 da[NV], db[NV];
    int64_t base = (int64_t)blockIdx.x * TEAMS;
    if (base < M) load_row_groups<NV, TPB>(x, base + team, M, ld, groups, t, da);
    for (; base < M; base += 2 * stride) {
        load_row_groups<NV, TPB>(x, base + stride + team, M, ld, groups, t, db);
        row_codes(base + team, da, 0);
        if (base + stride >= M) break;
        load_row_groups<NV, TPB>(x, base + 2 * stride + team, M, ld, groups, t, da);
        row_codes(base + stride + team, db, 1);
    }
}

template <typename T, int NV, int WPR>
static void launch_act_rows(const T* x, int64_t M, int64_t K, int64_t ld, const float* inv_s, int mode, int8_t* xq,
                            float* x_scale, uint32_t* gmax, hipStream_t st) {
    constexpr int rpb = 4 / WPR;
    const int64_t blocks = (M + rpb - 1) / rpb;
    hipLaunchKernelGGL((k_quant_act<T, NV, WPR>), dim3((unsigned)blocks), dim3(256), 0, st, x, M, K, ld, inv_s,
                       mode, xq, x_scale, gmax);
}

// Blocks per CU of k_quant_act_stream (measured best grids: about the
// resident count for one group per thread; for two groups 4 blocks, each with
// twice the rows to amortise its inv_s load: 13.5 vs 13.9 us at 4096x4096;
// fewer for the wider rows).
static int act_stream_blocks_per_cu(int nv) { return nv <= 1 ? 8 : nv <= 2 ? 4 : nv <= 6 ? 3 : 2; }

template <int NV>
static void launch_act_stream_nv(const bf16_t* x, int64_t M, int64_t K, int64_t ld, const float* inv_s, int mode,
                                 int8_t* xq, float* x_scale, const uint32_t* gmax, hipStream_t st) {
    int cus = 0, dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) !=
                                                 hipSuccess || cus <= 0)
        cus = 256;
    const int64_t grid = std::min<int64_t>(M, (int64_t)cus * act_stream_blocks_per_cu(NV));
    if (mode == 2)
        hipLaunchKernelGGL((k_quant_act_stream<NV, true>), dim3((unsigned)grid), dim3(256), 0, st, x, M, K, ld, inv_s,
                           xq, x_scale, gmax);
    else
        hipLaunchKernelGGL((k_quant_act_stream<NV, false>), dim3((unsigned)grid), dim3(256), 0, st, x, M, K, ld,
                           inv_s, xq, x_scale, gmax);
}

static void launch_act_stream(const bf16_t* x, int64_t M, int64_t K, int64_t ld, const float* inv_s, int mode,
                              int8_t* xq, float* x_scale, const uint32_t* gmax, hipStream_t st) {
    switch ((K / 8 + 255) / 256) {
        case 1: return launch_act_stream_nv<1>(x, M, K, ld, inv_s, mode, xq, x_scale, gmax, st);
        case 2: return launch_act_stream_nv<2>(x, M, K, ld, inv_s, mode, xq, x_scale, gmax, st);
        case 3: return launch_act_stream_nv<3>(x, M, K, ld, inv_s, mode, xq, x_scale, gmax, st);
        case 4: return launch_act_stream_nv<4>(x, M, K, ld, inv_s, mode, xq, x_scale, gmax, st);
        case 5: return launch_act_stream_nv<5>(x, M, K, ld, inv_s, mode, xq, x_scale, gmax, st);
        case 6: return launch_act_stream_nv<6>(x, M, K, ld, inv_s, mode, xq, x_scale, gmax, st);
        case 7: return launch_act_stream_nv<7>(x, M, K, ld, inv_s, mode, xq, x_scale, gmax, st);
        default: return launch_act_stream_nv<8>(x, M, K, ld, inv_s, mode, xq, x_scale, gmax, st);
    }
}

// Grid for the max pass: about four blocks per CU (the register footprint
// allows it for every NV), each walking about M / grid rows.
static void launch_act_absmax_stream(const bf16_t* x, int64_t M, int64_t K, int64_t ld, const float* inv_s,
                                     uint32_t* gmax, hipStream_t st) {
    int cus = 0, dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) !=
                                                 hipSuccess || cus <= 0)
        cus = 256;
    const int64_t grid = std::min<int64_t>(M, (int64_t)cus * 4);
    const dim3 g((unsigned)grid);
    // x of up to 256 MB: 8 % off the two-pass per-tensor codes at 8192x12288
    const int keep = (uint64_t)M * (uint64_t)ld * 2u <= (256ull << 20) ? 1 : 0;
    switch ((K / 8 + 255) / 256) {
        case 1: hipLaunchKernelGGL((k_act_absmax_stream<1>), g, dim3(256), 0, st, x, M, K, ld, inv_s, gmax, keep); break;
        case 2: hipLaunchKernelGGL((k_act_absmax_stream<2>), g, dim3(256), 0, st, x, M, K, ld, inv_s, gmax, keep); break;
        case 3: hipLaunchKernelGGL((k_act_absmax_stream<3>), g, dim3(256), 0, st, x, M, K, ld, inv_s, gmax, keep); break;
        case 4: hipLaunchKernelGGL((k_act_absmax_stream<4>), g, dim3(256), 0, st, x, M, K, ld, inv_s, gmax, keep); break;
        case 5: hipLaunchKernelGGL((k_act_absmax_stream<5>), g, dim3(256), 0, st, x, M, K, ld, inv_s, gmax, keep); break;
        case 6: hipLaunchKernelGGL((k_act_absmax_stream<6>), g, dim3(256), 0, st, x, M, K, ld, inv_s, gmax, keep); break;
        case 7: hipLaunchKernelGGL((k_act_absmax_stream<7>), g, dim3(256), 0, st, x, M, K, ld, inv_s, gmax, keep); break;
        default: hipLaunchKernelGGL((k_act_absmax_stream<8>), g, dim3(256), 0, st, x, M, K, ld, inv_s, gmax, keep); break;
    }
}

template <typename T>
static void dispatch_act(const T* x, int64_t M, int64_t K, int64_t ld, const float* inv_s, int mode, int8_t* xq,
                         float* x_scale, uint32_t* gmax, hipStream_t st) {
    const int64_t groups = K / 8;
    if constexpr (std::is_same<T, bf16_t>::value) {
        if (groups <= 8 * 256 && rows_aligned16(x, ld, 2)) {
            if (mode == 1) return launch_act_absmax_stream(x, M, K, ld, inv_s, gmax, st);
            return launch_act_stream(x, M, K, ld, inv_s, mode, xq, x_scale, gmax, st);
        }
    }
    if (groups <= 1 * kWave) return launch_act_rows<T, 1, 1>(x, M, K, ld, inv_s, mode, xq, x_scale, gmax, st);
    if (groups <= 2 * kWave) return launch_act_rows<T, 2, 1>(x, M, K, ld, inv_s, mode, xq, x_scale, gmax, st);
    if (groups <= 4 * kWave) return launch_act_rows<T, 4, 1>(x, M, K, ld, inv_s, mode, xq, x_scale, gmax, st);
    if (groups <= 8 * kWave) return launch_act_rows<T, 8, 1>(x, M, K, ld, inv_s, mode, xq, x_scale, gmax, st);
    if (groups <= 4 * 4 * kWave) return launch_act_rows<T, 4, 4>(x, M, K, ld, inv_s, mode, xq, x_scale, gmax, st);
    if (groups <= 6 * 4 * kWave) return launch_act_rows<T, 6, 4>(x, M, K, ld, inv_s, mode, xq, x_scale, gmax, st);
    if (groups <= 8 * 4 * kWave) return launch_act_rows<T, 8, 4>(x, M, K, ld, inv_s, mode, xq, x_scale, gmax, st);
    hipLaunchKernelGGL((k_quant_act_long<T>), dim3((unsigned)M), dim3(256), 0, st, x, M, K, ld, inv_s, mode, xq,
                       x_scale, gmax);
}

hipError_t launch_codes_both(const void* w, int64_t K, int64_t N, int64_t ldw, const float* s, const uint32_t* colmax,
                             int8_t* wq, float* w_scale, const void* x, int64_t M, int64_t ldx, const float* inv_s,
                             int8_t* xq, float* x_scale, hipStream_t st) {
    if (K <= 0 || N <= 0 || M <= 0 || !s || !inv_s) return hipErrorNotSupported;
    const int64_t groups = K / 8;
    if (K % 8 != 0 || groups > 2 * 256 || !rows_aligned16(w, ldw, 2) || !rows_aligned16(x, ldx, 2) ||
        !qw_rows_addressable(ldw, 2))
        return hipErrorNotSupported;
    const int64_t tiles = ((N + kQwTile - 1) / kQwTile) * ((K + kQwTile - 1) / kQwTile);
    int cus = 0, dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) !=
                                                 hipSuccess || cus <= 0)
        cus = 256;
    const int64_t rows = std::min<int64_t>(M, (int64_t)cus * 8);  // 8 row blocks per CU beside the tiles
    if (tiles + rows > 0x7FFFFFFF) return hipErrorNotSupported;
    const dim3 grid((unsigned)(tiles + rows));
    const bf16_t* wb = static_cast<const bf16_t*>(w);
    const bf16_t* xb = static_cast<const bf16_t*>(x);
    // activation codes of up to 64 MB stay cacheable for the GEMM: 0.9 us off
    // the 2048x4096x4096 GEMM that follows
    const bool keep = (uint64_t)M * (uint64_t)K <= (64ull << 20);
    auto go = [&](auto nv, auto kp) {
        hipLaunchKernelGGL((k_codes_both<decltype(nv)::value, decltype(kp)::value>), grid, dim3(256), 0, st, wb, K, N,
                           ldw, s, colmax, wq, w_scale, tiles, xb, M, ldx, inv_s, xq, x_scale, weight_codes_stream(K, N));
    };
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    if (groups <= 256) { if (keep) go(I1{}, std::true_type{}); else go(I1{}, std::false_type{}); }
    else { if (keep) go(I2{}, std::true_type{}); else go(I2{}, std::false_type{}); }
    return hipGetLastError();
}

// Blocks per CU of k_ln_quant<NV, TPB, 1, *>: what its register footprint
// lets reside at once (the grid walks all rows with that many blocks).
static int ln_blocks_per_cu(int nv, int tpb) {
    const int waves_per_simd = nv <= 1 ? 8 : nv <= 2 ? 5 : nv <= 4 ? 3 : 2;
    return std::max(1, waves_per_simd * 4 / (tpb / kWave));
}

// TEAMS == 1: the resident blocks per CU; TEAMS > 1: one block per CU (its
// LDS holds gamma and beta), at most ceil(M / TEAMS) blocks.
template <int NV, int TPB, int TEAMS>
static hipError_t launch_ln_rows(const bf16_t* x, int64_t M, int64_t K, int64_t ld, const float* gamma,
                                 const float* beta, float eps, int8_t* xq, float* x_scale, hipStream_t st) {
    // the kernel reads groups t + TPB q unchecked for q < NV - 1
    const int64_t groups = K / 8;
    if (groups <= (int64_t)(NV - 1) * TPB || groups > (int64_t)NV * TPB) return hipErrorInvalidValue;
    int cus = 0, dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) !=
                                                 hipSuccess || cus <= 0)
        cus = 256;
    const int64_t per_cu = TEAMS > 1 ? 1 : ln_blocks_per_cu(NV, TPB);
    const dim3 grid((unsigned)std::min<int64_t>((M + TEAMS - 1) / TEAMS, (int64_t)cus * per_cu));
    if (beta)
        hipLaunchKernelGGL((k_ln_quant<NV, TPB, TEAMS, true>), grid, dim3(TPB * TEAMS), 0, st, x, M, K, ld, gamma,
                           beta, eps, xq, x_scale);
    else
        hipLaunchKernelGGL((k_ln_quant<NV, TPB, TEAMS, false>), grid, dim3(TPB * TEAMS), 0, st, x, M, K, ld, gamma,
                           beta, eps, xq, x_scale);
    return hipGetLastError();
}

// Threads per row grow with K so that each thread keeps at most 6 groups
// (48 channels, with their gamma and beta) in registers up to 12288
// channels; NV is always ceil(groups / TPB).
hipError_t launch_ln_quant(const void* x, int64_t M, int64_t K, int64_t ld, const float* gamma, const float* beta,
                           float eps, int8_t* xq, float* x_scale, hipStream_t st) {
    if (M <= 0) return hipSuccess;
    const bf16_t* xb = static_cast<const bf16_t*>(x);
    const int64_t groups = K / 8;
#define SQ_LN(NV, TPB, TEAMS) \
    return launch_ln_rows<NV, TPB, TEAMS>(xb, M, K, ld, gamma, beta, eps, xq, x_scale, st)
    if (groups <= 64) SQ_LN(1, 64, 1);
    if (groups <= 128) SQ_LN(2, 64, 1);
    if (groups <= 192) SQ_LN(3, 64, 1);
    if (groups <= 256) SQ_LN(4, 64, 1);
    if (groups <= 384) SQ_LN(3, 128, 1);
    if (groups <= 512) SQ_LN(4, 128, 1);
    if (groups <= 768) SQ_LN(3, 256, 1);
    if (groups <= 1024) SQ_LN(4, 256, 1);
    if (groups <= 1280) SQ_LN(5, 256, 1);
    if (groups <= 1536) SQ_LN(6, 256, 1);
    // beyond 12288 channels two teams of 512 threads share gamma/beta in LDS
    // (4 wavefronts per SIMD): 141 vs 155 us at 8192x16384; below, the teams
    // form was slower (103 vs 96 us at 8192x12288 with three teams of 256)
    if (groups <= 2048) SQ_LN(4, 512, 2);
#undef SQ_LN
    return hipErrorNotSupported;
}

// gamma_out[j] = fl(gamma[j] * inv_s[j]); beta_out likewise when beta is given.
__global__ __launch_bounds__(256) void k_fold_ln(const float* __restrict__ gamma, const float* __restrict__ beta,
                                                 const float* __restrict__ inv_s, int64_t K,
                                                 float* __restrict__ gamma_out, float* __restrict__ beta_out) {
    const int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (j >= K) return;
    gamma_out[j] = gamma[j] * inv_s[j];
    if (beta) beta_out[j] = beta[j] * inv_s[j];
}

hipError_t launch_fold_ln(const float* gamma, const float* beta, const float* inv_s, int64_t K, float* gamma_out,
                          float* beta_out, hipStream_t st) {
    if (K <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_fold_ln, dim3((unsigned)((K + 255) / 256)), dim3(256), 0, st, gamma, beta, inv_s, K,
                       gamma_out, beta_out);
    return hipGetLastError();
}

hipError_t launch_quant_act(const void* x, bool bf16, int64_t M, int64_t K, int64_t ld, const float* inv_s,
                            int mode, int8_t* xq, float* x_scale, uint32_t* gmax, hipStream_t st) {
    if (M <= 0) return hipSuccess;
    if (bf16)
        dispatch_act(static_cast<const bf16_t*>(x), M, K, ld, inv_s, mode, xq, x_scale, gmax, st);
    else
        dispatch_act(static_cast<const float*>(x), M, K, ld, inv_s, mode, xq, x_scale, gmax, st);
    return hipGetLastError();
}

}  // namespace sqk
