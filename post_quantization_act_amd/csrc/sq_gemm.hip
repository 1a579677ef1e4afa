// INT8 x INT8 -> int32 GEMM with the SmoothQuant dequantization epilogue on
// gfx950 matrix cores (v_mfma_i32_32x32x32_i8).
//
//   acc[m, n] = sum_k Xq[m, k] * Wq[n, k]        (exact int32)
//   y[m, n]   = bf16_rne(fl(fl(float(acc) * x_scale[m]) * w_scale[n]))
//
// Both operands are K-contiguous (Xq [M, K], Wq [N, K]).  The kernels compute
// the transposed product D = Wq . Xq^T so that each lane's accumulator
// registers run along n, which is the contiguous axis of y: four consecutive
// outputs leave as one 8-byte bf16 store.
//
// Two kernels:
//  - k_gemm_ring (K % 128 == 0, operands below 4 GiB): block tile BN x BM,
//    8 wavefronts in a WGN x WGM grid (two per SIMD, so one wavefront's
//    LDS and barrier waits are covered by the other's MFMAs), each owning
//    (BN/WGN) x (BM/WGM) of 32 x 32 MFMA blocks with its accumulators in
//    VGPRs.  Operand tiles of 128 bytes of k per row ("stages") are copied
//    from global memory straight into a two-buffer LDS ring with
//    global_load_lds_dwordx4, so no registers stage them and each row request
//    is one full 128-byte line.  Each stage is four k-steps of 32; fragments
//    of k-step s+1 are read from LDS while the matrix cores work on k-step s,
//    and the only workgroup barrier of a stage sits between k-steps 2 and 3:
//    after it the next stage is complete in LDS and the buffer of this stage
//    is free, so the copy of stage k+2 is issued during k-step 3.
//  - k_gemm_generic: any K % 16 == 0; register-staged double buffer.
//  - k_gemm_decode (M <= 16): weight-streaming kernel, see below.
// Blocks are dealt round-robin to the 8 XCDs; tiles are renumbered so each
// XCD walks a contiguous run of a grouped (m-major within groups of 8 tile
// rows) raster and concurrent blocks on one XCD share operand panels in its L2.
#include <algorithm>
#include <atomic>
#include <climits>
#include <cstdint>
#include <type_traits>

#include "sq_device.h"
#include "sq_internal.h"

namespace sqk {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) char lds_char;

constexpr int kBK = 128;  // bytes of k per stage (one 128-byte line per row)

// Slot (in 16-byte units) of chunk c (0..7) of row r inside a stage: chunks are
// XOR-swizzled by (r >> 1) & 7 so that the 16 rows a quarter-wavefront reads
// for one MFMA fragment, and the 8 rows x 8 chunks one 1-KB copy writes, hit
// distinct LDS banks.
__device__ __forceinline__ int swz(int r, int c) { return r * 8 + (c ^ ((r >> 1) & 7)); }

// Output tile renumbering: blocks are dealt round-robin to the 8 XCDs, so give
// each XCD a contiguous run of virtual tile ids, then walk them in groups of
// `group_m` tile rows (m-major inside a group).  tile_of: the tile of block b
// in a launch of nb blocks (one tile per block).
__device__ __forceinline__ void tile_of(int b, int nb, int tiles_n, int tiles_m, int group_m, int& tn, int& tm) {
    const int xcd = b % 8, l = b / 8, per = nb / 8, rem = nb % 8;
    const int v = (xcd < rem ? xcd * (per + 1) : rem * (per + 1) + (xcd - rem) * per) + l;
    const int group = group_m * tiles_n;
    const int g = v / group, first_m = g * group_m;
    const int gm = min(tiles_m - first_m, group_m);
    const int r = v % group;
    tm = first_m + r % gm;
    tn = r / gm;
}
__device__ __forceinline__ void tile_of_block(int tiles_n, int tiles_m, int group_m, int& tn, int& tm) {
    tile_of(blockIdx.x, gridDim.x, tiles_n, tiles_m, group_m, tn, tm);
}

// The 16-bit half of the LLM.int8()-style product (page "4.2 W8A8 量化与
// SmoothQuant" section 2): outlier input channels are multiplied in bf16 and
// added to the dequantized INT8 result.  The operands are compact copies of
// the outlier channels, k-contiguous and zero-padded to a multiple of 16:
// w_ot[N, kp] (rows of W) and x_o[M, kp] (columns of X); *count is the number
// of outlier channels.
struct OutlierOps {
    const uint16_t* x_o;
    const uint16_t* w_ot;
    const int32_t* count;
    int64_t kp;
};

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

// Sums over the outlier channels t of w_ot[n, t] * x_o[m, t] for the TN 32x32
// blocks of rows nbase + 32 a .. and columns m0 .., in the 32x32 accumulator
// layout, on v_mfma_f32_32x32x16_bf16 (lane l supplies row l % 32 and
// channels 8 (l / 32) .. +7 of each 16-channel step; products are exact in
// fp32 and summed in fp32).  All TN + 1 fragments of a step are loaded
// together, one step ahead of the matrix cores.  Rows past the matrix edge
// are clamped (never stored).
template <int TN>
__device__ __forceinline__ void outlier_blocks(const OutlierOps& op, int n16, int nbase, int m0, int N, int M,
                                               int lane, v16f (&o)[TN]) {
    const int fr = lane % 32, fh = lane / 32;
    const uint16_t* pa[TN];
#pragma unroll
    for (int a = 0; a < TN; ++a) {
        pa[a] = op.w_ot + (int64_t)min(nbase + a * 32 + fr, N - 1) * op.kp + 8 * fh;
        o[a] = v16f{};
    }
    const uint16_t* pb = op.x_o + (int64_t)min(m0 + fr, M - 1) * op.kp + 8 * fh;
    if (n16 == 0) return;
    uint4 ua[TN], ub = ld16(pb);
#pragma unroll
    for (int a = 0; a < TN; ++a) ua[a] = ld16(pa[a]);
    for (int t = 16;; t += 16) {
        const bool more = t < n16;  // uniform over the wavefront
        uint4 na[TN], nb;
        if (more) {
            nb = ld16(pb + t);
#pragma unroll
            for (int a = 0; a < TN; ++a) na[a] = ld16(pa[a] + t);
        }
#pragma unroll
        for (int a = 0; a < TN; ++a)
            o[a] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, ua[a]), __builtin_bit_cast(v8bf, ub),
                                                           o[a], 0, 0, 0);
        if (!more) break;
        ub = nb;
#pragma unroll
        for (int a = 0; a < TN; ++a) ua[a] = na[a];
    }
}

// Dequantize and store one wavefront's (TN*32) x (TM*32) block of accumulators.
// 32x32 accumulator layout: the lane holds column (lane % 32) of a 32x32 block
// (here: m) and rows 8*g + 4*(lane/32) + e, e = 0..3, in registers 4*g + e
// (here: n).
// x_scale is read at index m * xs_step: xs_step = 1 per token, 0 per tensor.
// kOut: 0 bf16, 1 fp32; kAcc: also store the int32 accumulators; kOut >= 2
// marks N % 4 != 0 (element-wise stores), with the output type kOut - 2.
// kO: add the 16-bit outlier product, y = fl(y8 + y16) (op is unused otherwise).
template <int TN, int TM, int kOut, bool kAcc, bool kO = false>
__device__ __forceinline__ void epilogue(const v16i (&acc)[TN][TM], int nbase, int mbase, int lane,
                                         const float* __restrict__ x_scale, int xs_step,
                                         const float* __restrict__ w_scale, int M, int N, int ldy,
                                         void* __restrict__ y, int32_t* __restrict__ acc_out,
                                         const OutlierOps& op = OutlierOps{}) {
    const int fr = lane % 32, fh = lane / 32;
    constexpr bool n_vec = kOut < 2;
    constexpr int kTy = kOut & 1;
    int n16 = 0;
    if constexpr (kO) n16 = (__builtin_amdgcn_readfirstlane(op.count[0]) + 15) & ~15;
#pragma unroll
    for (int b = 0; b < TM; ++b) {
        const int m = mbase + b * 32 + fr;
        // (every lane takes part in the matrix-core addend, so no early exit
        // for rows past M when kO)
        if (!kO && m >= M) continue;
        const float xs = m < M ? x_scale[m * xs_step] : 0.0f;
        v16f ob[kO ? TN : 1];
        if constexpr (kO) outlier_blocks<TN>(op, n16, nbase, mbase + b * 32, N, M, lane, ob);
        if (kO && m >= M) continue;
#pragma unroll
        for (int a = 0; a < TN; ++a) {
            const v16f& o = ob[kO ? a : 0];
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int n = nbase + a * 32 + 8 * g + 4 * fh;
                if (n >= N) continue;
                int32_t av[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) av[e] = acc[a][b][4 * g + e];
                if constexpr (n_vec) {
                    const float4 ws = *reinterpret_cast<const float4*>(w_scale + n);
                    float y0 = ((float)av[0] * xs) * ws.x;
                    float y1 = ((float)av[1] * xs) * ws.y;
                    float y2 = ((float)av[2] * xs) * ws.z;
                    float y3 = ((float)av[3] * xs) * ws.w;
                    if constexpr (kO) {
                        y0 += o[4 * g + 0];
                        y1 += o[4 * g + 1];
                        y2 += o[4 * g + 2];
                        y3 += o[4 * g + 3];
                    }
                    const int64_t off = (int64_t)m * ldy + n;
                    if constexpr (kTy == 0) {
                        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(y) + off) =
                            make_uint2(pack_bf16x2(y0, y1), pack_bf16x2(y2, y3));
                    } else {
                        *reinterpret_cast<float4*>(static_cast<float*>(y) + off) = make_float4(y0, y1, y2, y3);
                    }
                    if constexpr (kAcc) *reinterpret_cast<int4*>(acc_out + off) = make_int4(av[0], av[1], av[2], av[3]);
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        if (n + e >= N) break;
                        float v = ((float)av[e] * xs) * w_scale[n + e];
                        if constexpr (kO) v += o[4 * g + e];
                        const int64_t off = (int64_t)m * ldy + n + e;
                        if constexpr (kTy == 0) {
                            static_cast<uint16_t*>(y)[off] = (uint16_t)(pack_bf16x2(v, 0.0f) & 0xFFFFu);
                        } else {
                            static_cast<float*>(y)[off] = v;
                        }
                        if constexpr (kAcc) acc_out[off] = av[e];
                    }
                }
            }
            // one 32x32 block at a time: keeps the AGPR -> VGPR copies short-lived
            __builtin_amdgcn_sched_barrier(0);
        }
    }
}

// The bf16 epilogue through LDS (N % 8 == 0, LDS free after the main loop):
// per group of 32 token rows, the wavefront writes its dequantized outputs
// into its own [m][n] LDS region (row stride WN + 8 elements, 16-byte aligned
// rows), then copies them out 16 bytes (8 outputs) per lane along n, so each
// store instruction covers whole 256-byte runs of rows of y instead of 64
// scattered 8-byte pieces.  The stores are nontemporal: y is written once,
// and dirty lines left in L2 would be written back at the end of the launch.
// Same arithmetic as epilogue<> per element.
// sx, sw: the wavefront's token and weight scales, staged in LDS.
template <int TN, int TM>
__device__ __forceinline__ void epilogue_bf16_lds(const v16i (&acc)[TN][TM], int nbase, int mbase, int lane,
                                                  const float* sx, const float* sw, int M, int N, int ldy,
                                                  uint16_t* __restrict__ y, uint16_t* ldsw) {
    constexpr int WN = TN * 32, RS = WN + 8, CH = WN / 8;
    static_assert((32 * CH) % 64 == 0, "copy-out chunks");
    const int fr = lane % 32, fh = lane / 32;
#pragma unroll
    for (int b = 0; b < TM; ++b) {
        const float xs = sx[b * 32 + fr];
#pragma unroll
        for (int a = 0; a < TN; ++a) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int nl = a * 32 + 8 * g + 4 * fh;
                const float4 ws = *reinterpret_cast<const float4*>(sw + nl);
                const float y0 = ((float)acc[a][b][4 * g + 0] * xs) * ws.x;
                const float y1 = ((float)acc[a][b][4 * g + 1] * xs) * ws.y;
                const float y2 = ((float)acc[a][b][4 * g + 2] * xs) * ws.z;
                const float y3 = ((float)acc[a][b][4 * g + 3] * xs) * ws.w;
                *reinterpret_cast<uint2*>(ldsw + fr * RS + nl) = make_uint2(pack_bf16x2(y0, y1), pack_bf16x2(y2, y3));
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // this wavefront's writes land before its reads
#pragma unroll
        for (int i = 0; i < 32 * CH / 64; ++i) {
            const int c = lane + 64 * i;
            const int ml = c / CH, nc = c % CH;
            const int mm = mbase + b * 32 + ml, n = nbase + nc * 8;
            const uint4 v = *reinterpret_cast<const uint4*>(ldsw + ml * RS + nc * 8);
            if (mm < M && n < N) st16_stream(y + (int64_t)mm * ldy + n, v);  // written once
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // reads done before the next group reuses the region
    }
}

// ---- ring kernel: global -> LDS copies without registers -----------------------

// One 16-byte-per-lane copy from global memory (base + voff) to LDS at
// lds_off + 16 * lane.  The LDS destination goes through M0; the instruction
// has no register result (the data lands in LDS), so its completion is
// tracked only by vmcnt, which the kernel waits on explicitly before the
// barrier that publishes the stage.
__device__ __forceinline__ void copy16_to_lds(const int8_t* base, uint32_t voff, uint32_t lds_off) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
                 :
                 : "s"(lds_off), "v"(voff), "s"(base)
                 : "memory", "m0");
}

// One dword per lane from global memory (base + voff) to LDS at lds_off + 4 * lane.
__device__ __forceinline__ void copy4_to_lds(const void* base, uint32_t voff, uint32_t lds_off) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, %2"
                 :
                 : "s"(lds_off), "v"(voff), "s"(base)
                 : "memory", "m0");
}

// vmcnt wait and LDS-only barrier as asm with a memory clobber, so that no LDS
// read of copied data is moved above them.  The copies are the only vector
// memory loads in flight in the kernels that use them, and loads complete in
// order, so vmcnt(n) means "all but the n most recent copies have landed".
template <int kN>
__device__ __forceinline__ void wait_vmcnt() {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kN) : "memory");
}
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

template <int BN, int BM, int WGN, int WGM, int NS, int kOut, bool kAcc, bool kO>
__global__ __launch_bounds__(64 * WGN * WGM) void k_gemm_ring(const int8_t* __restrict__ xq, const float* __restrict__ x_scale,
                                                   int xs_step, const int8_t* __restrict__ wq,
                                                   const float* __restrict__ w_scale, int M, int N, int K,
                                                   void* __restrict__ y, int ldy, int32_t* __restrict__ acc_out,
                                                   int tiles_n, int tiles_m, int group_m, OutlierOps op) {
    constexpr int NW = WGN * WGM;             // wavefronts per block
    constexpr int WN = BN / WGN, WM = BM / WGM, TN = WN / 32, TM = WM / 32;
    constexpr int ROWS = BN + BM;             // rows of a stage: Wq tile rows, then Xq tile rows
    constexpr int STAGE = ROWS * 8;           // 16-byte slots per stage
    constexpr int COPIES = ROWS / 8;          // 1-KB copies per stage (8 rows each)
    constexpr int L = COPIES / NW;            // copies per wavefront per stage
    constexpr int NMF = TN * TM;              // MFMAs per k-step
    constexpr int NRD = TN + TM;              // fragment reads per k-step
    constexpr int DR = (NRD + NMF - 1) / NMF, DD = (L + NMF - 1) / NMF;
    static_assert(COPIES % NW == 0 && BN % 8 == 0 && WN % 32 == 0 && WM % 32 == 0, "tile");
    static_assert(NS >= 2 && NS * STAGE * 16 <= 160 * 1024, "LDS");
    __shared__ uint4 lds[NS * STAGE];

    const int lane = threadIdx.x % kWave;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int wn = wave % WGN, wm = wave / WGN;
    int tn, tm;
    tile_of_block(tiles_n, tiles_m, group_m, tn, tm);
    const int n0 = tn * BN, m0 = tm * BM;

    // Copy j of this wavefront (global copy index i = wave + NW j) fills rows
    // 8i .. 8i+7 of a stage: lane -> row 8i + lane/8 and LDS chunk lane%8,
    // which holds logical chunk (lane%8) ^ ((row >> 1) & 7).  Rows past the
    // matrix edge are clamped to the last row (read, never stored).
    uint32_t off[L];
#pragma unroll
    for (int j = 0; j < L; ++j) {
        const int i = wave + NW * j;
        const int r = 8 * i + lane / 8;
        const int c = (lane % 8) ^ ((r >> 1) & 7);
        if (r < BN) off[j] = (uint32_t)min(n0 + r, N - 1) * (uint32_t)K + c * 16;
        else off[j] = (uint32_t)min(m0 + r - BN, M - 1) * (uint32_t)K + c * 16;
    }
    const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_char*)lds;
    auto copy = [&](int kt, int j) {
        const int i = wave + NW * j;
        const uint32_t la = __builtin_amdgcn_readfirstlane(lds0 + ((kt % NS) * STAGE + i * 64) * 16);
        copy16_to_lds(8 * i < BN ? wq : xq, off[j] + (uint32_t)kt * kBK, la);
    };

    const int fr = lane % 32, fh = lane / 32;
    v16i acc[TN][TM];
#pragma unroll
    for (int a = 0; a < TN; ++a)
#pragma unroll
        for (int b = 0; b < TM; ++b)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[a][b][e] = 0;

    v4i fa[2][TN], fb[2][TM];  // fragments of two consecutive k-steps
    auto read_frag = [&](int buf, int ks, int q, int sl) {
        const uint4* base = lds + buf * STAGE;
        const int c = 2 * ks + fh;
        if (q < TN) {
            const uint4 u = base[swz(wn * WN + q * 32 + fr, c)];
            fa[sl][q] = v4i{(int)u.x, (int)u.y, (int)u.z, (int)u.w};
        } else {
            const uint4 u = base[swz(BN + wm * WM + (q - TN) * 32 + fr, c)];
            fb[sl][q - TN] = v4i{(int)u.x, (int)u.y, (int)u.z, (int)u.w};
        }
    };
    // One k-step: NMF MFMAs on fragment slot `sl`; between them, the reads of
    // k-step `rks` of LDS buffer `rbuf` into slot `rsl`, and the copies of
    // stage `ckt`.  sched_barrier keeps this interleaving in program order.
    // Copies [c_lo, c_hi) of stage ckt are spread over the k-step's MFMAs.
    auto kstep = [&](int sl, bool rd, int rbuf, int rks, int rsl, bool cp, int ckt, int c_lo, int c_hi) {
        const int cn = c_hi - c_lo, cper = (cn + NMF - 1) / NMF;
#pragma unroll
        for (int j = 0; j < NMF; ++j) {
            const int a = j / TM, b = j % TM;
            acc[a][b] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fa[sl][a], fb[sl][b], acc[a][b], 0, 0, 0);
#pragma unroll
            for (int u = 0; u < DR; ++u)
                if (rd && j * DR + u < NRD) read_frag(rbuf, rks, j * DR + u, rsl);
#pragma unroll
            for (int u = 0; u < DD; ++u)
                if (cp && u < cper && j * cper + u < cn) copy(ckt, c_lo + j * cper + u);
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    // A stage's L copies go out in PARTS parts: the first in k-step 3 of the
    // iteration that frees its buffer, the others in k-steps 0 .. PARTS-2 of
    // the next iteration, so the copy traffic is not one burst per stage.
    // Stage kt+1's last part then still precedes the L copies of stage kt+2
    // (NS = 3) or is itself waited for (NS = 2): the vmcnt waits are unchanged.
    constexpr int PARTS = (NS >= 3 && L % 3 == 0) ? 3 : (L % 2 == 0 ? 2 : 1);
    constexpr int LP = L / PARTS;

    // The tile's scales for the bf16 epilogue: w_scale of its BN rows of Wq,
    // then x_scale of its BM token rows (clamped at the edges), copied into
    // LDS ahead of the first stage (older than every copy, so the prologue's
    // wait covers them).
    constexpr bool kLdsEpi = kOut == 0 && !kAcc && !kO;
    __shared__ __align__(16) float scl[kLdsEpi ? BN + BM : 1];
    if constexpr (kLdsEpi) {
        static_assert(BN % 64 == 0 && BM % 64 == 0 && (BN + BM) / 64 <= NW, "scale staging");
        if (wave < (BN + BM) / 64) {
            const int r = wave * 64 + lane;
            const uint32_t la = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_char*)scl + wave * 256);
            if (wave * 64 < BN)
                copy4_to_lds(w_scale, (uint32_t)min(n0 + r, N - 1) * 4u, la);
            else
                copy4_to_lds(x_scale, (uint32_t)(min(m0 + r - BN, M - 1) * xs_step) * 4u, la);
        }
    }
    // Prologue: stages 0 .. NS-1 in flight, wait for stage 0.
    const int nk = K / kBK;
#pragma unroll
    for (int s = 0; s < NS; ++s)
        if (s < nk) {
#pragma unroll
            for (int j = 0; j < L; ++j) copy(s, j);
        }
    if (nk >= NS)
        wait_vmcnt<L*(NS - 1)>();
    else
        wait_vmcnt<0>();
    lds_barrier();
    if (nk > 0) {
#pragma unroll
        for (int q = 0; q < NRD; ++q) read_frag(0, 0, q, 0);
    }
    // Steady state: iteration kt reads stage kt+1 from LDS and copies stage
    // kt+NS into the buffer of stage kt; the last NS iterations copy nothing.
    int kt = 0, buf = 0;
    for (; kt + NS < nk; ++kt) {
        const int nbuf = buf + 1 == NS ? 0 : buf + 1;
        const bool late = kt > 0;  // the rest of stage kt-1+NS's copies
        __builtin_amdgcn_sched_barrier(0);
        kstep(0, true, buf, 1, 1, late && PARTS > 1, kt - 1 + NS, LP, 2 * LP);
        kstep(1, true, buf, 2, 0, late && PARTS > 2, kt - 1 + NS, 2 * LP, 3 * LP);
        kstep(0, true, buf, 3, 1, false, 0, 0, 0);
        // This wavefront's copies of stage kt+1 have landed (those of stages
        // kt+2 .. kt+NS-1 may stay in flight); after the barrier every
        // wavefront's have, and every read of this stage's buffer is done.
        wait_vmcnt<L*(NS - 2)>();
        lds_barrier();
        kstep(1, true, nbuf, 0, 0, true, kt + NS, 0, LP);
        buf = nbuf;
    }
    for (; kt < nk; ++kt) {
        const int nbuf = buf + 1 == NS ? 0 : buf + 1;
        const bool late = kt > 0 && kt - 1 + NS < nk;
        __builtin_amdgcn_sched_barrier(0);
        kstep(0, true, buf, 1, 1, late && PARTS > 1, kt - 1 + NS, LP, 2 * LP);
        kstep(1, true, buf, 2, 0, late && PARTS > 2, kt - 1 + NS, 2 * LP, 3 * LP);
        kstep(0, true, buf, 3, 1, false, 0, 0, 0);
        wait_vmcnt<0>();
        lds_barrier();
        kstep(1, kt + 1 < nk, nbuf, 0, 0, false, 0, 0, 0);
        buf = nbuf;
    }
    if constexpr (kLdsEpi) {
        static_assert(NW * 32 * (WN + 8) * 2 <= NS * STAGE * 16, "LDS for the bf16 epilogue");
        if (N % 8 == 0 && ldy % 8 == 0) {
            lds_barrier();  // every wavefront is done reading the ring
            uint16_t* ldsw = reinterpret_cast<uint16_t*>(lds) + wave * 32 * (WN + 8);
            epilogue_bf16_lds<TN, TM>(acc, n0 + wn * WN, m0 + wm * WM, lane, scl + BN + wm * WM, scl + wn * WN, M,
                                      N, ldy, static_cast<uint16_t*>(y), ldsw);
            return;
        }
    }
    epilogue<TN, TM, kOut, kAcc, kO>(acc, n0 + wn * WN, m0 + wm * WM, lane, x_scale, xs_step, w_scale, M, N, ldy, y,
                                     acc_out, op);
}

// ---- persistent ring kernel: tiles walked per block, epilogue overlapped ----------
//
// The deployed product (bf16 output through the LDS epilogue, N % 8 == 0, no
// accumulator store, K % (128 NS) == 0) over many rounds of tiles.  The grid is
// one block per CU (a multiple of 8, so block p stays on XCD p % 8); block p
// computes the tiles blocks p, p + G, p + 2G, ... of the one-tile-per-block
// launch would, in that order.  Within a tile the main loop is k_gemm_ring's.
// Between tiles the next tile's first stage and its scales are copied while the
// current tile finishes: its stage 0 goes into the ring buffer freed two stages
// before the end (in the last two iterations, as a regular stage would), its
// scales into the other half of a double-buffered scale area; the epilogue
// stages its outputs in the buffer of the last stage (free once every
// wavefront passed the last iteration's barrier); after a barrier the next
// tile's stage 1 follows.  So the CU streams the next tile's operands while it
// dequantizes and stores, instead of waiting for them at the start of every
// tile.
template <int BN, int BM, int WGN, int WGM, int NS>
__global__ __launch_bounds__(64 * WGN * WGM) void k_gemm_persist(
    const int8_t* __restrict__ xq, const float* __restrict__ x_scale, int xs_step, const int8_t* __restrict__ wq,
    const float* __restrict__ w_scale, int M, int N, int K, uint16_t* __restrict__ y, int ldy, int tiles_n,
    int tiles_m, int group_m, int ntiles) {
    constexpr int NW = WGN * WGM;
    constexpr int WN = BN / WGN, WM = BM / WGM, TN = WN / 32, TM = WM / 32;
    constexpr int ROWS = BN + BM, STAGE = ROWS * 8, COPIES = ROWS / 8, L = COPIES / NW;
    constexpr int NMF = TN * TM, NRD = TN + TM;
    constexpr int DR = (NRD + NMF - 1) / NMF, DD = (L + NMF - 1) / NMF;
    constexpr int PARTS = (NS >= 3 && L % 3 == 0) ? 3 : (L % 2 == 0 ? 2 : 1);
    constexpr int LP = L / PARTS;
    constexpr int SC = BN + BM;  // scales per tile
    static_assert(COPIES % NW == 0 && WN % 32 == 0 && WM % 32 == 0, "tile");
    static_assert(BN % 64 == 0 && BM % 64 == 0 && (SC / 64) % NW == 0 || SC / 64 < NW, "scale staging");
    static_assert(NS * STAGE * 16 + 2 * SC * 4 <= 160 * 1024, "LDS");
    static_assert(NW * 32 * (WN + 8) * 2 <= STAGE * 16, "the epilogue's staging fits one ring buffer");
    __shared__ uint4 lds[NS * STAGE];
    __shared__ __align__(16) float scl[2 * SC];

    const int lane = threadIdx.x % kWave;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int wn = wave % WGN, wm = wave / WGN;
    const int fr = lane % 32, fh = lane / 32;
    const int nk = K / kBK;
    const int G = gridDim.x;
    const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_char*)lds;
    const uint32_t scl0 = (uint32_t)(uintptr_t)(lds_char*)scl;

    // Copy j of a stage fills rows 8i .. 8i+7 (i = wave + NW j): lane -> row
    // 8i + lane/8 = r0 + 8 NW j, LDS chunk lane%8 holding logical chunk
    // (lane%8) ^ ((row>>1)&7), which is the same for every j (8 NW j is a
    // multiple of 16).  Source offsets are formed per copy from r0 and that
    // chunk; rows past the edge are clamped (read, never stored).
    static_assert((8 * NW) % 16 == 0, "one chunk swizzle per wavefront");
    const int r0 = 8 * wave + lane / 8;
    const uint32_t cb = (uint32_t)(((lane % 8) ^ ((r0 >> 1) & 7)) * 16);
    auto copy_from = [&](int tn0, int tm0, int st, int j) {  // stage st of the tile at (tn0, tm0), copy j
        const int i = wave + NW * j;
        const int r = r0 + 8 * NW * j;
        const uint32_t la = __builtin_amdgcn_readfirstlane(lds0 + ((st % NS) * STAGE + i * 64) * 16);
        const uint32_t row = 8 * i < BN ? (uint32_t)min(tn0 + r, N - 1) : (uint32_t)min(tm0 + r - BN, M - 1);
        copy16_to_lds(8 * i < BN ? wq : xq, row * (uint32_t)K + cb + (uint32_t)st * kBK, la);
    };
    // The tile's w_scale rows then x_scale rows into scale buffer `half`.
    auto copy_scales = [&](int n0, int m0, int half) {
#pragma unroll
        for (int c0 = 0; c0 < SC / 64; c0 += NW) {
            const int c = c0 + wave;  // 64 scales per copy
            if (c < SC / 64) {
                const int r = c * 64 + lane;
                const uint32_t la = __builtin_amdgcn_readfirstlane(scl0 + (half * SC + c * 64) * 4);
                if (c * 64 < BN)
                    copy4_to_lds(w_scale, (uint32_t)min(n0 + r, N - 1) * 4u, la);
                else
                    copy4_to_lds(x_scale, (uint32_t)(min(m0 + r - BN, M - 1) * xs_step) * 4u, la);
            }
        }
    };

    int tn, tm;
    int vb = blockIdx.x;
    tile_of(vb, ntiles, tiles_n, tiles_m, group_m, tn, tm);
    int n0 = tn * BN, m0 = tm * BM;
    int n0n = 0, m0n = 0;

    v16i acc[TN][TM];
    v4i fa[2][TN], fb[2][TM];
    auto read_frag = [&](int buf, int ks, int q, int sl) {
        const uint4* base = lds + buf * STAGE;
        const int c = 2 * ks + fh;
        if (q < TN) {
            const uint4 u = base[swz(wn * WN + q * 32 + fr, c)];
            fa[sl][q] = v4i{(int)u.x, (int)u.y, (int)u.z, (int)u.w};
        } else {
            const uint4 u = base[swz(BN + wm * WM + (q - TN) * 32 + fr, c)];
            fb[sl][q - TN] = v4i{(int)u.x, (int)u.y, (int)u.z, (int)u.w};
        }
    };
    // Copy j of "stage" st of the ring: st < nk is this tile's stage st, st == nk
    // the next tile's stage 0 (when there is one); later ones are issued after
    // the epilogue.
    bool has_next = false;
    auto copy = [&](int st, int j) {
        if (st < nk) copy_from(n0, m0, st, j);
        else if (st == nk && has_next) copy_from(n0n, m0n, 0, j);
    };
    auto kstep = [&](int sl, bool rd, int rbuf, int rks, int rsl, bool cp, int ckt, int c_lo, int c_hi) {
        const int cn = c_hi - c_lo, cper = (cn + NMF - 1) / NMF;
#pragma unroll
        for (int j = 0; j < NMF; ++j) {
            const int a = j / TM, b = j % TM;
            acc[a][b] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fa[sl][a], fb[sl][b], acc[a][b], 0, 0, 0);
#pragma unroll
            for (int u = 0; u < DR; ++u)
                if (rd && j * DR + u < NRD) read_frag(rbuf, rks, j * DR + u, rsl);
#pragma unroll
            for (int u = 0; u < DD; ++u)
                if (cp && u < cper && j * cper + u < cn) copy(ckt, c_lo + j * cper + u);
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // Prologue of the first tile: its scales and stages 0 .. NS-1.
    copy_scales(n0, m0, 0);
#pragma unroll
    for (int st = 0; st < NS; ++st)
#pragma unroll
        for (int j = 0; j < L; ++j) copy_from(n0, m0, st, j);
    wait_vmcnt<L*(NS - 1)>();
    lds_barrier();
#pragma unroll
    for (int q = 0; q < NRD; ++q) read_frag(0, 0, q, 0);

    for (int it = 0;; ++it) {
        const int vbn = vb + G;
        has_next = vbn < ntiles;
        if (has_next) {
            int tnn, tmn;
            tile_of(vbn, ntiles, tiles_n, tiles_m, group_m, tnn, tmn);
            n0n = tnn * BN;
            m0n = tmn * BM;
        }
#pragma unroll
        for (int a = 0; a < TN; ++a)
#pragma unroll
            for (int b = 0; b < TM; ++b)
#pragma unroll
                for (int e = 0; e < 16; ++e) acc[a][b][e] = 0;

        // The ring position restarts at buffer 0 with every tile (nk % NS == 0).
        int kt = 0, buf = 0;
        for (; kt + NS < nk; ++kt) {
            const int nbuf = buf + 1 == NS ? 0 : buf + 1;
            const bool late = kt > 0;
            __builtin_amdgcn_sched_barrier(0);
            kstep(0, true, buf, 1, 1, late && PARTS > 1, kt - 1 + NS, LP, 2 * LP);
            kstep(1, true, buf, 2, 0, late && PARTS > 2, kt - 1 + NS, 2 * LP, 3 * LP);
            kstep(0, true, buf, 3, 1, false, 0, 0, 0);
            wait_vmcnt<L*(NS - 2)>();
            lds_barrier();
            kstep(1, true, nbuf, 0, 0, true, kt + NS, 0, LP);
            buf = nbuf;
        }
        // The last NS iterations: the stages after the last one are the next
        // tile's stage 0 (copied here) and its stage 1 .. (after the epilogue).
        for (; kt < nk; ++kt) {
            const int nbuf = buf + 1 == NS ? 0 : buf + 1;
            const bool late = kt > 0;
            __builtin_amdgcn_sched_barrier(0);
            kstep(0, true, buf, 1, 1, late && PARTS > 1, kt - 1 + NS, LP, 2 * LP);
            kstep(1, true, buf, 2, 0, late && PARTS > 2, kt - 1 + NS, 2 * LP, 3 * LP);
            kstep(0, true, buf, 3, 1, false, 0, 0, 0);
            if (kt + 1 < nk) wait_vmcnt<0>();  // the tile's last stage has landed (nothing newer is in flight)
            lds_barrier();                        // in the last iteration: every read of the last buffer is done
            if (kt + NS == nk && has_next) copy_scales(n0n, m0n, (it + 1) & 1);
            kstep(1, kt + 1 < nk, nbuf, 0, 0, kt + NS == nk, kt + NS, 0, LP);
            buf = nbuf;
        }
        // Epilogue: outputs staged in the buffer of the last stage, scales from
        // this tile's half of the scale area.
        {
            uint16_t* ldsw = reinterpret_cast<uint16_t*>(lds + ((nk - 1) % NS) * STAGE) + wave * 32 * (WN + 8);
            const float* sc = scl + (it & 1) * SC;
            epilogue_bf16_lds<TN, TM>(acc, n0 + wn * WN, m0 + wm * WM, lane, sc + BN + wm * WM, sc + wn * WN, M, N,
                                      ldy, y, ldsw);
        }
        if (!has_next) break;
        // Every wavefront is done with its staging region: the next tile's
        // stages 1 .. NS-1 may overwrite the ring.
        lds_barrier();
#pragma unroll
        for (int st = 1; st < NS; ++st)
#pragma unroll
            for (int j = 0; j < L; ++j) copy_from(n0n, m0n, st, j);
        wait_vmcnt<L*(NS - 1)>();  // stage 0 and the scales of the next tile (and the stores before them)
        lds_barrier();
        vb = vbn;
        n0 = n0n;
        m0 = m0n;
#pragma unroll
        for (int q = 0; q < NRD; ++q) read_frag(0, 0, q, 0);
    }
}

// ---- generic kernel: any K % 16 == 0 -------------------------------------------

template <int BN, int BM, int kOut, bool kAcc, bool kO>
__global__ __launch_bounds__(256) void k_gemm_generic(const int8_t* __restrict__ xq, const float* __restrict__ x_scale,
                                                      int xs_step, const int8_t* __restrict__ wq,
                                                      const float* __restrict__ w_scale, int M, int N, int K,
                                                      void* __restrict__ y, int ldy, int32_t* __restrict__ acc_out,
                                                      int tiles_n, int tiles_m, int group_m, OutlierOps op) {
    constexpr int WN = BN / 2, WM = BM / 2;
    constexpr int TN = WN / 32, TM = WM / 32;
    constexpr int A_CHUNKS = BN * 8 / 256;  // 16-byte chunks per thread per stage
    constexpr int B_CHUNKS = BM * 8 / 256;
    constexpr int STAGE = (BN + BM) * 8;    // uint4 slots per stage

    __shared__ uint4 lds[2 * STAGE];

    const int tid = threadIdx.x;
    const int wave = tid / kWave, lane = tid % kWave;
    const int wn = wave % 2, wm = wave / 2;
    int tn, tm;
    tile_of_block(tiles_n, tiles_m, group_m, tn, tm);
    const int n0 = tn * BN, m0 = tm * BM;

    // Source rows of this thread's chunks (clamped into the matrix so ragged
    // edges read valid memory; their results are never stored).  A chunk past
    // K reads its row's first chunk and is zeroed when written to LDS.
    const int8_t* a_src[A_CHUNKS];
    const int8_t* b_src[B_CHUNKS];
    int a_slot[A_CHUNKS], b_slot[B_CHUNKS], a_kc[A_CHUNKS], b_kc[B_CHUNKS];
#pragma unroll
    for (int i = 0; i < A_CHUNKS; ++i) {
        const int q = tid + i * 256;
        const int r = q / 8, c = q % 8;
        a_src[i] = wq + (int64_t)min(n0 + r, N - 1) * K;
        a_kc[i] = c * 16;
        a_slot[i] = swz(r, c);
    }
#pragma unroll
    for (int i = 0; i < B_CHUNKS; ++i) {
        const int q = tid + i * 256;
        const int r = q / 8, c = q % 8;
        b_src[i] = xq + (int64_t)min(m0 + r, M - 1) * K;
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
#pragma unroll
        for (int i = 0; i < A_CHUNKS; ++i) ra[i] = ld16(a_src[i] + (k0 + a_kc[i] < K ? k0 + a_kc[i] : 0));
#pragma unroll
        for (int i = 0; i < B_CHUNKS; ++i) rb[i] = ld16(b_src[i] + (k0 + b_kc[i] < K ? k0 + b_kc[i] : 0));
    };
    auto lstore = [&](int buf, int kt) {
        uint4* base = lds + buf * STAGE;
        const int k0 = kt * kBK;
        if (k0 + kBK <= K) {
#pragma unroll
            for (int i = 0; i < A_CHUNKS; ++i) base[a_slot[i]] = ra[i];
#pragma unroll
            for (int i = 0; i < B_CHUNKS; ++i) base[b_slot[i]] = rb[i];
        } else {
#pragma unroll
            for (int i = 0; i < A_CHUNKS; ++i) {
                const uint32_t mk = k0 + a_kc[i] < K ? 0xFFFFFFFFu : 0u;
                base[a_slot[i]] = make_uint4(ra[i].x & mk, ra[i].y & mk, ra[i].z & mk, ra[i].w & mk);
            }
#pragma unroll
            for (int i = 0; i < B_CHUNKS; ++i) {
                const uint32_t mk = k0 + b_kc[i] < K ? 0xFFFFFFFFu : 0u;
                base[b_slot[i]] = make_uint4(rb[i].x & mk, rb[i].y & mk, rb[i].z & mk, rb[i].w & mk);
            }
        }
    };

    const int fr = lane % 32, fh = lane / 32;
    v4i af[2][TN], bfr[2][TM];
    auto rfrag = [&](int buf, int ks, int slot) {
        const uint4* base = lds + buf * STAGE;
        const int c = 2 * ks + fh;
#pragma unroll
        for (int a = 0; a < TN; ++a) {
            const uint4 u = base[swz(wn * WN + a * 32 + fr, c)];
            af[slot][a] = v4i{(int)u.x, (int)u.y, (int)u.z, (int)u.w};
        }
#pragma unroll
        for (int b = 0; b < TM; ++b) {
            const uint4 u = base[BN * 8 + swz(wm * WM + b * 32 + fr, c)];
            bfr[slot][b] = v4i{(int)u.x, (int)u.y, (int)u.z, (int)u.w};
        }
    };

    if (nk > 0) {
        gload(0);
        lstore(0, 0);
    }
    __syncthreads();
    if (nk > 0) rfrag(0, 0, 0);
    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < nk) gload(kt + 1);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int ks = 0; ks < kBK / 32; ++ks) {
            if (ks < kBK / 32 - 1) rfrag(cur, ks + 1, (ks + 1) & 1);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int a = 0; a < TN; ++a)
#pragma unroll
                for (int b = 0; b < TM; ++b)
                    acc[a][b] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[ks & 1][a], bfr[ks & 1][b], acc[a][b], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
        if (kt + 1 < nk) {
            lstore(cur ^ 1, kt + 1);
            __syncthreads();
            rfrag(cur ^ 1, 0, 0);
        }
    }
    epilogue<TN, TM, kOut, kAcc, kO>(acc, n0 + wn * WN, m0 + wm * WM, lane, x_scale, xs_step, w_scale, M, N, ldy, y,
                                     acc_out, op);
}

// ---- decode kernel: few tokens, the weight stream is the cost ---------------------
//
// For M <= 16 the product is bound by reading Wq once from HBM.  Each block
// owns 32 output channels; its 4 wavefronts split K into quarters and stream
// their part of the 32 weight rows straight into MFMA operand registers
// (v_mfma_i32_16x16x64_i8: A = 16 weight rows x 64 k, B = the 16 token rows x
// 64 k, read from L2 where the small Xq stays resident).  The four int32
// partial tiles are summed through LDS, then one wavefront dequantizes.
// 16x16 accumulator layout: lane l holds D[4*(l/16) + i][l % 16], i = 0..3,
// i.e. four consecutive output channels n of token m = l % 16.
template <int kOut, bool kAcc>
__global__ __launch_bounds__(256) void k_gemm_decode(const int8_t* __restrict__ xq, const float* __restrict__ x_scale,
                                                     int xs_step, const int8_t* __restrict__ wq,
                                                     const float* __restrict__ w_scale, int M, int N, int K,
                                                     void* __restrict__ y, int32_t* __restrict__ acc_out) {
    constexpr int U = 4;  // k-steps of 64 in flight per wavefront
    __shared__ v4i part[4][2][kWave];
    const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
    const int n0 = blockIdx.x * 32;
    const int r16 = lane % 16, kc = (lane / 16) * 16;  // operand row and 16-byte k chunk of this lane
    const int8_t* a0 = wq + (int64_t)min(n0 + r16, N - 1) * K + kc;
    const int8_t* a1 = wq + (int64_t)min(n0 + 16 + r16, N - 1) * K + kc;
    const int8_t* bx = xq + (int64_t)min(r16, M - 1) * K + kc;
    // K split into 4 contiguous ranges of whole 64-byte steps (the last may be partial)
    const int steps = (K + 63) / 64;
    const int per = (steps + 3) / 4;
    const int s0 = wave * per, s1 = min(steps, s0 + per);
    v4i acc0 = {0, 0, 0, 0}, acc1 = {0, 0, 0, 0};
    auto load = [&](const int8_t* p, int k) -> v4i {
        // chunks at or past K read the row start and are zeroed
        const bool in = k + kc < K;
        const uint4 u = in ? ld16_stream(p + k) : make_uint4(0, 0, 0, 0);
        return v4i{(int)u.x, (int)u.y, (int)u.z, (int)u.w};
    };
    auto loadb = [&](int k) -> v4i {
        const bool in = k + kc < K;
        const uint4 u = in ? ld16(bx + k) : make_uint4(0, 0, 0, 0);
        return v4i{(int)u.x, (int)u.y, (int)u.z, (int)u.w};
    };
    int st = s0;
    for (; st + U <= s1; st += U) {
        v4i fa0[U], fa1[U], fb[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int k = (st + u) * 64;
            fa0[u] = load(a0, k);
            fa1[u] = load(a1, k);
            fb[u] = loadb(k);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            acc0 = __builtin_amdgcn_mfma_i32_16x16x64_i8(fa0[u], fb[u], acc0, 0, 0, 0);
            acc1 = __builtin_amdgcn_mfma_i32_16x16x64_i8(fa1[u], fb[u], acc1, 0, 0, 0);
        }
    }
    for (; st < s1; ++st) {
        const int k = st * 64;
        const v4i f0 = load(a0, k), f1 = load(a1, k), fb = loadb(k);
        acc0 = __builtin_amdgcn_mfma_i32_16x16x64_i8(f0, fb, acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_i32_16x16x64_i8(f1, fb, acc1, 0, 0, 0);
    }
    part[wave][0][lane] = acc0;
    part[wave][1][lane] = acc1;
    __syncthreads();
    if (wave != 0) return;
    const int m = lane % 16;
    if (m >= M) return;
    const float xs = x_scale[m * xs_step];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        v4i t = part[0][h][lane];
#pragma unroll
        for (int w = 1; w < 4; ++w) t += part[w][h][lane];
        const int n = n0 + 16 * h + 4 * (lane / 16);
        if (n >= N) continue;
        const int64_t off = (int64_t)m * N + n;
        constexpr int kTy = kOut & 1;
        if (kOut < 2) {  // N % 4 == 0: four consecutive outputs at once
            const float4 ws = *reinterpret_cast<const float4*>(w_scale + n);
            const float y0 = ((float)t[0] * xs) * ws.x, y1 = ((float)t[1] * xs) * ws.y;
            const float y2 = ((float)t[2] * xs) * ws.z, y3 = ((float)t[3] * xs) * ws.w;
            if constexpr (kTy == 0)
                *reinterpret_cast<uint2*>(static_cast<uint16_t*>(y) + off) =
                    make_uint2(pack_bf16x2(y0, y1), pack_bf16x2(y2, y3));
            else
                *reinterpret_cast<float4*>(static_cast<float*>(y) + off) = make_float4(y0, y1, y2, y3);
            if constexpr (kAcc) *reinterpret_cast<int4*>(acc_out + off) = make_int4(t[0], t[1], t[2], t[3]);
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                if (n + e >= N) break;
                const float v = ((float)t[e] * xs) * w_scale[n + e];
                if constexpr (kTy == 0)
                    static_cast<uint16_t*>(y)[off + e] = (uint16_t)(pack_bf16x2(v, 0.0f) & 0xFFFFu);
                else
                    static_cast<float*>(y)[off + e] = v;
                if constexpr (kAcc) acc_out[off + e] = t[e];
            }
        }
    }
}

// ---- decode kernel, LDS-ring variant (K % 2048 == 0, K <= 16384) ------------------
//
// Same product as k_gemm_decode, streamed so that every load instruction reads
// whole 128-byte lines: one block of 16 wavefronts per CU; wavefront w owns
// the SPW = K / 2048 chunks of 128 k-bytes that start at byte 2048 sp + 128 w,
// sp < SPW (so at stage sp the 16 wavefronts read one contiguous 2 KB of every
// row of the group), and keeps the token operand of those chunks in registers
// for the whole kernel.  Work items are groups of 16 output channels, dealt
// round-robin to the blocks.  A stage is 16 weight rows x 128 bytes, copied by
// two global_load_lds_dwordx4 (8 rows x 128 bytes each, nontemporal: the
// stream is read once) into the wavefront's own NST-stage LDS ring; chunk c of
// row r sits at slot 8 r + (c ^ ((r >> 1) & 7)), so the MFMA fragment reads
// are conflict-free.  No workgroup barrier guards the rings (each is private
// to a wavefront); only explicit vmcnt waits do, and no other vector-memory
// instruction runs during the stream: scales are staged in LDS first, the 16
// partial tiles of a group are summed through LDS by one wavefront, which
// keeps the int32 sum in registers, and the epilogue and all stores run after
// the last stage.

constexpr int kDrWaves = 16, kDrStages = 3, kDrStageBytes = 128, kDrMaxGroups = 24;
constexpr int kDrSums = (kDrMaxGroups + kDrWaves - 1) / kDrWaves;  // groups summed per wavefront

__device__ __forceinline__ void copy16_to_lds_nt(const int8_t* base, uint32_t voff, uint32_t lds_off) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2 nt"
                 :
                 : "s"(lds_off), "v"(voff), "s"(base)
                 : "memory", "m0");
}

template <int SPW>
__global__ __launch_bounds__(64 * kDrWaves) void k_gemm_decode_ring(
    const int8_t* __restrict__ xq, const float* __restrict__ x_scale, int xs_step, const int8_t* __restrict__ wq,
    const float* __restrict__ w_scale, int M, int N, int K, void* __restrict__ y, bool y_bf16,
    int32_t* __restrict__ acc_out) {
    constexpr int NW = kDrWaves, NST = kDrStages, SB = kDrStageBytes;
    constexpr int CPR = SB / 16;     // 16-byte chunks per row per stage (8)
    constexpr int SLOTS = 16 * CPR;  // 16-byte slots per stage
    constexpr int NCP = SB / 64;     // copies per stage (2), 8 rows each
    constexpr int RPC = 1024 / SB;   // rows per copy
    constexpr int KS = SB / 64;      // MFMA k-steps per stage
    __shared__ uint4 ring_all[NW * NST * SLOTS];
    __shared__ v4i part[NW * 64];
    __shared__ __align__(16) float wsl[kDrMaxGroups * 16];
    __shared__ float xsl[16];
    auto h = [](int r) { return (r >> 1) & 7; };
    const int lane = threadIdx.x % kWave;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int G = (N + 15) / 16;
    const int ngroups = (G - (int)blockIdx.x + (int)gridDim.x - 1) / (int)gridDim.x;
    // k-chunks of this wavefront: stage sp covers bytes sp * NW * SB + wave * SB .. + SB of the rows, so
    // at each stage the 16 wavefronts read one contiguous NW * SB bytes of every row of the group
    auto kofs = [&](int sp) { return sp * (NW * SB) + wave * SB; };

    const uint32_t ring = (uint32_t)(uintptr_t)(lds_char*)(ring_all + wave * NST * SLOTS);
    const int rr = lane / CPR, cl = lane % CPR;
    const int T = ngroups * SPW;  // stages of this wavefront
    auto issue = [&](int t) {
        const int gi = t / SPW, sp = t % SPW;
        const int g = (int)blockIdx.x + gi * (int)gridDim.x;
        const uint32_t la = __builtin_amdgcn_readfirstlane(ring + (uint32_t)((t % NST) * SLOTS * 16));
#pragma unroll
        for (int i = 0; i < NCP; ++i) {
            const int r = RPC * i + rr;
            const int n = min(16 * g + r, N - 1);
            const uint32_t off = (uint32_t)n * (uint32_t)K + (uint32_t)(kofs(sp) + 16 * (cl ^ h(r)));
            copy16_to_lds_nt(wq, off, la + i * 1024);
        }
    };
    // the weight stream starts first; the token operand loads while its first stages are in flight
#pragma unroll
    for (int t = 0; t < NST - 1; ++t)
        if (t < T) issue(t);

    // token operand: lane l holds token l % 16, 16-byte chunk l / 16 of each 64-byte k-step
    v4i xb[SPW][KS];
    {
        const int8_t* xr = xq + (int64_t)min(lane % 16, M - 1) * K + 16 * (lane / 16);
#pragma unroll
        for (int sp = 0; sp < SPW; ++sp)
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                const uint4 u = ld16(xr + kofs(sp) + s * 64);
                xb[sp][s] = v4i{(int)u.x, (int)u.y, (int)u.z, (int)u.w};
            }
        if (threadIdx.x < 16) xsl[threadIdx.x] = x_scale[min((int)threadIdx.x, M - 1) * xs_step];
    }
    // consume the operand here so the compiler's own waits for these loads come
    // before the stream and never inside it
#pragma unroll
    for (int sp = 0; sp < SPW; ++sp)
#pragma unroll
        for (int s = 0; s < KS; ++s) asm volatile("" ::"v"(xb[sp][s]));
    for (int i = threadIdx.x; i < ngroups * 16; i += 64 * NW) {
        const int g = (int)blockIdx.x + (i / 16) * (int)gridDim.x;
        wsl[i] = w_scale[min(16 * g + i % 16, N - 1)];
    }
    wait_vmcnt<0>();
    __syncthreads();  // the staged scales

    v4i acc = {0, 0, 0, 0};
    v4i sums[kDrSums];
#pragma unroll
    for (int q = 0; q < kDrSums; ++q) sums[q] = v4i{0, 0, 0, 0};
    const int fr = lane % 16, fc = lane / 16;
    for (int gi = 0; gi < ngroups; ++gi) {
#pragma unroll
        for (int sp = 0; sp < SPW; ++sp) {
            const int t = gi * SPW + sp;
            if (t + NST - 1 < T) {
                issue(t + NST - 1);
                wait_vmcnt<NCP*(NST - 1)>();  // stage t has landed; the later ones stay in flight
            } else {
                wait_vmcnt<0>();
            }
            const uint4* st = ring_all + wave * NST * SLOTS + (t % NST) * SLOTS;
            v4i fa[KS];
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                const uint4 u = st[CPR * fr + ((4 * s + fc) ^ h(fr))];
                fa[s] = v4i{(int)u.x, (int)u.y, (int)u.z, (int)u.w};
            }
#pragma unroll
            for (int s = 0; s < KS; ++s) acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(fa[s], xb[sp][s], acc, 0, 0, 0);
        }
        // group done: the 16 partial tiles are summed by wavefront gi % NW
        part[wave * 64 + lane] = acc;
        acc = v4i{0, 0, 0, 0};
        lds_barrier();
        if (wave == (gi % NW)) {
            v4i sum = part[lane];
#pragma unroll
            for (int w = 1; w < NW; ++w) sum += part[w * 64 + lane];
#pragma unroll
            for (int q = 0; q < kDrSums; ++q)
                if (gi / NW == q) sums[q] = sum;
        }
        lds_barrier();  // part is reused by the next group
    }

    // epilogue: wavefront w stores the groups gi = w + NW q; 16x16 accumulator
    // layout, lane l holds channels 4 (l / 16) + e of token l % 16
#pragma unroll
    for (int q = 0; q < kDrSums; ++q) {
        const int gi = wave + NW * q;
        if (gi >= ngroups) break;
        const int g = (int)blockIdx.x + gi * (int)gridDim.x;
        const int m = lane % 16, n = 16 * g + 4 * (lane / 16);
        if (m >= M || n >= N) continue;
        const v4i sum = sums[q];
        const float xs = xsl[m];
        const float* ws = wsl + gi * 16 + 4 * (lane / 16);
        const int64_t off = (int64_t)m * N + n;
        if (n + 3 < N && N % 4 == 0) {
            const float y0 = ((float)sum[0] * xs) * ws[0], y1 = ((float)sum[1] * xs) * ws[1];
            const float y2 = ((float)sum[2] * xs) * ws[2], y3 = ((float)sum[3] * xs) * ws[3];
            if (y_bf16)
                *reinterpret_cast<uint2*>(static_cast<uint16_t*>(y) + off) =
                    make_uint2(pack_bf16x2(y0, y1), pack_bf16x2(y2, y3));
            else
                *reinterpret_cast<float4*>(static_cast<float*>(y) + off) = make_float4(y0, y1, y2, y3);
            if (acc_out) *reinterpret_cast<int4*>(acc_out + off) = make_int4(sum[0], sum[1], sum[2], sum[3]);
        } else {
            for (int e = 0; e < 4 && n + e < N; ++e) {
                const float v = ((float)sum[e] * xs) * ws[e];
                if (y_bf16)
                    static_cast<uint16_t*>(y)[off + e] = (uint16_t)(pack_bf16x2(v, 0.0f) & 0xFFFFu);
                else
                    static_cast<float*>(y)[off + e] = v;
                if (acc_out) acc_out[off + e] = sum[e];
            }
        }
    }
}

// Compute units of the current device, queried once per device.  The cache
// is read and written atomically (relaxed: every thread that fills an entry
// stores the same value), so concurrent first calls from several host threads
// are safe.
static int device_cu_count() {
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int n = cache[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cache[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

static bool decode_ring_fits(int64_t M, int64_t N, int64_t K) {
    if (M > 16 || K < 2048 || K % 2048 != 0 || K > 16384 || (uint64_t)N * (uint64_t)K >= (1ull << 32)) return false;
    const int64_t G = (N + 15) / 16;
    const int64_t grid = std::min<int64_t>(device_cu_count(), G);
    return (G + grid - 1) / grid <= kDrMaxGroups;
}

static void launch_decode_ring(const int8_t* xq, const float* x_scale, bool per_tensor, const int8_t* wq,
                               const float* w_scale, int M, int N, int K, void* y, bool y_bf16, int32_t* acc_out,
                               hipStream_t st) {
    const int G = (N + 15) / 16;
    const dim3 grid((unsigned)std::min(device_cu_count(), G));
    const int step = per_tensor ? 0 : 1;
#define SQ_DR(S)                                                                                                   \
    hipLaunchKernelGGL((k_gemm_decode_ring<S>), grid, dim3(64 * kDrWaves), 0, st, xq, x_scale, step, wq, w_scale, M, \
                       N, K, y, y_bf16, acc_out)
    switch (K / 2048) {
        case 1: SQ_DR(1); break;
        case 2: SQ_DR(2); break;
        case 3: SQ_DR(3); break;
        case 4: SQ_DR(4); break;
        case 5: SQ_DR(5); break;
        case 6: SQ_DR(6); break;
        case 7: SQ_DR(7); break;
        default: SQ_DR(8); break;
    }
#undef SQ_DR
}

static void launch_decode(const int8_t* xq, const float* x_scale, bool per_tensor, const int8_t* wq,
                          const float* w_scale, int M, int N, int K, void* y, bool y_bf16, int32_t* acc_out,
                          hipStream_t st) {
    const dim3 grid((unsigned)((N + 31) / 32));
    const int step = per_tensor ? 0 : 1;
    const int out = (y_bf16 ? 0 : 1) + (N % 4 == 0 ? 0 : 2);
    auto go = [&](auto out_c, auto acc_c) {
        hipLaunchKernelGGL((k_gemm_decode<decltype(out_c)::value, decltype(acc_c)::value>), grid, dim3(256), 0, st,
                           xq, x_scale, step, wq, w_scale, M, N, K, y, acc_out);
    };
    using T_ = std::true_type;
    using F_ = std::false_type;
    switch (out) {
        case 0: if (acc_out) go(std::integral_constant<int, 0>{}, T_{}); else go(std::integral_constant<int, 0>{}, F_{}); break;
        case 1: if (acc_out) go(std::integral_constant<int, 1>{}, T_{}); else go(std::integral_constant<int, 1>{}, F_{}); break;
        case 2: if (acc_out) go(std::integral_constant<int, 2>{}, T_{}); else go(std::integral_constant<int, 2>{}, F_{}); break;
        default: if (acc_out) go(std::integral_constant<int, 3>{}, T_{}); else go(std::integral_constant<int, 3>{}, F_{}); break;
    }
}

// ---- launchers ---------------------------------------------------------------------


// Calls go(out, acc, o) with compile-time constants for the output mode
// (0 bf16, 1 fp32, +2 when N % 4 != 0), the int32 accumulator store and the
// 16-bit outlier addend (built without the accumulator store).
template <typename Go>
static void dispatch_variant(bool y_bf16, int N, int ldy, bool acc, bool outl, Go&& go) {
    using T_ = std::true_type;
    using F_ = std::false_type;
    const int out = (y_bf16 ? 0 : 1) + (N % 4 == 0 && ldy % 4 == 0 ? 0 : 2);
    auto by_out = [&](auto a, auto o) {
        switch (out) {
            case 0: go(std::integral_constant<int, 0>{}, a, o); break;
            case 1: go(std::integral_constant<int, 1>{}, a, o); break;
            case 2: go(std::integral_constant<int, 2>{}, a, o); break;
            default: go(std::integral_constant<int, 3>{}, a, o); break;
        }
    };
    if (outl) by_out(F_{}, T_{});
    else if (acc) by_out(T_{}, F_{});
    else by_out(F_{}, F_{});
}

template <int BN, int BM>
static void launch_generic(const int8_t* xq, const float* x_scale, bool per_tensor, const int8_t* wq,
                           const float* w_scale, int M, int N, int K, void* y, bool y_bf16, int32_t* acc_out,
                           const OutlierOps* op, int group_m, hipStream_t st) {
    const int tiles_n = (N + BN - 1) / BN, tiles_m = (M + BM - 1) / BM;
    const dim3 grid((unsigned)(tiles_n * tiles_m));
    const int step = per_tensor ? 0 : 1;  // x_scale index step
    const OutlierOps ops = op ? *op : OutlierOps{};
    dispatch_variant(y_bf16, N, N, acc_out != nullptr, op != nullptr, [&](auto out_c, auto acc_c, auto o_c) {
        hipLaunchKernelGGL((k_gemm_generic<BN, BM, decltype(out_c)::value, decltype(acc_c)::value,
                                           decltype(o_c)::value>),
                           grid, dim3(256), 0, st, xq, x_scale, step, wq, w_scale, M, N, K, y, N, acc_out, tiles_n,
                           tiles_m, group_m, ops);
    });
}

// Columns [n0, n0 + N) of the product (wq, w_scale, the outlier rows and the
// output start at column n0; ldy is the output's row stride).
template <int BN, int BM, int WGN, int WGM, int NS>
static void launch_ring(const int8_t* xq, const float* x_scale, bool per_tensor, const int8_t* wq,
                        const float* w_scale, int M, int N, int K, void* y, bool y_bf16, int32_t* acc_out,
                        const OutlierOps* op, int group_m, hipStream_t st, int n0 = 0, int ldy = -1) {
    if (ldy < 0) ldy = N;
    const int tiles_n = (N + BN - 1) / BN, tiles_m = (M + BM - 1) / BM;
    const dim3 grid((unsigned)(tiles_n * tiles_m));
    const int step = per_tensor ? 0 : 1;
    OutlierOps ops = op ? *op : OutlierOps{};
    if (op) ops.w_ot += (int64_t)n0 * ops.kp;
    void* yc = static_cast<char*>(y) + (int64_t)n0 * (y_bf16 ? 2 : 4);
    int32_t* accc = acc_out ? acc_out + n0 : nullptr;
    dispatch_variant(y_bf16, N, ldy, acc_out != nullptr, op != nullptr, [&](auto out_c, auto acc_c, auto o_c) {
        hipLaunchKernelGGL((k_gemm_ring<BN, BM, WGN, WGM, NS, decltype(out_c)::value, decltype(acc_c)::value,
                                        decltype(o_c)::value>),
                           grid, dim3(64 * WGN * WGM), 0, st, xq, x_scale, step, wq + (int64_t)n0 * K,
                           w_scale + n0, M, N, K, yc, ldy, accc, tiles_n, tiles_m, group_m, ops);
    });
}

// The 256 x 256 product through the persistent kernel when the call is the
// deployed one (bf16 output, no accumulator store, no outlier addend, N and
// the output stride multiples of 8, K a multiple of 256); returns false (and
// launches nothing) otherwise.  Columns [n0, n0 + N) as launch_ring.
static bool launch_persist256(const int8_t* xq, const float* x_scale, bool per_tensor, const int8_t* wq,
                              const float* w_scale, int M, int N, int K, void* y, bool y_bf16, int32_t* acc_out,
                              const OutlierOps* op, int group_m, hipStream_t st, int n0 = 0, int ldy = -1) {
    if (ldy < 0) ldy = N;
    if (!y_bf16 || acc_out || op || N % 8 != 0 || ldy % 8 != 0 || K % 256 != 0 || K < 256) return false;
    const int tiles_n = (N + 255) / 256, tiles_m = (M + 255) / 256, ntiles = tiles_n * tiles_m;
    const int cus = (int)std::max<int64_t>(8, device_cu_count() / 8 * 8);
    const int grid = std::min(ntiles, cus);
    hipLaunchKernelGGL((k_gemm_persist<256, 256, 4, 2, 2>), dim3((unsigned)grid), dim3(512), 0, st, xq, x_scale,
                       per_tensor ? 0 : 1, wq + (int64_t)n0 * K, w_scale + n0, M, N, K,
                       static_cast<uint16_t*>(y) + n0, ldy, tiles_n, tiles_m, group_m, ntiles);
    return true;
}

// Which kernel a product of this shape runs (the one rule both the launcher
// and gemm_kernel_name use).
enum class GemmPath { kNone, kDecodeRing, kDecode, kRing256, kRing256Split, kRing256x128, kRing128, kGeneric };

// When the last round of 256 x 256 tiles over the CUs is at most half full,
// the columns split: the first n1 columns hold whole rounds of 256 x 256
// tiles, the rest run as one more launch of 256 x 128 tiles that fills at
// most one round.  Returns n1 (a multiple of 256), or 0 when no such split
// exists.
static int64_t ring256_split_cols(int64_t M, int64_t N, int64_t cus) {
    const int64_t tm = (M + 255) / 256, tn = (N + 255) / 256;
    const int64_t tiles = tm * tn, full = tiles / cus, rest = tiles - full * cus;
    if (full == 0 || rest == 0 || 2 * rest > cus || (full * cus) % tm != 0) return 0;
    const int64_t tn1 = full * cus / tm;
    if (tn1 >= tn) return 0;
    const int64_t tail = ((N - tn1 * 256 + 255) / 256) * ((M + 127) / 128);
    return tail <= cus ? tn1 * 256 : 0;
}

static GemmPath gemm_path(int64_t M, int64_t N, int64_t K, bool outl = false) {
    if (M <= 0 || N <= 0) return GemmPath::kNone;
    if (M <= 16 && K > 0 && !outl) return decode_ring_fits(M, N, K) ? GemmPath::kDecodeRing : GemmPath::kDecode;
    const bool ring = K > 0 && K % kBK == 0 && (uint64_t)N * (uint64_t)K < (1ull << 32) &&
                      (uint64_t)M * (uint64_t)K < (1ull << 32);
    if (!ring) return GemmPath::kGeneric;
    // Tile shape by estimated time: rounds of tiles over the CUs, each round
    // weighted by the measured time of a stage per CU relative to 256 x 128
    // tiles (one block per CU, three-stage 144 KB ring): 256 x 256 tiles (one
    // block per CU, two-stage 128 KB ring) take about 1.6x for twice the work,
    // a CU running two 128 x 128 blocks about 1.2x.  Weights x5 in integers;
    // ties go to the larger tile.
    const int64_t cus = device_cu_count();
    const int64_t t256 = ((N + 255) / 256) * ((M + 255) / 256);
    const int64_t t_wide = ((N + 255) / 256) * ((M + 127) / 128);
    const int64_t t128 = ((N + 127) / 128) * ((M + 127) / 128);
    const int64_t c256 = 8 * ((t256 + cus - 1) / cus);
    const int64_t c_wide = 5 * ((t_wide + cus - 1) / cus);
    const int64_t c128 = 6 * ((t128 + 2 * cus - 1) / (2 * cus));
    const int64_t split = ring256_split_cols(M, N, cus);
    const int64_t c_split = split > 0 ? 8 * (t256 / cus) + 5 : INT64_MAX;
    if (c256 <= c_wide && c256 <= c128 && c256 <= c_split) return GemmPath::kRing256;
    if (c_split <= c_wide && c_split <= c128) return GemmPath::kRing256Split;
    if (c_wide <= c128) return GemmPath::kRing256x128;
    return GemmPath::kRing128;
}

const char* gemm_kernel_name(int64_t M, int64_t N, int64_t K, bool outl) {
    switch (gemm_path(M, N, K, outl)) {
        case GemmPath::kDecodeRing:
            return "k_gemm_decode_ring (one block of 16 wavefronts per CU, per-wavefront LDS rings of 128-byte stages)";
        case GemmPath::kDecode: return "k_gemm_decode (32 output channels per block, K split over 4 wavefronts)";
        case GemmPath::kRing256:
            if (!outl && K % 256 == 0)
                return "k_gemm_persist<256,256,4,2,2> (one block per CU walking 256x256 tiles, 8 wavefronts of 64x128, "
                       "2 stages) for bf16 output without accumulator store and N % 8 == 0, else k_gemm_ring<256,256,4,2,2>";
            return "k_gemm_ring<256,256,4,2,2> (256x256 tile, 8 wavefronts of 64x128, 2 stages)";
        case GemmPath::kRing256Split:
            if (!outl && K % 256 == 0)
                return "k_gemm_persist<256,256,4,2,2> (or k_gemm_ring<256,256,4,2,2>) on whole rounds of columns + "
                       "k_gemm_ring<256,128,4,2,3> on the remaining columns (one round)";
            return "k_gemm_ring<256,256,4,2,2> on whole rounds of columns + k_gemm_ring<256,128,4,2,3> on the "
                   "remaining columns (one round)";
        case GemmPath::kRing256x128:
            return "k_gemm_ring<256,128,4,2,3> (256x128 tile, 8 wavefronts of 64x64, 3 stages)";
        case GemmPath::kRing128: return "k_gemm_ring<128,128,2,4,2> (128x128 tile, 8 wavefronts of 64x32, 2 stages)";
        case GemmPath::kGeneric: return "k_gemm_generic<256,128> (register-staged, any K % 16 == 0)";
        default: return "none (empty product)";
    }
}

static hipError_t launch_gemm(const int8_t* xq, const float* x_scale, bool per_tensor, const int8_t* wq,
                              const float* w_scale, int64_t M64, int64_t N64, int64_t K64, void* y, bool y_bf16,
                              int32_t* acc_out, const OutlierOps* op, hipStream_t st) {
    const int M = (int)M64, N = (int)N64, K = (int)K64;
    switch (gemm_path(M64, N64, K64, op != nullptr)) {
        case GemmPath::kNone: return hipSuccess;
        case GemmPath::kDecodeRing:
            launch_decode_ring(xq, x_scale, per_tensor, wq, w_scale, M, N, K, y, y_bf16, acc_out, st);
            break;
        case GemmPath::kDecode:
            launch_decode(xq, x_scale, per_tensor, wq, w_scale, M, N, K, y, y_bf16, acc_out, st);
            break;
        case GemmPath::kRing256:
            if (!launch_persist256(xq, x_scale, per_tensor, wq, w_scale, M, N, K, y, y_bf16, acc_out, op, 4, st))
                launch_ring<256, 256, 4, 2, 2>(xq, x_scale, per_tensor, wq, w_scale, M, N, K, y, y_bf16, acc_out, op,
                                               4, st);
            break;
        case GemmPath::kRing256Split: {
            const int n1 = (int)ring256_split_cols(M64, N64, device_cu_count());
            if (!launch_persist256(xq, x_scale, per_tensor, wq, w_scale, M, n1, K, y, y_bf16, acc_out, op, 4, st, 0, N))
                launch_ring<256, 256, 4, 2, 2>(xq, x_scale, per_tensor, wq, w_scale, M, n1, K, y, y_bf16, acc_out, op,
                                               4, st, 0, N);
            launch_ring<256, 128, 4, 2, 3>(xq, x_scale, per_tensor, wq, w_scale, M, N - n1, K, y, y_bf16, acc_out, op,
                                           8, st, n1, N);
            break;
        }
        case GemmPath::kRing256x128:
            launch_ring<256, 128, 4, 2, 3>(xq, x_scale, per_tensor, wq, w_scale, M, N, K, y, y_bf16, acc_out, op, 4,
                                           st);
            break;
        case GemmPath::kRing128:
            launch_ring<128, 128, 2, 4, 2>(xq, x_scale, per_tensor, wq, w_scale, M, N, K, y, y_bf16, acc_out, op, 8,
                                           st);
            break;
        case GemmPath::kGeneric:
            launch_generic<256, 128>(xq, x_scale, per_tensor, wq, w_scale, M, N, K, y, y_bf16, acc_out, op, 8, st);
            break;
    }
    return hipGetLastError();
}

hipError_t launch_gemm_w8a8(const int8_t* xq, const float* x_scale, bool per_tensor, const int8_t* wq,
                            const float* w_scale, int64_t M, int64_t N, int64_t K, void* y, bool y_bf16,
                            int32_t* acc_out, hipStream_t st) {
    return launch_gemm(xq, x_scale, per_tensor, wq, w_scale, M, N, K, y, y_bf16, acc_out, nullptr, st);
}

hipError_t launch_gemm_w8a8_outlier(const int8_t* xq, const float* x_scale, const int8_t* wq, const float* w_scale,
                                    int64_t M, int64_t N, int64_t K, const uint16_t* x_o, const uint16_t* w_ot,
                                    int64_t kp, const int32_t* count, void* y, bool y_bf16, hipStream_t st) {
    const OutlierOps op{x_o, w_ot, count, kp};
    return launch_gemm(xq, x_scale, false, wq, w_scale, M, N, K, y, y_bf16, nullptr, &op, st);
}

}  // namespace sqk
