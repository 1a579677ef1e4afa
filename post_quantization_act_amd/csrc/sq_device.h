// Device-side helpers shared by the gfx950 kernels of the library.
#pragma once

#include <hip/hip_runtime.h>
#include <type_traits>
#include <stdint.h>

namespace sqk {

constexpr int kWave = 64;  // CDNA wavefront width

// Element types the kernels read.  A bf16 value is carried as its 16-bit
// pattern; widening to fp32 places it in the upper half (exact).
struct bf16_t {
    uint16_t bits;
};

template <typename T>
struct Elem;

template <>
struct Elem<bf16_t> {
    static constexpr int kPerVec = 8;  // elements per 16-byte load
};

template <>
struct Elem<float> {
    static constexpr int kPerVec = 4;
};

__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xFFFF0000u); }

// 16-byte global load (one global_load_dwordx4).
__device__ __forceinline__ uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }

// 16-byte streaming load: the nontemporal hint marks data read once, which
// keeps it from displacing reused lines and lifts HBM read throughput.
typedef unsigned v4u_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld16_stream(const void* p) {
    const v4u_t t = __builtin_nontemporal_load(reinterpret_cast<const v4u_t*>(p));
    return make_uint4(t.x, t.y, t.z, t.w);
}

// Buffer descriptor of `bytes` bytes at p (raw buffer, no stride): loads at
// offsets at or past `bytes` return zero and do not access memory.  The
// fourth dword is the gfx9-family default for 32-bit raw accesses.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_rsrc(const void* p, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, bytes, 0x00020000);
}

// 16-byte buffer load at byte offset off with the nontemporal hint (zero when
// off is out of the descriptor's range).
__device__ __forceinline__ uint4 ld16_buf_stream(__amdgpu_buffer_rsrc_t rs, int off) {
    const v4u_t t = __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 2);
    return make_uint4(t.x, t.y, t.z, t.w);
}

// 4-byte buffer load at byte offset off (zero out of range).
__device__ __forceinline__ float ld4_buf(__amdgpu_buffer_rsrc_t rs, int off) {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, off, 0, 0));
}

// Streaming stores (nontemporal hint) for outputs written once.
__device__ __forceinline__ void st16_stream(void* p, uint4 v) {
    __builtin_nontemporal_store(v4u_t{v.x, v.y, v.z, v.w}, reinterpret_cast<v4u_t*>(p));
}
typedef unsigned v2u_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void st8_stream(void* p, uint2 v) {
    __builtin_nontemporal_store(v2u_t{v.x, v.y}, reinterpret_cast<v2u_t*>(p));
}

// Widen the 8 consecutive elements at p (16-byte aligned) to fp32.
__device__ __forceinline__ void load8(const bf16_t* p, float (&v)[8]) {
    uint4 q = ld16_stream(p);
    v[0] = bf16_lo(q.x); v[1] = bf16_hi(q.x);
    v[2] = bf16_lo(q.y); v[3] = bf16_hi(q.y);
    v[4] = bf16_lo(q.z); v[5] = bf16_hi(q.z);
    v[6] = bf16_lo(q.w); v[7] = bf16_hi(q.w);
}

__device__ __forceinline__ void load8(const float* p, float (&v)[8]) {
    uint4 a = ld16_stream(p), b = ld16_stream(p + 4);
    v[0] = __uint_as_float(a.x); v[1] = __uint_as_float(a.y);
    v[2] = __uint_as_float(a.z); v[3] = __uint_as_float(a.w);
    v[4] = __uint_as_float(b.x); v[5] = __uint_as_float(b.y);
    v[6] = __uint_as_float(b.z); v[7] = __uint_as_float(b.w);
}

// Bounds-checked variant for the ragged end of a row: elements at or beyond
// `n` (counted from p) read as 0.
template <typename T>
__device__ __forceinline__ void load8_tail(const T* p, int64_t n, float (&v)[8]) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        if (i < n) {
            if constexpr (sizeof(T) == 2) {
                v[i] = __uint_as_float(uint32_t(reinterpret_cast<const uint16_t*>(p)[i]) << 16);
            } else {
                v[i] = reinterpret_cast<const float*>(p)[i];
            }
        } else {
            v[i] = 0.0f;
        }
    }
}

// kVec: rows are 16-byte aligned, so a full group is one vector load;
// otherwise (a weight whose row stride is not a multiple of 16 bytes) every
// element is loaded on its own.
template <bool kVec = true, typename T>
__device__ __forceinline__ void load8_any(const T* p, int64_t n, float (&v)[8]) {
    if (kVec && n >= 8) load8(p, v);
    else load8_tail(p, n, v);
}

// True when every row of a matrix starts on a 16-byte boundary.
__host__ __device__ inline bool rows_aligned16(const void* p, int64_t ld, int64_t elem_bytes) {
    return (reinterpret_cast<uintptr_t>(p) & 15u) == 0 && (ld * elem_bytes) % 16 == 0;
}

// Max over the wavefront (all 64 lanes end with the result).
// Cross-lane reductions over a wavefront without the LDS crossbar: DPP moves
// inside each row of 16 lanes (lane ^ 1, lane ^ 2, the half-row mirror and the
// row mirror leave every lane of a row with the row's result), then the four
// rows' results read into scalar registers and combined, so every lane
// returns the wavefront's result.  Call with the whole wavefront active.
template <int kCtrl>
__device__ __forceinline__ int dpp_move(int v) {
    return __builtin_amdgcn_update_dpp(v, v, kCtrl, 0xF, 0xF, false);
}
constexpr int kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppHalfMirror = 0x141, kDppMirror = 0x140;

__device__ __forceinline__ float wave_max(float v) {
    auto step = [&](auto ctrl) {
        v = fmaxf(v, __int_as_float(dpp_move<decltype(ctrl)::value>(__float_as_int(v))));
    };
    step(std::integral_constant<int, kDppXor1>{});
    step(std::integral_constant<int, kDppXor2>{});
    step(std::integral_constant<int, kDppHalfMirror>{});
    step(std::integral_constant<int, kDppMirror>{});
    const int b = __float_as_int(v);
    return fmaxf(fmaxf(__int_as_float(__builtin_amdgcn_readlane(b, 0)), __int_as_float(__builtin_amdgcn_readlane(b, 16))),
                 fmaxf(__int_as_float(__builtin_amdgcn_readlane(b, 32)), __int_as_float(__builtin_amdgcn_readlane(b, 48))));
}

// Sum over a wavefront in fp64, by the same moves (each half of the double
// moved on its own).  The order of the additions differs from a sequential
// loop, so it is exact only where every partial sum is (integer values whose
// sums stay below 2^53, as the callers use it).
__device__ __forceinline__ double wave_sum_f64(double v) {
    auto step = [&](auto ctrl) {
        const uint64_t u = __builtin_bit_cast(uint64_t, v);
        const int lo = dpp_move<decltype(ctrl)::value>((int)(uint32_t)u);
        const int hi = dpp_move<decltype(ctrl)::value>((int)(uint32_t)(u >> 32));
        v += __builtin_bit_cast(double, ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo);
    };
    step(std::integral_constant<int, kDppXor1>{});
    step(std::integral_constant<int, kDppXor2>{});
    step(std::integral_constant<int, kDppHalfMirror>{});
    step(std::integral_constant<int, kDppMirror>{});
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    const int lo = (int)(uint32_t)u, hi = (int)(uint32_t)(u >> 32);
    auto lane = [&](int l) {
        return __builtin_bit_cast(double, ((uint64_t)(uint32_t)__builtin_amdgcn_readlane(hi, l) << 32) |
                                              (uint32_t)__builtin_amdgcn_readlane(lo, l));
    };
    return (lane(0) + lane(16)) + (lane(32) + lane(48));
}

// Symmetric INT8 code of v with multiplier r: clamp(rne(fl(v*r)), -127, 127).
// If the group max is so small that r = 127/max overflowed to +inf, a zero
// element gives 0 * inf = NaN, which codes to 0 (non-zero ones clamp).
__device__ __forceinline__ int code8(float v, float r) {
    float t = __builtin_rintf(v * r);
    t = (t == t) ? t : 0.0f;
    t = fminf(fmaxf(t, -127.0f), 127.0f);
    return static_cast<int>(t);
}

// Same code when r is finite (then v * r is finite and no NaN can arise):
// one v_med3_f32 clamps.
__device__ __forceinline__ int code8_finite(float v, float r) {
    const float t = __builtin_rintf(v * r);
    return static_cast<int>(__builtin_amdgcn_fmed3f(t, -127.0f, 127.0f));
}

// The code of v as the low byte of a float's bit pattern, for a group whose
// max magnitude m bounds |v| and whose r is finite: then |fl(v * r)| is at
// most 127 (1 + 2^-23)^2 < 127.5, so no clamp is needed, and adding
// 1.5 * 2^23 rounds fl(v * r) to an integer, half to even (the sum lies in
// [2^23, 2^24), where the unit in the last place is 1).  The sum's bits are
// 0x4B400000 + code, whose low byte is the code in two's complement.  The
// product and the sum round separately (contraction is off), so the byte
// equals code8_finite(v, r).
__device__ __forceinline__ uint32_t code8_bounded_bits(float v, float r) {
    return __float_as_uint(v * r + 12582912.0f);
}

// Pack the low bytes of four code8_bounded_bits patterns (a first).
__device__ __forceinline__ uint32_t pack4_low(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
    const uint32_t ab = __builtin_amdgcn_perm(b, a, 0x0c0c0400u);  // a.byte0, b.byte0, 0, 0
    const uint32_t cd = __builtin_amdgcn_perm(d, c, 0x0c0c0400u);
    return __builtin_amdgcn_perm(cd, ab, 0x05040100u);
}

// Pack four codes (low byte first) into one dword.
__device__ __forceinline__ uint32_t pack4(int a, int b, int c, int d) {
    return (uint32_t(a) & 0xFFu) | ((uint32_t(b) & 0xFFu) << 8) | ((uint32_t(c) & 0xFFu) << 16) |
           (uint32_t(d) << 24);
}

// Scale and multiplier of a group with max magnitude m (m >= 0):
// scale = fl(m / 127), r = fl(127 / m), r = 0 when m = 0.  Both are
// correctly rounded fp32 divisions.
__device__ __forceinline__ void group_scale(float m, float& scale, float& r) {
    scale = m / 127.0f;
    r = m > 0.0f ? 127.0f / m : 0.0f;
}

// fp32 -> bf16 bits, round to nearest even (gfx950 v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
    bf2 r;
    r.x = static_cast<__bf16>(lo);
    r.y = static_cast<__bf16>(hi);
    return __builtin_bit_cast(uint32_t, r);
}

}  // namespace sqk
