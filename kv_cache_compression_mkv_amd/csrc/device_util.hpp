// Device helpers for gfx950 (wave64): storage conversions and wave primitives.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mkv {

// ---- storage element types -------------------------------------------------
struct Bf16 {
    using bits_t = uint16_t;
    static constexpr int bytes = 2;
};
struct F32 {
    using bits_t = uint32_t;
    static constexpr int bytes = 4;
};

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// binary64 -> bfloat16 bits, round to nearest even in one step.
// Round to odd into binary32 first (truncate the binary64 significand and
// set the last kept bit when anything nonzero was cut off), then round
// binary32 -> bfloat16 to nearest even. Binary32 keeps 16 more significand
// bits than bfloat16 in every range, normal and subnormal, and an odd-rounded
// intermediate with at least two extra bits makes the second rounding equal
// to a direct one (Boldo and Melquiond, "Emulation of FMA and correctly
// rounded sums: proved algorithms using rounding to odd", IEEE Trans.
// Computers 57(4), 2008).
__device__ __forceinline__ uint16_t f64_to_bf16(double x) {
    const uint64_t b = (uint64_t)__double_as_longlong(x);
    const uint32_t sign = (uint32_t)(b >> 48) & 0x8000u;
    const uint32_t ah = (uint32_t)(b >> 32) & 0x7FFFFFFFu, lo = (uint32_t)b;
    if (ah - 0x38100000u < 0x47F00000u - 0x38100000u) {
        // 2^-126 <= |x| < 2^128 (binary32 normal range): rebias the exponent,
        // keep the top 23 fraction bits and OR in the sticky bit of the rest
        const uint32_t f = ((ah - 0x38000000u) << 3) | (lo >> 29) | ((lo & 0x1FFFFFFFu) != 0u ? 1u : 0u);
        return (uint16_t)(sign | ((f + 0x7FFFu + ((f >> 16) & 1u)) >> 16));
    }
    const int ex = (int)((b >> 52) & 0x7ff);
    const uint64_t m = b & 0xFFFFFFFFFFFFFull;
    if (ex == 0x7ff) return (uint16_t)(sign | (m ? 0x7FC0u : 0x7F80u));
    const int E = ex - 1023;
    uint32_t f;  // |x| rounded to odd, as binary32 bits
    if (ex == 0) {
        f = m ? 1u : 0u;  // binary64 subnormal: far below bf16; keeps only its sticky bit
    } else if (E > 127) {
        f = 0x7F7FFFFFu;  // beyond binary32: largest odd finite, rounds to inf below
    } else if (E >= -126) {
        f = ((uint32_t)(E + 127) << 23) | (uint32_t)(m >> 29) | (uint32_t)((m & 0x1FFFFFFFull) != 0);
    } else {
        const uint64_t sig = m | (1ull << 52);
        const int sh = -97 - E;  // binary32 subnormal quantum is 2^-149
        if (sh >= 64) {
            f = 1u;
        } else {
            f = (uint32_t)(sig >> sh) | (uint32_t)((sig & ((1ull << sh) - 1)) != 0);
        }
    }
    const uint32_t r = (f + 0x7FFFu + ((f >> 16) & 1u)) >> 16;
    return (uint16_t)(sign | r);
}

// binary64 -> binary32 bits: the hardware conversion rounds to nearest even.
__device__ __forceinline__ uint32_t f64_to_f32_bits(double x) { return __float_as_uint((float)x); }

template <typename ST>
__device__ __forceinline__ typename ST::bits_t round_store(double x);
template <>
__device__ __forceinline__ uint16_t round_store<Bf16>(double x) { return f64_to_bf16(x); }
template <>
__device__ __forceinline__ uint32_t round_store<F32>(double x) { return f64_to_f32_bits(x); }

template <typename ST>
__device__ __forceinline__ float bits_to_float(typename ST::bits_t v);
template <>
__device__ __forceinline__ float bits_to_float<Bf16>(uint16_t v) { return __uint_as_float((uint32_t)v << 16); }
template <>
__device__ __forceinline__ float bits_to_float<F32>(uint32_t v) { return __uint_as_float(v); }

// IEEE totalOrder key of a stored value (unsigned compare = value order, -0 < +0).
template <typename ST>
__device__ __forceinline__ uint32_t order_key(typename ST::bits_t v);
template <>
__device__ __forceinline__ uint32_t order_key<Bf16>(uint16_t v) {
    const uint32_t u = v;
    return (u & 0x8000u) ? (~u & 0xFFFFu) : (u | 0x8000u);
}
template <>
__device__ __forceinline__ uint32_t order_key<F32>(uint32_t v) {
    return (v & 0x80000000u) ? ~v : (v | 0x80000000u);
}
template <typename ST>
__device__ __forceinline__ typename ST::bits_t key_to_bits(uint32_t k);
template <>
__device__ __forceinline__ uint16_t key_to_bits<Bf16>(uint32_t k) {
    return (uint16_t)((k & 0x8000u) ? (k & 0x7FFFu) : (~k & 0xFFFFu));
}
template <>
__device__ __forceinline__ uint32_t key_to_bits<F32>(uint32_t k) {
    return (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
}

// order-preserving key of a float32 score (larger score -> larger key)
__device__ __forceinline__ uint32_t score_key(float s) {
    const uint32_t u = __float_as_uint(s);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// ---- wave64 primitives ------------------------------------------------------
__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & 63); }
__device__ __forceinline__ uint64_t lanes_below(int lane) { return (lane == 0) ? 0ull : (~0ull >> (64 - lane)); }
// number of set bits of m at lanes below this one (mbcnt: no 64-bit mask held)
__device__ __forceinline__ int rank_below(uint64_t m) {
    return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}
__device__ __forceinline__ int popc64(uint64_t m) { return __popcll(m); }
__device__ __forceinline__ uint64_t ballot(bool p) { return __ballot(p); }

template <typename T>
__device__ __forceinline__ T shfl_xor(T v, int m) { return __shfl_xor(v, m, 64); }

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}
__device__ __forceinline__ int wave_sum_i(int v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}
__device__ __forceinline__ uint32_t wave_max_u(uint32_t v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, o, 64));
    return v;
}
__device__ __forceinline__ uint32_t wave_min_u(uint32_t v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = min(v, (uint32_t)__shfl_xor((int)v, o, 64));
    return v;
}

// make the wave's LDS writes visible to the wave's later LDS reads
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

}  // namespace mkv
