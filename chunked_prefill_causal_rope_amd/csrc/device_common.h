// Device-side helpers shared by the gfx950 kernels: vector types for the
// matrix-core builtins, bfloat16 bit conversions, wave reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// 16-byte global/LDS accesses as native vectors (no struct copies).
__device__ __forceinline__ u32x4_t ld16(const void* p) { return *reinterpret_cast<const u32x4_t*>(p); }
__device__ __forceinline__ void st16(void* p, u32x4_t v) { *reinterpret_cast<u32x4_t*>(p) = v; }

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
    return __uint_as_float(((uint32_t)b) << 16);
}

// Pack two floats into two bfloat16 (round to nearest even), low half = a.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    bf16x2_t v;
    v.x = (__bf16)a;
    v.y = (__bf16)b;
    return __builtin_bit_cast(uint32_t, v);
}

// Round a double to bfloat16, ties to even, in one rounding.  The double is
// first narrowed to float with round-to-odd (truncate, then set the last bit
// when inexact); float keeps more than bfloat16's 8 significant bits plus two,
// so the second, ties-to-even narrowing then rounds exactly as a direct one.
// Written with selects only (no divergent branches).
__device__ __forceinline__ uint16_t f64_to_bf16_bits(double x) {
    const float f = (float)x;                 // ties to even
    const double back = (double)f;
    const uint32_t uf = __float_as_uint(f);
    const bool inexact = back != x;           // also true for NaN
    const bool above = __builtin_fabs(back) > __builtin_fabs(x);
    uint32_t u = (inexact && above) ? uf - 1u : uf;   // step toward zero
    u = inexact ? (u | 1u) : u;                        // sticky bit
    const uint32_t rounded = (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
    const uint32_t qnan = (uf >> 16) | 0x40u;
    const uint64_t ux = __builtin_bit_cast(uint64_t, x);
    const bool nan = (ux & 0x7fffffffffffffffull) > 0x7ff0000000000000ull;
    return (uint16_t)(nan ? qnan : rounded);
}

// Out of line so the compiler keeps it off the common path below.
__device__ __attribute__((noinline)) uint16_t f64_to_bf16_bits_rare(double x) { return f64_to_bf16_bits(x); }

// The same rounding done on the double's bit pattern, for results in
// bfloat16's normal range (|x| in [2^-126, 2^128), after rounding up to
// infinity): round to nearest even on the 45 dropped mantissa bits, then
// rebias the exponent.  Anything else (tiny, infinite, NaN) takes the
// float path above.  Integer instructions only, on the common path.
__device__ __forceinline__ uint16_t f64_to_bf16_bits_fast(double x) {
    const uint64_t u = __builtin_bit_cast(uint64_t, x);
    const uint32_t lo = (uint32_t)u, hi = (uint32_t)(u >> 32);
    const uint32_t e = (hi >> 20) & 0x7ffu;
    // dropped bits: hi[12:0] and lo; half = hi bit 12, kept lsb = hi bit 13
    const bool half = (hi & 0x1000u) != 0;
    const bool rest = ((hi & 0xfffu) | lo) != 0;
    const bool lsb = (hi & 0x2000u) != 0;
    const uint32_t rhi = (hi & ~0x1fffu) + ((half && (rest || lsb)) ? 0x2000u : 0u);
    const uint32_t sign = (hi >> 16) & 0x8000u;
    const uint32_t em = (rhi >> 13) & 0x3ffffu;          // exponent (11) : mantissa (7)
    uint32_t b = em > (1150u << 7 | 0x7fu) ? 0x7f80u : em - (896u << 7);
    if (__builtin_expect(e < 897u || e == 0x7ffu, 0)) return f64_to_bf16_bits_rare(x);
    return (uint16_t)(sign | b);
}

template <typename T> struct Elem;
template <> struct Elem<float> {
    __device__ static double load(const float* p) { return (double)*p; }
    __device__ static void store(float* p, double x) { *p = (float)x; }
};
template <> struct Elem<uint16_t> {
    __device__ static double load(const uint16_t* p) { return (double)bf16_to_f32(*p); }
    __device__ static void store(uint16_t* p, double x) { *p = f64_to_bf16_bits(x); }
};

// Each shuffle is evaluated exactly once, by every lane: a cross-lane read
// (ds_bpermute) placed under a divergent branch would read from lanes that are
// switched off.
template <typename T>
__device__ __forceinline__ T wave_max(T v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const T other = __shfl_xor(v, o);
        v = v > other ? v : other;
    }
    return v;
}

template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

}  // namespace attn
