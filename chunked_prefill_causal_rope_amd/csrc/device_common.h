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
// Fourth word of a raw buffer resource on gfx9-family parts (32-bit data
// format; byte offsets, no swizzle, no index).
constexpr int kBufferWord3 = 0x00020000;
// A raw buffer resource over n_bytes from p.  The values must be the same in
// every lane; the readfirstlanes let the compiler keep the resource in scalar
// registers (a resource it cannot prove uniform makes it wrap every load in a
// loop over the lanes' distinct values).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t uniform_rsrc(const void* p, int n_bytes) {
    const uint64_t u = reinterpret_cast<uint64_t>(p);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
    return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(((uint64_t)hi << 32) | lo), (short)0,
                                             __builtin_amdgcn_readfirstlane(n_bytes), kBufferWord3);
}
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

// IEEE half precision (binary16), round to nearest even.
__device__ __forceinline__ uint16_t f16_bits(float x) { return __builtin_bit_cast(uint16_t, (_Float16)x); }
__device__ __forceinline__ float f16_value(uint16_t u) { return (float)__builtin_bit_cast(_Float16, u); }
__device__ __forceinline__ uint32_t pack_f16x2(float a, float b) {
    return (uint32_t)f16_bits(a) | ((uint32_t)f16_bits(b) << 16);
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

// n doubles (n even) to n/2 words of two bfloat16 (low half = even index),
// each value rounded once, ties to even.  Common path: the hardware's
// double->float and float->bfloat16 conversions, both ties to even.
// Rounding twice can only differ from rounding once when the first result
// lies exactly halfway between two bfloat16 neighbours (low 16 bits 0x8000);
// if any value of the group does, in any active lane, the group is redone
// with the exact conversion above (the test is a wave ballot, so the branch
// is uniform and the common path carries no per-lane flags).
template <int N>
__device__ __forceinline__ void f64_to_bf16_packed(const double* v, uint32_t* u) {
    float f[N];
    uint64_t mid = 0;
#pragma unroll
    for (int j = 0; j < N; ++j) {
        f[j] = (float)v[j];
        mid |= __builtin_amdgcn_ballot_w64((__float_as_uint(f[j]) & 0xffffu) == 0x8000u);
    }
#pragma unroll
    for (int j = 0; j < N / 2; ++j) u[j] = pack_bf16x2(f[2 * j], f[2 * j + 1]);
    if (__builtin_expect(mid != 0, 0)) {
#pragma unroll
        for (int j = 0; j < N / 2; ++j)
            u[j] = (uint32_t)f64_to_bf16_bits(v[2 * j]) | ((uint32_t)f64_to_bf16_bits(v[2 * j + 1]) << 16);
    }
}

// Split partials keep a row's output normalised by its own row sum, O/l (a
// convex combination of V rows), as half precision, scaled by 2^-e when the
// row's largest magnitude would not fit (e >= 0, kept beside m and l): half
// the bytes of float partials, relative rounding 2^-11 of the row's largest.
__device__ __forceinline__ int part_scale_exp(float maxabs) {
    // maxabs < 2^k; keep scaled values below 2^15 (half's largest is ~2^16)
    const int k = __builtin_amdgcn_frexp_expf(maxabs);
    return k > 15 ? k - 15 : 0;
}

// Output gate of the attention output ([ATT] fn apply_gate: times
// sigmoid(g) per element; fn apply_projected_gate: times softplus(g), one g
// per head or per element).  The gate value of output row `row` (token *
// n_heads + head), dim d, is at p[row * ld + d] (p[row * ld] per head), in
// the call's dtype.
enum { kGateNone = 0, kGateSigmoid = 1, kGateSoftplusHead = 2, kGateSoftplus = 3 };
struct GateRef {
    const void* p;
    int mode, ld, bf16;
};
__device__ __forceinline__ float gate_factor(const GateRef& g, size_t row, int d) {
    const size_t i = row * (size_t)g.ld + (g.mode == kGateSoftplusHead ? 0 : d);
    const float x = g.bf16 ? bf16_to_f32(reinterpret_cast<const uint16_t*>(g.p)[i])
                           : reinterpret_cast<const float*>(g.p)[i];
    if (g.mode == kGateSigmoid) return 1.f / (1.f + expf(-x));
    return fmaxf(x, 0.f) + log1pf(expf(-fabsf(x)));
}
// The same factors from the hardware exp2/log2/reciprocal (relative error a
// few float ulps; softplus of very negative x loses relative accuracy but
// not absolute), for the bf16 kernels' epilogues.
constexpr float kLn2 = 0.6931471805599453f;
__device__ __forceinline__ float gate_fast(int mode, float x) {
    if (mode == kGateSigmoid) return __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-x * kLog2e));
    const float e = __builtin_amdgcn_exp2f(-__builtin_fabsf(x) * kLog2e);
    return fmaxf(x, 0.f) + __builtin_amdgcn_logf(1.f + e) * kLn2;
}
// bf16 gate value of (row, d) and its factor, fast form
__device__ __forceinline__ float gate_factor_bf16(const GateRef& g, size_t row, int d) {
    const size_t i = row * (size_t)g.ld + (g.mode == kGateSoftplusHead ? 0 : d);
    return gate_fast(g.mode, bf16_to_f32(reinterpret_cast<const uint16_t*>(g.p)[i]));
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
