// Measured roofline denominators for this part: a loop of bf16 matrix-core
// products and a streaming read of device memory.  The attention kernels'
// throughput is reported against the published peaks and against these
// measured ones, taken on the same GPU in the same run.
//
// Neither kernel computes anything of the method; they exist so the
// fraction of peak can be stated against what the part actually sustains
// (clock under load, memory efficiency) as well as against its datasheet.
#include <hip/hip_runtime.h>

#include "../../include/attn.h"
#include "device_common.h"

namespace attn {

// Each wave keeps four independent 32x32x16 bf16 accumulators in flight, so
// the matrix pipe never waits on a result.  The operands stay in registers,
// so the loop issues products only.  With random == 0 they are small
// constants with few distinct bits; with random == 1 each accumulator gets
// its own hashed bfloat16 operands (random signs and mantissas, magnitudes
// 2^-2..2^2), so consecutive products see different, fully toggling data, as
// the attention kernels' products do.  The part's clock under load depends on
// that switching activity, so the two modes bound the sustained matrix rate
// from above (constants) and for data like the kernels' (random).  A
// lane-dependent sum of the accumulators is written per wave, which keeps the
// products live.
__device__ __forceinline__ __bf16 hashed_bf16(uint32_t x) {
    x ^= x >> 16;
    x *= 0x7feb352du;
    x ^= x >> 15;
    x *= 0x846ca68bu;
    x ^= x >> 16;
    const uint32_t e = 125u + (x & 3u);   // exponent field: 2^-2 .. 2^1
    return __builtin_bit_cast(__bf16, (uint16_t)(((x >> 31) << 15) | (e << 7) | ((x >> 8) & 0x7fu)));
}

__global__ __launch_bounds__(256) void calib_mfma_kernel(int iters, int random, float* out) {
    const int lane = threadIdx.x & 63;
    const uint32_t seed = (blockIdx.x * 256u + threadIdx.x) * 64u;
    bf16x8_t a[4], b[4];
#pragma unroll
    for (int k = 0; k < 4; ++k)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            a[k][i] = random ? hashed_bf16(seed + 16u * k + i) : (__bf16)(0.001f * (float)((lane + i) & 7));
            b[k][i] = random ? hashed_bf16(seed + 16u * k + 8u + i) : (__bf16)(0.002f * (float)((lane * 3 + i) & 7));
        }
    f32x16_t c0 = {}, c1 = {}, c2 = {}, c3 = {};
    for (int it = 0; it < iters; ++it) {
        c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[0], b[0], c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[1], b[1], c1, 0, 0, 0);
        c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[2], b[2], c2, 0, 0, 0);
        c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[3], b[3], c3, 0, 0, 0);
    }
    float s = 0.f;
#pragma unroll
    for (int q = 0; q < 16; ++q) s += c0[q] + c1[q] + c2[q] + c3[q];
    s = wave_sum(s);
    if (lane == 0) out[blockIdx.x * (blockDim.x / 64) + (threadIdx.x >> 6)] = s;
}

// Streaming read of n16 16-byte words: workgroup w reads its own contiguous
// share (per_wg words), eight nontemporal loads in flight per lane; the
// words are folded with xor and one value per wave is written.
__global__ __launch_bounds__(256) void calib_read_kernel(const u32x4_t* src, size_t n16, size_t per_wg, uint32_t* out) {
    const size_t b0 = (size_t)blockIdx.x * per_wg;
    const size_t b1 = b0 + per_wg < n16 ? b0 + per_wg : n16;
    u32x4_t acc = {0u, 0u, 0u, 0u};
    constexpr int U = 8;
    for (size_t i = b0 + threadIdx.x; i < b1; i += 256 * U) {
        u32x4_t v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const size_t j = i + (size_t)u * 256;
            v[u] = j < b1 ? __builtin_nontemporal_load(src + j) : u32x4_t{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < U; ++u) acc ^= v[u];
    }
    uint32_t x = acc.x ^ acc.y ^ acc.z ^ acc.w;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) x ^= __shfl_xor(x, o);
    if ((threadIdx.x & 63) == 0) out[blockIdx.x * (blockDim.x / 64) + (threadIdx.x >> 6)] = x;
}

}  // namespace attn

extern "C" {

int attn_calibrate_mfma(int n_workgroups, int iters, int random_operands, float* out, void* stream) {
    if (n_workgroups <= 0 || iters <= 0 || !out || (random_operands != 0 && random_operands != 1)) return ATTN_EINVAL;
    attn::calib_mfma_kernel<<<dim3((unsigned)n_workgroups), dim3(256), 0, (hipStream_t)stream>>>(iters, random_operands,
                                                                                                   out);
    return hipGetLastError() == hipSuccess ? ATTN_OK : ATTN_EDEVICE;
}

int attn_calibrate_read(const void* src, size_t bytes, int n_workgroups, uint32_t* out, void* stream) {
    if (!src || !out || n_workgroups <= 0 || bytes < 16 || (bytes & 15) ||
        (reinterpret_cast<uintptr_t>(src) & 15))
        return ATTN_EINVAL;
    const size_t n16 = bytes / 16;
    attn::calib_read_kernel<<<dim3((unsigned)n_workgroups), dim3(256), 0, (hipStream_t)stream>>>(
        static_cast<const attn::u32x4_t*>(src), n16, (n16 + n_workgroups - 1) / n_workgroups, out);
    return hipGetLastError() == hipSuccess ? ATTN_OK : ATTN_EDEVICE;
}

}  // extern "C"
