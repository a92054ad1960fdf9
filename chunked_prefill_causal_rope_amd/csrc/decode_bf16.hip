// bf16 decode attention: one query per sequence (chunk = 1) over a long
// head-major cache.  Memory-bound: every K/V byte of the context is read once
// per KV group, shared by the group's G query heads.
//
// cortiq-engine 0.5.39 src/attention.rs: fn attention_head (scores, max-
// subtracted softmax, output and probabilities; "cost grows linearly with the
// stored context"), fn attend_all_heads (a KV group's K/V is streamed once for
// all of its query heads).
//
// Design (gfx950):
//  * The context of each (sequence, KV group) is split into parts of
//    split_len keys, one single-wave workgroup per part, so a batch of long
//    sequences gives thousands of independent streams to cover HBM latency.
//  * Scores for 64 keys come from four v_mfma_f32_16x16x32_bf16: A = the
//    group's queries (rows = heads, padded to 16), B = K rows straight from
//    global memory (each lane loads 16 contiguous bytes of one key row).
//  * P.V runs on the vector ALU in float32: each lane owns 8 dims of V for
//    every (512/head_dim)-th key, so one wave instruction loads 1 KB of
//    consecutive rows; the
//    probabilities and the per-head rescale factors go through LDS.
//  * Each part leaves (m, l, O) in the workspace and, when asked, its raw
//    log2-domain scores in the probabilities buffer; the combine kernel merges
//    the parts with log-sum-exp and turns the scores into probabilities.
#include "device_common.h"
#include "launch.h"

namespace attn {

constexpr int kDecKB = 64;      // keys per iteration
constexpr int kPartPadD = 4;    // (m, l, pad, pad) before O in a partial
constexpr int kDecMaxGroup = 16;

int decode_group_limit() { return kDecMaxGroup; }

__device__ __forceinline__ f32x4_t mfma16(bf16x8_t a, bf16x8_t b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

template <int HD, int GQ>
__global__ __launch_bounds__(64) void decode_split_kernel(DecodeArgs a) {
    constexpr int NK = HD / 32;                 // K-steps per 16x16x32 product
    constexpr int LPR = HD / 8;                 // lanes per V row (8 dims each)
    constexpr int KPI = 64 / LPR;               // V rows per wave instruction
    constexpr int VROWS = kDecKB / KPI;         // V rows per lane per iteration
    __shared__ float pbuf[kDecKB * 16];
    __shared__ float abuf[16];

    const int lane = threadIdx.x;
    int id = blockIdx.x;
    const int g = id % a.n_kv;
    id /= a.n_kv;
    const int s = id % a.n_splits;
    const int b = id / a.n_splits;
    if (b >= a.n_seq) return;
    const int ctx = min(min(a.ctx[b], a.max_ctx), a.cap);
    const int k_lo = s * a.split_len;
    const int k_hi = min(k_lo + a.split_len, ctx);
    if (k_lo >= k_hi) return;
    const int G = a.group;

    const int qh = lane & 15;    // score layout: key column / query-row index
    const int quad = lane >> 4;  // score layout: heads 4*quad .. 4*quad+3
    const int c = lane % LPR;    // P.V layout: dims 8c .. 8c+7
    const int kr = lane / LPR;   // P.V layout: keys kr, kr+KPI, ...

    bf16x8_t qa[NK];
    {
        const uint16_t* qb =
            reinterpret_cast<const uint16_t*>(a.q) + ((size_t)b * a.n_heads + g * G) * HD;
#pragma unroll
        for (int k = 0; k < NK; ++k) {
            uint4 u = make_uint4(0, 0, 0, 0);
            if (qh < G) u = *reinterpret_cast<const uint4*>(qb + (size_t)qh * HD + 32 * k + 8 * quad);
            qa[k] = __builtin_bit_cast(bf16x8_t, u);
        }
    }
    const size_t base = ((size_t)b * a.n_kv + g) * (size_t)a.cap * HD;
    const uint16_t* kc = reinterpret_cast<const uint16_t*>(a.k_cache) + base;
    const uint16_t* vc = reinterpret_cast<const uint16_t*>(a.v_cache) + base;
    float* prow = a.probs ? a.probs + ((size_t)b * a.n_heads + g * G) * a.probs_ld : nullptr;

    float m_run[4], l_run[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        m_run[r] = -INFINITY;
        l_run[r] = 0.f;
    }
    float o[GQ][8];
#pragma unroll
    for (int hh = 0; hh < GQ; ++hh)
#pragma unroll
        for (int e = 0; e < 8; ++e) o[hh][e] = 0.f;
    const float sl = a.scale * kLog2e;

    for (int k0 = k_lo; k0 < k_hi; k0 += kDecKB) {
        uint4 kf[4][NK];
#pragma unroll
        for (int blk = 0; blk < 4; ++blk) {
            const int key = k0 + 16 * blk + qh;
#pragma unroll
            for (int k = 0; k < NK; ++k)
                kf[blk][k] = key < k_hi
                                 ? *reinterpret_cast<const uint4*>(kc + (size_t)key * HD + 32 * k + 8 * quad)
                                 : make_uint4(0, 0, 0, 0);
        }
        uint4 vf[VROWS];
#pragma unroll
        for (int ii = 0; ii < VROWS; ++ii) {
            const int key = k0 + kr + KPI * ii;
            vf[ii] = key < k_hi ? *reinterpret_cast<const uint4*>(vc + (size_t)key * HD + 8 * c)
                                : make_uint4(0, 0, 0, 0);
        }
        // scores: S[blk][r] = head 4*quad + r, key k0 + 16*blk + qh
        float x[4][4];
#pragma unroll
        for (int blk = 0; blk < 4; ++blk) {
            f32x4_t S = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int k = 0; k < NK; ++k) S = mfma16(qa[k], __builtin_bit_cast(bf16x8_t, kf[blk][k]), S);
            const bool ok = k0 + 16 * blk + qh < k_hi;
#pragma unroll
            for (int r = 0; r < 4; ++r) x[blk][r] = ok ? S[r] * sl : -INFINITY;
        }
        if (prow) {
#pragma unroll
            for (int blk = 0; blk < 4; ++blk) {
                const int key = k0 + 16 * blk + qh;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int hh = 4 * quad + r;
                    if (hh < G && key < k_hi) prow[(size_t)hh * a.probs_ld + key] = x[blk][r];
                }
            }
        }
        float alpha[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            float mt = fmaxf(fmaxf(x[0][r], x[1][r]), fmaxf(x[2][r], x[3][r]));
#pragma unroll
            for (int off = 1; off < 16; off <<= 1) mt = fmaxf(mt, __shfl_xor(mt, off));
            const float m_new = fmaxf(m_run[r], mt);   // finite: key k0 is in range
            alpha[r] = __builtin_amdgcn_exp2f(m_run[r] - m_new);
            float ps = 0.f;
#pragma unroll
            for (int blk = 0; blk < 4; ++blk) {
                x[blk][r] = __builtin_amdgcn_exp2f(x[blk][r] - m_new);
                ps += x[blk][r];
            }
            l_run[r] = l_run[r] * alpha[r] + ps;
            m_run[r] = m_new;
        }
#pragma unroll
        for (int blk = 0; blk < 4; ++blk)
            *reinterpret_cast<float4*>(&pbuf[(16 * blk + qh) * 16 + 4 * quad]) =
                make_float4(x[blk][0], x[blk][1], x[blk][2], x[blk][3]);
        if (qh == 0)
            *reinterpret_cast<float4*>(&abuf[4 * quad]) =
                make_float4(alpha[0], alpha[1], alpha[2], alpha[3]);
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

#pragma unroll
        for (int hq = 0; hq < GQ / 4; ++hq) {
            const float4 al = *reinterpret_cast<const float4*>(&abuf[4 * hq]);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                o[4 * hq + 0][e] *= al.x;
                o[4 * hq + 1][e] *= al.y;
                o[4 * hq + 2][e] *= al.z;
                o[4 * hq + 3][e] *= al.w;
            }
        }
#pragma unroll
        for (int ii = 0; ii < VROWS; ++ii) {
            const int kl = kr + KPI * ii;
            float v[8];
            v[0] = bf16_lo(vf[ii].x);
            v[1] = bf16_hi(vf[ii].x);
            v[2] = bf16_lo(vf[ii].y);
            v[3] = bf16_hi(vf[ii].y);
            v[4] = bf16_lo(vf[ii].z);
            v[5] = bf16_hi(vf[ii].z);
            v[6] = bf16_lo(vf[ii].w);
            v[7] = bf16_hi(vf[ii].w);
#pragma unroll
            for (int hq = 0; hq < GQ / 4; ++hq) {
                const float4 p = *reinterpret_cast<const float4*>(&pbuf[kl * 16 + 4 * hq]);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    o[4 * hq + 0][e] += p.x * v[e];
                    o[4 * hq + 1][e] += p.y * v[e];
                    o[4 * hq + 2][e] += p.z * v[e];
                    o[4 * hq + 3][e] += p.w * v[e];
                }
            }
        }
        // pbuf/abuf are rewritten by the next iteration
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }

    // l: sum the 16 key-lanes of each head quad; O: sum the key residues
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int off = 1; off < 16; off <<= 1) l_run[r] += __shfl_xor(l_run[r], off);
#pragma unroll
    for (int hh = 0; hh < GQ; ++hh)
#pragma unroll
        for (int e = 0; e < 8; ++e)
#pragma unroll
            for (int off = LPR; off < 64; off <<= 1) o[hh][e] += __shfl_xor(o[hh][e], off);

    constexpr int PS = HD + kPartPadD;
    float* part = a.part + (((size_t)b * a.n_heads + g * G) * a.n_splits + s) * PS;
    const size_t head_stride = (size_t)a.n_splits * PS;
    if (qh == 0) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int hh = 4 * quad + r;
            if (hh < G) *reinterpret_cast<float2*>(part + hh * head_stride) = make_float2(m_run[r], l_run[r]);
        }
    }
    if (kr == 0) {
#pragma unroll
        for (int hh = 0; hh < GQ; ++hh) {
            if (hh < G) {
                float* dst = part + hh * head_stride + kPartPadD + 8 * c;
                *reinterpret_cast<float4*>(dst) = make_float4(o[hh][0], o[hh][1], o[hh][2], o[hh][3]);
                *reinterpret_cast<float4*>(dst + 4) = make_float4(o[hh][4], o[hh][5], o[hh][6], o[hh][7]);
            }
        }
    }
}

// One workgroup per (sequence, head): merge the parts that cover
// [0, ctx) and, when asked, rewrite the raw scores as probabilities
// P_j = 2^(x_j - m) / l.
template <int HD>
__global__ __launch_bounds__(256) void decode_combine_kernel(DecodeArgs a) {
    const int row = blockIdx.x;
    const int b = row / a.n_heads;
    const int tid = threadIdx.x;
    if (b >= a.n_seq) return;
    const int ctx = min(min(a.ctx[b], a.max_ctx), a.cap);
    float* orow = a.out + (size_t)row * HD;
    if (ctx < 1) {
        for (int d = tid; d < HD; d += 256) orow[d] = 0.f;
        return;
    }
    constexpr int PS = HD + kPartPadD;
    const int n_parts = min((ctx + a.split_len - 1) / a.split_len, a.n_splits);
    const float* pr = a.part + (size_t)row * a.n_splits * PS;
    float m = -INFINITY;
    for (int s = 0; s < n_parts; ++s) m = fmaxf(m, pr[(size_t)s * PS]);
    float l = 0.f;
    for (int s = 0; s < n_parts; ++s) l += pr[(size_t)s * PS + 1] * __builtin_amdgcn_exp2f(pr[(size_t)s * PS] - m);
    const float inv = 1.f / l;
    for (int d = tid; d < HD; d += 256) {
        float acc = 0.f;
        for (int s = 0; s < n_parts; ++s)
            acc += pr[(size_t)s * PS + kPartPadD + d] * __builtin_amdgcn_exp2f(pr[(size_t)s * PS] - m);
        orow[d] = acc * inv;
    }
    if (a.probs) {
        // P_j = 2^(x_j - m) / l over the row's ctx entries; 16-byte accesses
        // between a scalar head (up to the first aligned element) and tail
        float* prow = a.probs + (size_t)row * a.probs_ld;
        const int head = min((int)((4 - (((uintptr_t)prow >> 2) & 3)) & 3), ctx);
        for (int j = tid; j < head; j += 256) prow[j] = __builtin_amdgcn_exp2f(prow[j] - m) * inv;
        float4* p4 = reinterpret_cast<float4*>(prow + head);
        const int n4 = (ctx - head) >> 2;
        for (int j = tid; j < n4; j += 256) {
            float4 v = p4[j];
            v.x = __builtin_amdgcn_exp2f(v.x - m) * inv;
            v.y = __builtin_amdgcn_exp2f(v.y - m) * inv;
            v.z = __builtin_amdgcn_exp2f(v.z - m) * inv;
            v.w = __builtin_amdgcn_exp2f(v.w - m) * inv;
            p4[j] = v;
        }
        for (int j = head + 4 * n4 + tid; j < ctx; j += 256)
            prow[j] = __builtin_amdgcn_exp2f(prow[j] - m) * inv;
    }
}

template <int HD>
static void launch_decode_hd(const DecodeArgs& a, hipStream_t stream) {
    const long blocks = (long)a.n_seq * a.n_splits * a.n_kv;
    if (a.group <= 4)
        decode_split_kernel<HD, 4><<<dim3((unsigned)blocks), dim3(64), 0, stream>>>(a);
    else if (a.group <= 8)
        decode_split_kernel<HD, 8><<<dim3((unsigned)blocks), dim3(64), 0, stream>>>(a);
    else
        decode_split_kernel<HD, 16><<<dim3((unsigned)blocks), dim3(64), 0, stream>>>(a);
    decode_combine_kernel<HD><<<dim3((unsigned)(a.n_seq * a.n_heads)), dim3(256), 0, stream>>>(a);
}

hipError_t launch_decode_bf16(const DecodeArgs& a, hipStream_t stream) {
    if ((long)a.n_seq * a.n_splits * a.n_kv <= 0) return hipSuccess;
    if (a.head_dim == 128)
        launch_decode_hd<128>(a, stream);
    else
        launch_decode_hd<64>(a, stream);
    return hipGetLastError();
}

}  // namespace attn
