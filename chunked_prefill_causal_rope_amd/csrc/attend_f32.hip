// float32 causal attention, one wave per (query row, head), vector ALU.
// Serves both prefill rows (varlen descriptor) and decode rows (one row per
// sequence at position ctx-1, with optional probabilities).
//
// cortiq-engine 0.5.39 src/attention.rs, fn attention_head: scores
// q.K_j * scale over the stored keys, max-subtracted softmax, probabilities
// returned; the batched causal attend of fn qwen_attention_batch limits row bi
// to keys < s0+bi+1; with a sliding window (QwenAttnCfg.window) a row reads
// only its last `window` keys.  Keys are taken 64 at a time (one per lane)
// with an online maximum; each lane owns head_dim/64 output dims for the P.V
// sum.
#include "device_common.h"
#include "launch.h"

namespace attn {

template <int HD>
__global__ __launch_bounds__(256) void attend_f32_kernel(AttendF32Args a) {
    constexpr int PER = HD / 64;
    __shared__ float qs[4][HD];
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int item = blockIdx.x * 4 + wave;

    int b, t, pos, h;
    if (a.decode) {
        b = item / a.n_heads;
        h = item % a.n_heads;
        if (b >= a.n_seq) return;
        const int ctx = a.ring ? min(a.ctx[b], a.max_ctx) : min(min(a.ctx[b], a.max_ctx), a.cap);
        if (ctx < 1) {
            float* orow = a.out + ((size_t)b * a.n_heads + h) * HD;
            for (int e = lane; e < HD; e += 64) orow[e] = 0.f;
            return;
        }
        t = b;
        pos = ctx - 1;
    } else {
        b = blockIdx.y;
        const int i = item / a.n_heads;
        h = item % a.n_heads;
        const int t0 = a.cu_seq[b];
        const int len = min(a.cu_seq[b + 1] - t0, a.max_chunk);
        if (i >= len) return;
        t = t0 + i;
        pos = a.start[b] + i;
        if (t < 0 || t >= a.n_tok || pos < 0 || (!a.ring && pos >= a.cap)) return;
    }
    const int g = h / a.group;
    const float* q = a.q + ((size_t)t * a.n_heads + h) * HD;
    for (int e = lane; e < HD; e += 64) qs[wave][e] = q[e];
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    const size_t base = ((size_t)b * a.n_kv + g) * (size_t)a.cap * HD;
    const float* kc = a.k_cache + base;
    const float* vc = a.v_cache + base;
    const int n = pos + 1;
    // first key of the row's window (0 without one)
    const int first = a.window > 0 && n > a.window ? n - a.window : 0;
    const float sl = a.scale * kLog2e;
    // cache row of key j
    auto slot = [&](int j) { return a.ring ? j % a.cap : j; };

    auto score = [&](int j) -> float {
        const float4* kr = reinterpret_cast<const float4*>(kc + (size_t)slot(j) * HD);
        const float4* qr = reinterpret_cast<const float4*>(qs[wave]);
        float acc = 0.f;
#pragma unroll 8
        for (int d = 0; d < HD / 4; ++d) {
            const float4 kk = kr[d];
            const float4 qq = qr[d];
            acc += qq.x * kk.x + qq.y * kk.y + qq.z * kk.z + qq.w * kk.w;
        }
        return acc * sl;
    };

    float m = -INFINITY, l = 0.f;
    float o[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e) o[e] = 0.f;
    for (int j0 = first; j0 < n; j0 += 64) {
        const int j = j0 + lane;
        const float x = j < n ? score(j) : -INFINITY;
        const float m_new = fmaxf(m, wave_max(x));
        const float alpha = exp2f(m - m_new);
        const float p = exp2f(x - m_new);
        l = l * alpha + wave_sum(p);
#pragma unroll
        for (int e = 0; e < PER; ++e) o[e] *= alpha;
        const int cnt = min(64, n - j0);
        for (int jj = 0; jj < cnt; ++jj) {
            const float pj = __shfl(p, jj);
            const float* vr = vc + (size_t)slot(j0 + jj) * HD;
#pragma unroll
            for (int e = 0; e < PER; ++e) o[e] += pj * vr[lane + 64 * e];
        }
        m = m_new;
    }
    const float inv = 1.f / l;
    float* orow = a.out + ((size_t)t * a.n_heads + h) * HD;
#pragma unroll
    for (int e = 0; e < PER; ++e) {
        float y = o[e] * inv;
        if (a.gate.mode) y *= gate_factor(a.gate, (size_t)t * a.n_heads + h, lane + 64 * e);
        orow[lane + 64 * e] = y;
    }

    if (a.decode && a.probs) {
        float* prow = a.probs + ((size_t)b * a.n_heads + h) * a.probs_ld;
        for (int j = lane; j < n; j += 64) prow[j] = j < first ? 0.f : exp2f(score(j) - m) * inv;
    }
}

hipError_t launch_attend_f32(const AttendF32Args& a, hipStream_t stream) {
    dim3 grid;
    if (a.decode) {
        const long items = (long)a.n_seq * a.n_heads;
        grid = dim3((unsigned)((items + 3) / 4), 1);
    } else {
        const long items = (long)a.max_chunk * a.n_heads;
        grid = dim3((unsigned)((items + 3) / 4), (unsigned)a.n_seq);
    }
    if (grid.x == 0 || grid.y == 0) return hipSuccess;
    if (a.head_dim == 128)
        attend_f32_kernel<128><<<grid, dim3(256), 0, stream>>>(a);
    else
        attend_f32_kernel<64><<<grid, dim3(256), 0, stream>>>(a);
    return hipGetLastError();
}

}  // namespace attn
