// Per-head finish of projected rows: optional RMS qk-norm, then half-split
// RoPE, then one rounding to the stored dtype.  Used in place (or out of
// place) for queries, and for keys on their way into the head-major cache,
// where the matching value rows are copied alongside.
//
// Sources: cortiq-engine 0.5.39 src/attention.rs -- fn rmsnorm_head (norm in
// double, x*r*w or x*r*(1+w)), fn rope_rotate_scaled (pairs (i, i+rd/2), both
// outputs scaled), fn finish_projection (norm before RoPE, partial rotary on
// the first rd dims), fn qwen_attention_batch (every row of the chunk is
// appended before the chunk attends).
//
// General path: one workgroup per (token, group of 4 heads), one wave per
// head: the token's cos/sin table (rd/2 entries, double) is built in LDS by
// the workgroup and shared by its heads.  On both paths the arithmetic is
// double precision, so the stored value is the correctly rounded image of
// the exact finish (up to the last bits of the double sine and cosine).
#include "device_common.h"
#include "launch.h"
#include "rope_token.h"

namespace attn {

constexpr int kRopeThreads = 256;
constexpr int kRopeWaves = kRopeThreads / 64;
constexpr int kMaxHd = 128;

template <typename T, bool KV>
__global__ __launch_bounds__(kRopeThreads) void rope_rows_kernel(RopeArgs a) {
    __shared__ double cs_cos[kMaxHd / 2];
    __shared__ double cs_sin[kMaxHd / 2];
    __shared__ double rowbuf[kRopeWaves][kMaxHd];

    const int b = blockIdx.z;
    const int i = blockIdx.x;
    const int seq0 = a.cu_seq[b];
    const int len = a.cu_seq[b + 1] - seq0;
    if (i >= len) return;
    const int t = seq0 + i;
    const int pos = a.start[b] + i;
    if (t < 0 || t >= a.n_tok || pos < 0) return;
    if (KV && !a.ring && pos >= a.cap) return;
    const int slot = KV && a.ring ? pos % a.cap : pos;   // cache row of the position

    const int hd = a.head_dim;
    const int rd = a.rotary_dim;
    const int half = rd / 2;
    const int tid = threadIdx.x;
    for (int k = tid; k < half; k += kRopeThreads) {
        // position * f_k is exact in double (integer times a float)
        double th = (double)pos * (double)a.inv_freq[k];
        double sn, c;
        sincos_pos(th, &sn, &c);
        cs_cos[k] = c;
        cs_sin[k] = sn;
    }
    __syncthreads();

    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int h = blockIdx.y * kRopeWaves + wave;
    if (h >= a.n_heads) return;
    const T* src = reinterpret_cast<const T*>(a.x);
    T* dst = reinterpret_cast<T*>(a.y);
    double* row = rowbuf[wave];
    const double rs = (double)a.rope_scale;

    const T* xs = src + ((size_t)t * a.n_heads + h) * hd;
    // each lane holds dims lane and lane+64
    double x0 = lane < hd ? Elem<T>::load(xs + lane) : 0.0;
    double x1 = lane + 64 < hd ? Elem<T>::load(xs + lane + 64) : 0.0;
    if (a.norm != 0) {
        double ss = wave_sum(x0 * x0 + x1 * x1);
        double r = 1.0 / sqrt(ss / (double)hd + a.eps);
        if (lane < hd) {
            double w = (double)a.norm_w[lane];
            x0 = x0 * r * (a.norm == 2 ? 1.0 + w : w);
        }
        if (lane + 64 < hd) {
            double w = (double)a.norm_w[lane + 64];
            x1 = x1 * r * (a.norm == 2 ? 1.0 + w : w);
        }
    }
    if (lane < hd) row[lane] = x0;
    if (lane + 64 < hd) row[lane + 64] = x1;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    T* yd;
    if (KV) {
        yd = dst + (((size_t)b * a.n_heads + h) * a.cap + slot) * hd;
    } else {
        yd = dst + ((size_t)t * a.n_heads + h) * hd;
    }
#pragma unroll
    for (int rep = 0; rep < 2; ++rep) {
        const int e = lane + 64 * rep;
        if (e >= hd) continue;
        double v;
        if (e < half) {
            v = (row[e] * cs_cos[e] - row[e + half] * cs_sin[e]) * rs;
        } else if (e < rd) {
            const int k = e - half;
            v = (row[k] * cs_sin[k] + row[e] * cs_cos[k]) * rs;
        } else {
            v = row[e];
        }
        Elem<T>::store(yd + e, v);
    }
    if (KV) {
        const T* vs = reinterpret_cast<const T*>(a.v_src) + ((size_t)t * a.n_heads + h) * hd;
        T* vd = reinterpret_cast<T*>(a.v_dst) + (((size_t)b * a.n_heads + h) * a.cap + slot) * hd;
        if (a.v_norm) {
            // scale-less RMS norm of the V row, in double, rounded once
            const double v0 = lane < hd ? Elem<T>::load(vs + lane) : 0.0;
            const double v1 = lane + 64 < hd ? Elem<T>::load(vs + lane + 64) : 0.0;
            const double r = 1.0 / sqrt(wave_sum(v0 * v0 + v1 * v1) / (double)hd + a.eps);
            if (lane < hd) Elem<T>::store(vd + lane, v0 * r);
            if (lane + 64 < hd) Elem<T>::store(vd + lane + 64, v1 * r);
        } else {
            for (int e = lane; e < hd; e += 64) vd[e] = vs[e];
        }
    }
}

// Fast path (rotary_dim a multiple of 8): the per-token body in rope_token.h,
// one 256-thread workgroup per (kTokPerWg consecutive tokens, group of head
// rows).  Measured on a 2048-token, 48-head chunk with qk-norm: 1 token per
// workgroup is fastest (2, 4 and 8 tokens, each workgroup's loads all in
// flight first, were 1 %, 2.5 % and 5 % slower per step: fewer workgroups
// hide less of the per-token double-precision work).
#ifndef ATTN_ROPE_TOKENS
#define ATTN_ROPE_TOKENS 1
#endif
constexpr int kTokPerWg = ATTN_ROPE_TOKENS;

template <typename T, int HD>
__global__ __launch_bounds__(kTokThreads) void rope_token_kernel(RopeTokArgs a) {
    __shared__ RopeTokSmem<HD, kTokPerWg> sm;
    rope_token_body<T, HD, kTokThreads, kTokPerWg>(a, blockIdx.x * kTokPerWg, blockIdx.y, blockIdx.z, sm);
}

bool rope_token_path(const RopeArgs& a) {
    return a.rotary_dim % 8 == 0 && (a.head_dim == 64 || a.head_dim == 128);
}

template <typename T>
static void launch_token(const RopeTokArgs& t, int head_dim, int max_chunk, int n_seq, hipStream_t stream) {
    const int per_block = kTokThreads / (head_dim / 8);
    const dim3 grid((max_chunk + kTokPerWg - 1) / kTokPerWg, (t.nq + t.nk + per_block - 1) / per_block, n_seq);
    if (head_dim == 128) rope_token_kernel<T, 128><<<grid, dim3(kTokThreads), 0, stream>>>(t);
    else rope_token_kernel<T, 64><<<grid, dim3(kTokThreads), 0, stream>>>(t);
}

static RopeTokArgs token_args(const RopeArgs* q, const RopeArgs* kv) {
    const RopeArgs& r = q ? *q : *kv;
    RopeTokArgs t{};
    if (q) {
        t.qx = q->x;
        t.qy = q->y;
        t.qw = q->norm_w;
        t.nq = q->n_heads;
    }
    if (kv) {
        t.kx = kv->x;
        t.vx = kv->v_src;
        t.kc = kv->y;
        t.vc = kv->v_dst;
        t.kw = kv->norm_w;
        t.nk = kv->n_heads;
        t.cap = kv->cap;
        t.ring = kv->ring;
        t.v_norm = kv->v_norm;
    }
    t.cu_seq = r.cu_seq;
    t.start = r.start;
    t.inv_freq = r.inv_freq;
    t.eps = r.eps;
    t.rope_scale = r.rope_scale;
    t.n_tok = r.n_tok;
    t.rotary_dim = r.rotary_dim;
    t.norm = r.norm;
    return t;
}

template <typename T, bool KV>
static void launch_rope_typed(const RopeArgs& a, hipStream_t stream) {
    if (rope_token_path(a)) {
        launch_token<T>(token_args(KV ? nullptr : &a, KV ? &a : nullptr), a.head_dim, a.max_chunk, a.n_seq,
                        stream);
    } else {
        const dim3 grid(a.max_chunk, (a.n_heads + kRopeWaves - 1) / kRopeWaves, a.n_seq);
        rope_rows_kernel<T, KV><<<grid, dim3(kRopeThreads), 0, stream>>>(a);
    }
}

hipError_t launch_rope_rows(const RopeArgs& a, int dtype, bool kv, hipStream_t stream) {
    if (dtype == 0) {
        if (kv) launch_rope_typed<float, true>(a, stream);
        else launch_rope_typed<float, false>(a, stream);
    } else {
        if (kv) launch_rope_typed<uint16_t, true>(a, stream);
        else launch_rope_typed<uint16_t, false>(a, stream);
    }
    return hipGetLastError();
}

RopeTokArgs rope_token_args(const RopeArgs& q, const RopeArgs& kv) { return token_args(&q, &kv); }

// Queries and keys/values of one chunk: one launch on the token path (both
// share the position table), otherwise the two general launches.
hipError_t launch_rope_qkv(const RopeArgs& q, const RopeArgs& kv, int dtype, hipStream_t stream) {
    if (rope_token_path(q)) {
        const RopeTokArgs t = token_args(&q, &kv);
        if (dtype == 0) launch_token<float>(t, q.head_dim, q.max_chunk, q.n_seq, stream);
        else launch_token<uint16_t>(t, q.head_dim, q.max_chunk, q.n_seq, stream);
        return hipGetLastError();
    }
    hipError_t e = launch_rope_rows(q, dtype, false, stream);
    if (e == hipSuccess) e = launch_rope_rows(kv, dtype, true, stream);
    return e;
}

}  // namespace attn
