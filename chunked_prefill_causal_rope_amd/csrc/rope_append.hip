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
// One workgroup per (token, group of 4 heads), one wave per head: the token's
// cos/sin table (rd/2 entries, double) is built in LDS by the workgroup and
// shared by its heads.  The arithmetic is double precision, so the stored
// value is the correctly rounded image of the exact finish (up to the last
// bits of the double sine and cosine).
#include "device_common.h"
#include "launch.h"

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
    if (KV && pos >= a.cap) return;

    const int hd = a.head_dim;
    const int rd = a.rotary_dim;
    const int half = rd / 2;
    const int tid = threadIdx.x;
    for (int k = tid; k < half; k += kRopeThreads) {
        // position * f_k is exact in double (integer times a float)
        double th = (double)pos * (double)a.inv_freq[k];
        double sn, c;
        sincos(th, &sn, &c);
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
        yd = dst + (((size_t)b * a.n_heads + h) * a.cap + pos) * hd;
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
        T* vd = reinterpret_cast<T*>(a.v_dst) + (((size_t)b * a.n_heads + h) * a.cap + pos) * hd;
        for (int e = lane; e < hd; e += 64) vd[e] = vs[e];
    }
}

hipError_t launch_rope_rows(const RopeArgs& a, int dtype, bool kv, hipStream_t stream) {
    dim3 grid(a.max_chunk, (a.n_heads + kRopeWaves - 1) / kRopeWaves, a.n_seq);
    dim3 block(kRopeThreads);
    if (dtype == 0) {
        if (kv) rope_rows_kernel<float, true><<<grid, block, 0, stream>>>(a);
        else rope_rows_kernel<float, false><<<grid, block, 0, stream>>>(a);
    } else {
        if (kv) rope_rows_kernel<uint16_t, true><<<grid, block, 0, stream>>>(a);
        else rope_rows_kernel<uint16_t, false><<<grid, block, 0, stream>>>(a);
    }
    return hipGetLastError();
}

}  // namespace attn
