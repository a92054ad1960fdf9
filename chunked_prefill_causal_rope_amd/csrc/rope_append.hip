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

namespace attn {

constexpr int kRopeThreads = 256;
constexpr int kRopeWaves = kRopeThreads / 64;
constexpr int kMaxHd = 128;

// sin and cos of theta = position x inverse frequency (finite, |theta| below
// 2^40).  Cody-Waite reduction: k = theta * 2/pi rounded to an integer, and
// r = theta - k pi/2 with pi/2 split into three doubles, each step one fused
// multiply-add (absolute error of r near 2^-53).  On |r| <= pi/4 (plus
// rounding) the Taylor series of sin to degree 17 and of cos to degree 18
// truncate below 1e-19 relative; k mod 4 selects the quadrant's swap and
// signs.  Short, branch-free and light on registers.
constexpr double inv_factorial(int n) {
    double f = 1.0;
    for (int i = 2; i <= n; ++i) f *= (double)i;    // exact up to 18!
    return 1.0 / f;
}
__device__ __forceinline__ void sincos_pos(double th, double* sn, double* cs) {
    constexpr double kTwoOverPi = 0.6366197723675814;
    constexpr double kPio2a = 1.5707963267948966;         // pi/2 rounded to double
    constexpr double kPio2b = 6.123233995736766e-17;      // pi/2 - kPio2a, rounded
    constexpr double kPio2c = -1.4973849048591698e-33;    // pi/2 - kPio2a - kPio2b, rounded
    const double k = __builtin_rint(th * kTwoOverPi);
    double r = __builtin_fma(-k, kPio2a, th);
    r = __builtin_fma(-k, kPio2b, r);
    r = __builtin_fma(-k, kPio2c, r);
    const double z = r * r;
    // sin r = r + r z (-1/3! + z/5! - ... + z^7/17!)
    double ps = inv_factorial(17);
#pragma unroll
    for (int j = 7; j >= 1; --j) ps = __builtin_fma(ps, z, (j & 1 ? -1.0 : 1.0) * inv_factorial(2 * j + 1));
    const double s = __builtin_fma(r * z, ps, r);
    // cos r = 1 + z (-1/2! + z/4! - ... - z^8/18!)
    double pc = -inv_factorial(18);
#pragma unroll
    for (int j = 8; j >= 1; --j) pc = __builtin_fma(pc, z, (j & 1 ? -1.0 : 1.0) * inv_factorial(2 * j));
    const double c = __builtin_fma(z, pc, 1.0);
    const int n = (int)(k - 4.0 * __builtin_floor(k * 0.25));     // k mod 4, exact
    const double s1 = (n & 1) ? c : s;
    const double c1 = (n & 1) ? s : c;
    *sn = (n & 2) ? -s1 : s1;
    *cs = ((n + 1) & 2) ? -c1 : c1;
}

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

// Fast path, for rotary_dim a multiple of 8: one workgroup per (token, group
// of heads) with one pass and no loop.  A head row is handled by HD/8
// consecutive lanes, each owning 8 of its dims: a "pair" lane owns dims
// 4c..4c+3 and their RoPE partners 4c+rd/2.., a "pass" lane 8 dims past the
// rotary part.  Every lane issues its loads (and the matching V chunk for a
// key row) first; meanwhile the workgroup builds the token's cos/sin table
// (double) and the effective norm weights (w or 1 + w, double) in LDS.  The
// norm's sum of squares is a DPP reduction over the lanes of one row, and
// stores are 8 or 16 bytes wide.
template <typename T> struct Raw;
template <> struct Raw<uint16_t> {
    // 8 bf16 = 16 bytes
    u32x4_t w = {0u, 0u, 0u, 0u};
    __device__ void load4x2(const uint16_t* p0, const uint16_t* p1) {
        const u32x2_t a = *reinterpret_cast<const u32x2_t*>(p0);
        const u32x2_t b = *reinterpret_cast<const u32x2_t*>(p1);
        w = u32x4_t{a.x, a.y, b.x, b.y};
    }
    __device__ void load8(const uint16_t* p) { w = ld16(p); }
    // 8 values already in registers as 16-byte chunks (one for bf16)
    __device__ void from_chunks(const u32x4_t* c) { w = c[0]; }
    __device__ double get(int e) const {
        const uint32_t u = w[e >> 1];
        return (double)((e & 1) ? bf16_hi(u) : bf16_lo(u));
    }
};
template <> struct Raw<float> {
    f32x4_t lo = {0.f, 0.f, 0.f, 0.f}, hi = {0.f, 0.f, 0.f, 0.f};
    __device__ void load4x2(const float* p0, const float* p1) {
        lo = *reinterpret_cast<const f32x4_t*>(p0);
        hi = *reinterpret_cast<const f32x4_t*>(p1);
    }
    __device__ void load8(const float* p) {
        lo = *reinterpret_cast<const f32x4_t*>(p);
        hi = *reinterpret_cast<const f32x4_t*>(p + 4);
    }
    __device__ void from_chunks(const u32x4_t* c) {
        lo = __builtin_bit_cast(f32x4_t, c[0]);
        hi = __builtin_bit_cast(f32x4_t, c[1]);
    }
    __device__ double get(int e) const { return (double)(e < 4 ? lo[e] : hi[e - 4]); }
};

__device__ __forceinline__ void store_vals(uint16_t* p, const double* v, int n) {
    // n = 4 (8 bytes) or 8 (16 bytes), each value rounded once to bf16
    uint32_t u[4];
    if (n == 8) {
        f64_to_bf16_packed<8>(v, u);
        st16(p, u32x4_t{u[0], u[1], u[2], u[3]});
    } else {
        f64_to_bf16_packed<4>(v, u);
        *reinterpret_cast<u32x2_t*>(p) = u32x2_t{u[0], u[1]};
    }
}
__device__ __forceinline__ void store_vals(float* p, const double* v, int n) {
    *reinterpret_cast<f32x4_t*>(p) = f32x4_t{(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
    if (n == 8) *reinterpret_cast<f32x4_t*>(p + 4) = f32x4_t{(float)v[4], (float)v[5], (float)v[6], (float)v[7]};
}

// Sum over aligned groups of W (8 or 16) consecutive lanes, every lane of a
// group ending with its total: DPP pair, quad, half-row-mirror and row-mirror
// exchanges of the two 32-bit halves (no LDS round trips).
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v) {
    const int2 u = __builtin_bit_cast(int2, v);
    int2 r;
    r.x = __builtin_amdgcn_update_dpp(u.x, u.x, CTRL, 0xF, 0xF, false);
    r.y = __builtin_amdgcn_update_dpp(u.y, u.y, CTRL, 0xF, 0xF, false);
    return __builtin_bit_cast(double, r);
}
template <int W>
__device__ __forceinline__ double group_sum(double v) {
    static_assert(W == 8 || W == 16, "row groups of 8 or 16 lanes");
    v += dpp_f64<0xB1>(v);    // quad_perm 1,0,3,2
    v += dpp_f64<0x4E>(v);    // quad_perm 2,3,0,1
    v += dpp_f64<0x141>(v);   // row_half_mirror
    if (W == 16) v += dpp_f64<0x140>(v);   // row_mirror
    return v;
}

constexpr int kTokThreads = 256;

// One launch can finish a token's query heads (token-major, written to qy)
// and its key heads (into the cache, values copied alongside): "virtual"
// heads 0..nq-1 are the queries, nq..nq+nk-1 the keys.
struct RopeTokArgs {
    const void* qx;
    void* qy;
    const float* qw;
    int nq;
    const void* kx;
    const void* vx;
    void* kc;
    void* vc;
    const float* kw;
    int nk;
    const int32_t* cu_seq;
    const int32_t* start;
    const float* inv_freq;
    double eps;
    float rope_scale;
    int n_tok, cap, rotary_dim, norm, ring, v_norm;
};

template <typename T, int HD>
__global__ __launch_bounds__(kTokThreads) void rope_token_kernel(RopeTokArgs a) {
    constexpr int TPH = HD / 8;                // lanes per head row
    constexpr int HPB = kTokThreads / TPH;     // head rows per workgroup
    constexpr int VPER = 16 / sizeof(T);       // elements per 16-byte chunk
    constexpr int VCH = 8 / VPER;              // 16-byte V chunks per lane
    __shared__ double cs_cos[HD / 2];
    __shared__ double cs_sin[HD / 2];
    __shared__ double w_eff[2][HD];            // query weights, then key weights

    const int b = blockIdx.z;
    const int i = blockIdx.x;
    const int seq0 = a.cu_seq[b];
    const int len = a.cu_seq[b + 1] - seq0;
    if (i >= len) return;
    const int t = seq0 + i;
    const int pos = a.start[b] + i;
    if (t < 0 || t >= a.n_tok || pos < 0) return;
    const int nq = a.nq;
    // no cache row past the capacity (a ring has a row for every position)
    const int nk = a.ring || pos < a.cap ? a.nk : 0;
    const int slot = a.ring && a.nk ? pos % a.cap : pos;
    const int n_all = nq + nk;
    const int h_base = blockIdx.y * HPB;
    if (h_base >= n_all) return;               // uniform over the workgroup

    const int rd = a.rotary_dim;
    const int half = rd / 2;
    const int np = rd / 8;                     // pair lanes per row
    const int tid = threadIdx.x;
    const int c = tid % TPH;
    const bool pair = c < np;
    // first dim of this lane's 8 (pair: 4 + 4 at d0 and d0 + half)
    const int d0 = pair ? 4 * c : rd + 8 * (c - np);
    const int vh = h_base + tid / TPH;
    // rows of one head are whole groups of TPH lanes (whole DPP rows or half
    // rows), so a row is entirely valid or entirely past the last head, and
    // the norm's group sum reads only its own row
    const bool valid = vh < n_all;
    const bool is_q = vh < nq;
    const int kh = vh - nq;

    Raw<T> raw;
    u32x4_t vbuf[VCH] = {};
    if (valid) {
        const T* row = is_q ? reinterpret_cast<const T*>(a.qx) + ((size_t)t * nq + vh) * HD
                            : reinterpret_cast<const T*>(a.kx) + ((size_t)t * a.nk + kh) * HD;
        if (pair) raw.load4x2(row + d0, row + d0 + half);
        else raw.load8(row + d0);
        if (!is_q) {
            // this lane's share of the matching V row, copied unchanged
            const T* vs = reinterpret_cast<const T*>(a.vx) + ((size_t)t * a.nk + kh) * HD + c * 8;
#pragma unroll
            for (int j = 0; j < VCH; ++j) vbuf[j] = ld16(vs + j * VPER);
        }
    }

    for (int k = tid; k < half; k += kTokThreads) {
        // position * f_k is exact in double (integer times a float)
        const double th = (double)pos * (double)a.inv_freq[k];
        double sn, cn;
        sincos_pos(th, &sn, &cn);
        cs_cos[k] = cn;
        cs_sin[k] = sn;
    }
    if (a.norm != 0) {
        for (int k = tid; k < 2 * HD; k += kTokThreads) {
            const bool q_side = k < HD;
            if (q_side ? nq == 0 : nk == 0) continue;
            const double w = (double)(q_side ? a.qw[k] : a.kw[k - HD]);
            w_eff[q_side ? 0 : 1][k % HD] = a.norm == 2 ? 1.0 + w : w;
        }
    }
    __syncthreads();
    if (!valid) return;

    double v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = raw.get(e);
    if (a.norm != 0) {
        double ss = 0.0;
#pragma unroll
        for (int e = 0; e < 8; ++e) ss += v[e] * v[e];
        ss = group_sum<TPH>(ss);
        const double r = 1.0 / sqrt(ss / (double)HD + a.eps);
        const double* we = w_eff[is_q ? 0 : 1];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int d = pair ? d0 + (e & 3) + (e >> 2) * half : d0 + e;
            v[e] = v[e] * r * we[d];
        }
    }
    T* dst = is_q ? reinterpret_cast<T*>(a.qy) + ((size_t)t * nq + vh) * HD
                  : reinterpret_cast<T*>(a.kc) + (((size_t)b * a.nk + kh) * a.cap + slot) * HD;
    if (pair) {
        const double rs = (double)a.rope_scale;
        const bool scaled = a.rope_scale != 1.f;
        double y[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const double cn = cs_cos[d0 + e], sn = cs_sin[d0 + e];
            y[e] = v[e] * cn - v[e + 4] * sn;
            y[e + 4] = v[e] * sn + v[e + 4] * cn;
        }
        if (scaled) {
#pragma unroll
            for (int e = 0; e < 8; ++e) y[e] *= rs;
        }
        store_vals(dst + d0, y, 4);
        store_vals(dst + d0 + half, y + 4, 4);
    } else {
        store_vals(dst + d0, v, 8);
    }
    if (a.v_norm) {
        // V rows: scale-less RMS norm over the row's lanes (dims 8c..8c+7
        // each), in double, each value rounded once; query rows of the wave
        // take part in the row sums with their own (unused) groups
        Raw<T> vr;
        vr.from_chunks(vbuf);
        double w[8], ss = 0.0;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            w[e] = vr.get(e);
            ss += w[e] * w[e];
        }
        ss = group_sum<TPH>(ss);
        const double r = 1.0 / sqrt(ss / (double)HD + a.eps);
#pragma unroll
        for (int e = 0; e < 8; ++e) w[e] *= r;
        if (!is_q) store_vals(reinterpret_cast<T*>(a.vc) + (((size_t)b * a.nk + kh) * a.cap + slot) * HD + c * 8, w, 8);
    } else if (!is_q) {
        T* vd = reinterpret_cast<T*>(a.vc) + (((size_t)b * a.nk + kh) * a.cap + slot) * HD + c * 8;
#pragma unroll
        for (int j = 0; j < VCH; ++j) st16(vd + j * VPER, vbuf[j]);
    }
}

static bool token_path(const RopeArgs& a) {
    return a.rotary_dim % 8 == 0 && (a.head_dim == 64 || a.head_dim == 128);
}

template <typename T>
static void launch_token(const RopeTokArgs& t, int head_dim, int max_chunk, int n_seq, hipStream_t stream) {
    const int per_block = kTokThreads / (head_dim / 8);
    const dim3 grid(max_chunk, (t.nq + t.nk + per_block - 1) / per_block, n_seq);
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
    if (token_path(a)) {
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

// Queries and keys/values of one chunk: one launch on the token path (both
// share the position table), otherwise the two general launches.
hipError_t launch_rope_qkv(const RopeArgs& q, const RopeArgs& kv, int dtype, hipStream_t stream) {
    if (token_path(q)) {
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
