// Per-token finish of a chunk's rows (RMS qk-norm, half-split RoPE, one
// rounding), shared by the standalone RoPE launch and by the prefill kernels,
// which can run the next chunk's finish in the workgroups past their
// attention items.
//
// Sources: cortiq-engine 0.5.39 src/attention.rs -- fn rmsnorm_head (norm in
// double, x*r*w or x*r*(1+w)), fn rope_rotate_scaled (pairs (i, i+rd/2), both
// outputs scaled), fn finish_projection (norm before RoPE, partial rotary on
// the first rd dims), fn qwen_attention_batch (every row of the chunk is
// appended before the chunk attends).
#pragma once

#include "device_common.h"
#include "launch.h"

namespace attn {

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

// LDS of TOK tokens: their cos/sin tables and the effective norm weights.
template <int HD, int TOK = 1>
struct RopeTokSmem {
    double cs_cos[TOK][HD / 2];
    double cs_sin[TOK][HD / 2];
    double w_eff[2][HD];
};

// One workgroup of NT threads finishes head rows hb*HPB .. of tokens
// i0 .. i0+TOK-1 of sequence b: every thread issues the loads of all its
// tokens first, the tables of all of them are built while those are in
// flight, then each token's rows are finished in turn.  The only exit
// before the workgroup barrier depends on (i0, hb, b) alone, so the whole
// workgroup takes it together.
template <typename T, int HD, int NT, int TOK = 1>
__device__ __forceinline__ void rope_token_body(const RopeTokArgs& a, int i0, int hb, int b,
                                                RopeTokSmem<HD, TOK>& sm) {
    constexpr int TPH = HD / 8;                // lanes per head row
    constexpr int HPB = NT / TPH;              // head rows per workgroup
    constexpr int VPER = 16 / sizeof(T);       // elements per 16-byte chunk
    constexpr int VCH = 8 / VPER;              // 16-byte V chunks per lane
    auto& w_eff = sm.w_eff;                    // query weights, then key weights

    const int seq0 = a.cu_seq[b];
    const int len = a.cu_seq[b + 1] - seq0;
    const int p0 = a.start[b];
    const int nq = a.nq;
    const int h_base = hb * HPB;
    // the workgroup's tokens: packed row, position, cache row, head rows
    // (no cache row past the capacity; a ring has a row for every position)
    int tt[TOK], pp[TOK], slot[TOK], n_all[TOK];
    bool act[TOK];
    bool any = false;
#pragma unroll
    for (int u = 0; u < TOK; ++u) {
        const int i = i0 + u;
        tt[u] = seq0 + i;
        pp[u] = p0 + i;
        const int nk = a.ring || pp[u] < a.cap ? a.nk : 0;
        n_all[u] = nq + nk;
        slot[u] = a.ring && a.nk ? pp[u] % a.cap : pp[u];
        act[u] = i < len && tt[u] >= 0 && tt[u] < a.n_tok && pp[u] >= 0 && h_base < n_all[u];
        any = any || act[u];
    }
    if (!any) return;                          // uniform over the workgroup

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
    const bool is_q = vh < nq;
    const int kh = vh - nq;

    Raw<T> raw[TOK];
    u32x4_t vbuf[TOK][VCH];
#pragma unroll
    for (int u = 0; u < TOK; ++u) {
#pragma unroll
        for (int j = 0; j < VCH; ++j) vbuf[u][j] = u32x4_t{0u, 0u, 0u, 0u};
        if (!(act[u] && vh < n_all[u])) continue;
        const T* row = is_q ? reinterpret_cast<const T*>(a.qx) + ((size_t)tt[u] * nq + vh) * HD
                            : reinterpret_cast<const T*>(a.kx) + ((size_t)tt[u] * a.nk + kh) * HD;
        if (pair) raw[u].load4x2(row + d0, row + d0 + half);
        else raw[u].load8(row + d0);
        if (!is_q) {
            // this lane's share of the matching V row, copied unchanged
            const T* vs = reinterpret_cast<const T*>(a.vx) + ((size_t)tt[u] * a.nk + kh) * HD + c * 8;
#pragma unroll
            for (int j = 0; j < VCH; ++j) vbuf[u][j] = ld16(vs + j * VPER);
        }
    }

    for (int k = tid; k < TOK * half; k += NT) {
        const int u = k / half, f = k - u * half;
        // position * f_k is exact in double (integer times a float)
        const double th = (double)max(p0 + i0 + u, 0) * (double)a.inv_freq[f];
        double sn, cn;
        sincos_pos(th, &sn, &cn);
        sm.cs_cos[u][f] = cn;
        sm.cs_sin[u][f] = sn;
    }
    if (a.norm != 0) {
        for (int k = tid; k < 2 * HD; k += NT) {
            const bool q_side = k < HD;
            if (q_side ? nq == 0 : a.nk == 0) continue;
            const double w = (double)(q_side ? a.qw[k] : a.kw[k - HD]);
            w_eff[q_side ? 0 : 1][k % HD] = a.norm == 2 ? 1.0 + w : w;
        }
    }
    __syncthreads();

#pragma unroll
    for (int u = 0; u < TOK; ++u) {
        if (!(act[u] && vh < n_all[u])) continue;
        const double* cs_cos = sm.cs_cos[u];
        const double* cs_sin = sm.cs_sin[u];
        double v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = raw[u].get(e);
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
        T* dst = is_q ? reinterpret_cast<T*>(a.qy) + ((size_t)tt[u] * nq + vh) * HD
                      : reinterpret_cast<T*>(a.kc) + (((size_t)b * a.nk + kh) * a.cap + slot[u]) * HD;
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
            vr.from_chunks(vbuf[u]);
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
            if (!is_q) store_vals(reinterpret_cast<T*>(a.vc) + (((size_t)b * a.nk + kh) * a.cap + slot[u]) * HD + c * 8, w, 8);
        } else if (!is_q) {
            T* vd = reinterpret_cast<T*>(a.vc) + (((size_t)b * a.nk + kh) * a.cap + slot[u]) * HD + c * 8;
#pragma unroll
            for (int j = 0; j < VCH; ++j) st16(vd + j * VPER, vbuf[u][j]);
        }
    }
}

}  // namespace attn
