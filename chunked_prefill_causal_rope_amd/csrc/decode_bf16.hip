// bf16 decode attention: one query per sequence (chunk = 1) over a long
// head-major cache.  Memory-bound: every K/V byte of the context is read once
// per KV group, shared by the group's G query heads.
//
// cortiq-engine 0.5.39 src/attention.rs: fn attention_head (scores, max-
// subtracted softmax, output and probabilities; the work of one decode step is
// proportional to the number of cached positions), fn attend_all_heads (a KV
// group's K/V is streamed once for all of its query heads).
//
// Design (gfx950):
//  * The context of each (sequence, KV group) is split into parts of
//    split_len keys, one single-wave workgroup per part, so a batch of long
//    sequences gives thousands of independent streams.
//  * The wave walks its part 32 keys at a time with the next step's K and V
//    loads (16 KB, nontemporal: every byte is used once) in flight while the
//    current step is computed, so HBM always has work queued.
//  * Scores for 16 keys come from v_mfma_f32_16x16x32_bf16 with A = the
//    group's queries and B = K rows straight from global memory.  Query head
//    h sits in A row 4*(h/HPL) + h%HPL, so in the result the 16-lane group j
//    holds heads j*HPL.. and lane j*16+c holds key c: softmax reductions are
//    four DPP steps inside a 16-lane row.
//  * P.V runs on the vector ALU in float32: each lane owns 8 dims of V for
//    every (512/head_dim)-th key, so one wave load covers 1 KB of
//    consecutive rows; the probabilities reach those lanes through LDS.
//  * The running maximum only moves (and O is rescaled) when a score exceeds
//    it by more than 2^8; until then probabilities are referenced to the old
//    maximum, which leaves the softmax unchanged.
//  * Each part leaves (m, l, O) in the workspace and, when asked, its
//    unnormalised probabilities 2^(x - m) (x the log2-domain score, m the
//    part's running maximum) as half-precision values packed at the start of
//    each probabilities row -- half the bytes of the float scores, which
//    matters because writes among the K/V read stream cost far more than
//    their size.  The combine kernel merges the parts with log-sum-exp and
//    widens each row in place to the normalised float probabilities.
#include <algorithm>

#include "device_common.h"
#include "launch.h"

namespace attn {

constexpr int kDecKB = 32;      // keys per step
// A partial: (m, l, l_half, e) as floats, then O/l * 2^-e as head_dim halves
// (see part_scale_exp).
constexpr int kPartHeadD = 4;
__host__ __device__ constexpr int dec_part_words(int hd) { return kPartHeadD + hd / 2; }
constexpr int kDecMaxGroup = 16;
constexpr float kDecSlack = 8.f;
// LDS floats per wave that hold a part's raw scores (16 KB)
constexpr int kDecPartFloats = 4096;

int decode_group_limit() { return kDecMaxGroup; }

// Sliding window: a row reads keys [ctx - W, ctx).  The parts start at that
// first key rounded down to a step, so they begin on a step (and a 16-byte
// boundary of the half-precision rows) and the first step holds a key of the
// window; the keys between the part start and the window are masked.
__host__ __device__ constexpr int decode_window_first(int ctx, int window) {
    return window > 0 && ctx > window ? ctx - window : 0;
}
__host__ __device__ constexpr int decode_part_base(int ctx, int window) {
    return decode_window_first(ctx, window) / kDecKB * kDecKB;
}
// The keys and query rows of sequence b: decode, one query at ctx-1; a small
// chunk, nq queries at ctx-nq .. ctx-1 (ctx = start + len).  Returns false
// when the sequence has no row.
__device__ __forceinline__ bool decode_rows(const DecodeArgs& a, int b, int& ctx, int& nq) {
    if (a.cu_seq) {
        nq = min(a.cu_seq[b + 1] - a.cu_seq[b], a.n_q);
        const int st = a.start[b];
        if (nq <= 0 || st < 0) return false;
        ctx = a.ring ? st + nq : min(st + nq, a.cap);
        return true;
    }
    nq = 1;
    ctx = a.ring ? min(a.ctx[b], a.max_ctx) : min(min(a.ctx[b], a.max_ctx), a.cap);
    return true;
}
int decode_key_span(int max_ctx, int window) {
    return window > 0 && window < max_ctx ? std::min(window + kDecKB - 1, max_ctx) : max_ctx;
}

// Heads handled per KV group by the kernel instance (4, 8 or 16); with
// probabilities a part holds at most kDecPartFloats / that many keys.
static int decode_heads_padded(int group) { return group <= 4 ? 4 : group <= 8 ? 8 : 16; }
int decode_part_limit(int group, bool probs) {
    return probs ? kDecPartFloats / decode_heads_padded(group) : 1 << 30;
}

__device__ __forceinline__ f32x4_t mfma16(bf16x8_t a, bf16x8_t b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// DPP reductions over the 16 lanes of a row: pair, quad, half-row mirror,
// row mirror.  Every lane of the row ends with the result.
__device__ __forceinline__ float dpp_f(float x, int ctrl_sel) {
    const int v = __float_as_int(x);
    int r;
    switch (ctrl_sel) {
        case 0: r = __builtin_amdgcn_update_dpp(v, v, 0xB1, 0xF, 0xF, false); break;   // quad_perm 1,0,3,2
        case 1: r = __builtin_amdgcn_update_dpp(v, v, 0x4E, 0xF, 0xF, false); break;   // quad_perm 2,3,0,1
        case 2: r = __builtin_amdgcn_update_dpp(v, v, 0x141, 0xF, 0xF, false); break;  // row_half_mirror
        default: r = __builtin_amdgcn_update_dpp(v, v, 0x140, 0xF, 0xF, false); break; // row_mirror
    }
    return __int_as_float(r);
}
__device__ __forceinline__ float row16_max(float x) {
#pragma unroll
    for (int c = 0; c < 4; ++c) x = fmaxf(x, dpp_f(x, c));
    return x;
}
__device__ __forceinline__ float row16_sum(float x) {
#pragma unroll
    for (int c = 0; c < 4; ++c) x += dpp_f(x, c);
    return x;
}

// A 16-byte vector that only needs 4-byte alignment (probability rows start
// wherever probs_ld puts them; global accesses need no wider alignment).
typedef float f32x4_a4_t __attribute__((ext_vector_type(4), aligned(4)));

__device__ __forceinline__ u32x4_t ld16_nt(const uint16_t* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
}

// The workgroup is one wave, whose LDS accesses execute in program order, so
// exchanging values between lanes through LDS only needs the compiler to
// keep the accesses in order (a fence would also wait for the global loads
// in flight, which are the next step's prefetch).
__device__ __forceinline__ void lds_order() { asm volatile("" ::: "memory"); }

// A part's raw scores x, [head][key] in LDS (PK keys per head), written as
// half-precision 2^(x - m_h), m_h the head's running maximum in mr, to keys
// [base, base+n) of the heads' 16-bit rows (p <= 2^8: a score never exceeds
// the maximum by more than the slack).  The sums of the rounded values are
// added to lh, so the probabilities normalised by them sum to 1 exactly (up
// to float rounding).
typedef uint32_t u32x4_a4_t __attribute__((ext_vector_type(4), aligned(4)));
template <int PK>
__device__ __forceinline__ void write_half_scores(const float* sb, const float* mr, float* lh, uint16_t* hrow,
                                                  size_t hrow_ld, int G, int base, int n, int lane) {
    for (int t = lane; t < G * (PK / 8); t += 64) {
        const int hh = t / (PK / 8), kq = 8 * (t % (PK / 8));
        if (kq >= n) continue;
        const float m = mr[hh];
        uint32_t w[4];
        float sum = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            w[e] = pack_f16x2(__builtin_amdgcn_exp2f(sb[hh * PK + kq + 2 * e] - m),
                              __builtin_amdgcn_exp2f(sb[hh * PK + kq + 2 * e + 1] - m));
            // buffer entries past n hold nothing of this part
            if (kq + 2 * e < n) sum += f16_value((uint16_t)w[e]);
            if (kq + 2 * e + 1 < n) sum += f16_value((uint16_t)(w[e] >> 16));
        }
        atomicAdd(&lh[hh], sum);
        uint16_t* dst = hrow + hh * hrow_ld + base + kq;
        if (kq + 7 < n) {
            *reinterpret_cast<u32x4_a4_t*>(dst) = u32x4_a4_t{w[0], w[1], w[2], w[3]};
        } else {
#pragma unroll
            for (int e = 0; e < 7; ++e)
                if (kq + e < n) dst[e] = (uint16_t)(w[e >> 1] >> (16 * (e & 1)));
        }
    }
}

// After the running maximum moved, the values a part already wrote (keys
// [k_lo, k_lo + n)) are multiplied by the heads' factors fac, so every
// written value stays referenced to the current maximum.  Only parts longer
// than the LDS buffer write any before their end, and the maximum rarely
// moves after the first PK keys.
__device__ __forceinline__ void rescale_half_scores(const float* fac, float* lh, uint16_t* hrow, size_t hrow_ld,
                                                    int G, int k_lo, int n, int lane) {
    __threadfence();            // this wave's own earlier writes first
    if (lane < G) lh[lane] *= fac[lane];
    const int per = (n + 7) / 8;
    for (int t = lane; t < G * per; t += 64) {
        const int hh = t / per, kq = 8 * (t % per);
        const float f = fac[hh];
        uint16_t* dst = hrow + hh * hrow_ld + k_lo + kq;
        for (int e = 0; e < 8 && kq + e < n; ++e) dst[e] = f16_bits(f16_value(dst[e]) * f);
    }
    __threadfence();
}

// LONG: parts may be longer than the raw-score buffer (a small workspace);
// only that instance carries the mid-part writes and their rescale, which
// would otherwise add to the streaming loop's registers.  RING: the cache is
// a ring of cap rows (key k in row k mod cap) that has wrapped.
// Two waves per SIMD (at most 256 registers) where the instance fits them
// without spilling: occupancy is what keeps HBM busy, and left alone the
// compiler may take a few registers past the limit and halve it.
template <int HD, int HPL, bool PROBS, bool LONG, bool RING>
__global__ __launch_bounds__(64, (HPL == 1 || (HPL == 2 && !LONG) ? 2 : 1)) void decode_split_kernel(DecodeArgs a) {
    constexpr int GQ = 4 * HPL;                 // query heads per group handled
    constexpr int NK = HD / 32;                 // K-steps per 16x16x32 product
    constexpr int CPR = HD / 8;                 // 16-byte chunks per cache row
    constexpr int RPI = 64 / CPR;               // V rows per wave load
    constexpr int NV = kDecKB / RPI;            // V loads per lane per step
    __shared__ __attribute__((aligned(16))) float pbuf[kDecKB * GQ];   // P[key][head]
    __shared__ __attribute__((aligned(16))) float abuf[GQ];
    __shared__ float mref[GQ];                  // running maximum per head, for flushes
    __shared__ float lhalf[GQ];                 // sums of the written half-precision values
    // the part's raw scores, [head][key], written out once the part is done
    __shared__ __attribute__((aligned(16))) float sbuf[PROBS ? kDecPartFloats : 4];
    constexpr int PK = kDecPartFloats / GQ;     // longest part with probabilities

    const int lane = threadIdx.x;
    int id = blockIdx.x;
    const int g = id % a.n_kv;
    id /= a.n_kv;
    const int s = id % a.n_splits;
    const int b = id / a.n_splits;
    if (b >= a.n_seq) return;
    int ctx, nq_b;
    if (!decode_rows(a, b, ctx, nq_b)) return;
    // the first key any row reads: the window start of the first query
    const int k_first = decode_window_first(ctx - nq_b + 1, a.window);
    const int k_lo = decode_part_base(ctx - nq_b + 1, a.window) + s * a.split_len;
    const int k_hi = min(k_lo + a.split_len, ctx);
    if (k_lo >= k_hi) return;
    const int G = a.group;
    const int GV = G * a.n_q;                   // query rows of the group (heads x queries)
    if (PROBS && lane < GQ) lhalf[lane] = 0.f;

    const int col = lane & 15;   // score layout: key within a 16-key block
    const int grp = lane >> 4;   // score layout: heads grp*HPL .. grp*HPL+HPL-1
    const int vc_ = lane % CPR;  // P.V layout: dims 8*vc_ .. 8*vc_+7
    const int vr = lane / CPR;   // P.V layout: keys vr, vr+RPI, ...

    bf16x8_t qa[NK];
    {
        // A row `col` holds query row (col/4)*HPL + col%4 when col%4 < HPL:
        // query qi of head qh of the group
        const int hq = (col >> 2) * HPL + (col & 3);
        const int qi = hq / G, qh = hq - qi * G;
        const bool ok = (col & 3) < HPL && hq < GV && qi < nq_b;
        const size_t qt = a.cu_seq ? (size_t)a.cu_seq[b] + (ok ? qi : 0) : (size_t)b;
        const uint16_t* qb =
            reinterpret_cast<const uint16_t*>(a.q) + (qt * a.n_heads + g * G + (ok ? qh : 0)) * HD;
#pragma unroll
        for (int k = 0; k < NK; ++k) {
            u32x4_t u = {0u, 0u, 0u, 0u};
            if (ok) u = ld16(qb + 32 * k + 8 * grp);
            qa[k] = __builtin_bit_cast(bf16x8_t, u);
        }
    }
    const size_t base = ((size_t)b * a.n_kv + g) * (size_t)a.cap * HD;
    const uint16_t* kc = reinterpret_cast<const uint16_t*>(a.k_cache) + base;
    const uint16_t* vcache = reinterpret_cast<const uint16_t*>(a.v_cache) + base;
    // half-precision values of head hh, key k: element k of the row read as
    // 16-bit words (bytes 2k..2k+1 of the float row, inside its first ctx
    // entries)
    uint16_t* hrow = PROBS ? reinterpret_cast<uint16_t*>(a.probs + ((size_t)b * a.n_heads + g * G) * a.probs_ld)
                           : nullptr;
    const size_t hrow_ld = 2 * (size_t)a.probs_ld;   // 16-bit words per row

    float m_run[HPL], l_run[HPL];
#pragma unroll
    for (int r = 0; r < HPL; ++r) {
        m_run[r] = -INFINITY;
        l_run[r] = 0.f;
    }
    // keys each of this lane's rows may read: up to its own position, from
    // its window start
    int key_min[HPL], key_max[HPL];
#pragma unroll
    for (int r = 0; r < HPL; ++r) {
        const int pos = ctx - nq_b + (grp * HPL + r) / G;
        key_max[r] = min(pos, k_hi - 1);
        key_min[r] = a.window > 0 ? max(pos - a.window + 1, 0) : 0;
    }
    float o[GQ][8];
#pragma unroll
    for (int hh = 0; hh < GQ; ++hh)
#pragma unroll
        for (int e = 0; e < 8; ++e) o[hh][e] = 0.f;
    const float sl = a.scale * kLog2e;
    const int last = k_hi - 1;
    // Ring: the keys of the window this part reads, [key_lo, k_hi), span at
    // most cap rows, so key k (clamped up to key_lo: keys below the window
    // are masked) lives in row k - wrap, less cap once past the ring's end.
    const int key_lo = max(k_lo, k_first);
    const int wrap = RING ? key_lo - key_lo % a.cap : 0;
    auto row_of = [&](int key) __attribute__((always_inline)) {
        if (!RING) return key;
        const int r = max(key, key_lo) - wrap;
        return r >= a.cap ? r - a.cap : r;
    };

    // Rows past the part's end read as zeros (buffer loads) or re-read its
    // last row (ring); their scores are masked to -inf so their
    // probabilities are exactly 0.
    u32x4_t kf[2][2][NK], vf[2][NV];
    // Without a ring the part's rows are contiguous: each step's loads are
    // buffer loads from a resource over that step's rows (base and size in
    // scalar registers, fixed per-lane offsets: no per-load address
    // arithmetic), and rows past the part's end read as zeros without
    // touching memory.  Nontemporal (every byte is used once).
    constexpr int kNT = 2;       // cache policy bit: nontemporal
    const int koff = (col * HD + 8 * grp) * 2, voff = (vr * HD + 8 * vc_) * 2;
    auto load = [&](int k0, int buf) __attribute__((always_inline)) {
        if constexpr (!RING) {
            const int nb = min(max(k_hi - k0, 0), kDecKB) * HD * 2;
            const auto krs = uniform_rsrc(kc + (size_t)k0 * HD, nb);
            const auto vrs = uniform_rsrc(vcache + (size_t)k0 * HD, nb);
#pragma unroll
            for (int blk = 0; blk < 2; ++blk)
#pragma unroll
                for (int k = 0; k < NK; ++k)
                    kf[buf][blk][k] = __builtin_bit_cast(
                        u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(krs, koff + 16 * blk * HD * 2 + 64 * k, 0, kNT));
#pragma unroll
            for (int i = 0; i < NV; ++i)
                vf[buf][i] = __builtin_bit_cast(
                    u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(vrs, voff + RPI * i * HD * 2, 0, kNT));
            return;
        }
#pragma unroll
        for (int blk = 0; blk < 2; ++blk) {
            const int key = row_of(min(k0 + 16 * blk + col, last));
#pragma unroll
            for (int k = 0; k < NK; ++k) kf[buf][blk][k] = ld16_nt(kc + (size_t)key * HD + 32 * k + 8 * grp);
        }
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int key = row_of(min(k0 + RPI * i + vr, last));
            vf[buf][i] = ld16_nt(vcache + (size_t)key * HD + 8 * vc_);
        }
    };

    // Raw scores wait in LDS and are written once per PK keys (normally once
    // per part): a global write among the K/V reads stalls the read stream
    // far more than its size suggests (HBM read/write turnaround).
    auto flush = [&](int base, int n) __attribute__((always_inline)) {
        if (col == 0) {
#pragma unroll
            for (int r = 0; r < HPL; ++r) mref[grp * HPL + r] = m_run[r];
        }
        lds_order();
        write_half_scores<PK>(sbuf, mref, lhalf, hrow, hrow_ld, G, base, n, lane);
        lds_order();
    };

    auto step = [&](int k0, int buf) __attribute__((always_inline)) {
        float x[2][HPL];
#pragma unroll
        for (int blk = 0; blk < 2; ++blk) {
            f32x4_t S = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int k = 0; k < NK; ++k) S = mfma16(qa[k], __builtin_bit_cast(bf16x8_t, kf[buf][blk][k]), S);
            const int key = k0 + 16 * blk + col;
#pragma unroll
            for (int r = 0; r < HPL; ++r)
                x[blk][r] = key <= key_max[r] && key >= key_min[r] ? S[r] * sl : -INFINITY;
        }
        bool grow_any = false;
        float mt[HPL];
#pragma unroll
        for (int r = 0; r < HPL; ++r) {
            mt[r] = row16_max(fmaxf(x[0][r], x[1][r]));
            grow_any |= mt[r] > m_run[r] + kDecSlack;
        }
        if (__any(grow_any)) {
            float al[HPL];
#pragma unroll
            for (int r = 0; r < HPL; ++r) {
                const bool grow = mt[r] > m_run[r] + kDecSlack;
                al[r] = grow ? __builtin_amdgcn_exp2f(m_run[r] - mt[r]) : 1.f;
                m_run[r] = grow ? mt[r] : m_run[r];
                l_run[r] *= al[r];
            }
            if (col == 0) {
#pragma unroll
                for (int r = 0; r < HPL; ++r) abuf[grp * HPL + r] = al[r];
            }
            lds_order();
            if (PROBS && LONG && k0 - k_lo >= PK) rescale_half_scores(abuf, lhalf, hrow, hrow_ld, G, k_lo, (k0 - k_lo) / PK * PK, lane);
#pragma unroll
            for (int hq = 0; hq < GQ / 4; ++hq) {
                const float4 f = *reinterpret_cast<const float4*>(&abuf[4 * hq]);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    o[4 * hq + 0][e] *= f.x;
                    o[4 * hq + 1][e] *= f.y;
                    o[4 * hq + 2][e] *= f.z;
                    o[4 * hq + 3][e] *= f.w;
                }
            }
        }
        // a row none of whose keys so far was readable has m = -inf and
        // probabilities 0
        float m_use[HPL];
#pragma unroll
        for (int r = 0; r < HPL; ++r) m_use[r] = m_run[r] == -INFINITY ? 0.f : m_run[r];
#pragma unroll
        for (int blk = 0; blk < 2; ++blk)
#pragma unroll
            for (int r = 0; r < HPL; ++r) {
                const float p = __builtin_amdgcn_exp2f(x[blk][r] - m_use[r]);
                l_run[r] += p;
                pbuf[(16 * blk + col) * GQ + grp * HPL + r] = p;
            }
        lds_order();
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int kl = RPI * i + vr;
            float v[8];
            v[0] = bf16_lo(vf[buf][i].x);
            v[1] = bf16_hi(vf[buf][i].x);
            v[2] = bf16_lo(vf[buf][i].y);
            v[3] = bf16_hi(vf[buf][i].y);
            v[4] = bf16_lo(vf[buf][i].z);
            v[5] = bf16_hi(vf[buf][i].z);
            v[6] = bf16_lo(vf[buf][i].w);
            v[7] = bf16_hi(vf[buf][i].w);
#pragma unroll
            for (int hq = 0; hq < GQ / 4; ++hq) {
                const float4 p = *reinterpret_cast<const float4*>(&pbuf[kl * GQ + 4 * hq]);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    o[4 * hq + 0][e] += p.x * v[e];
                    o[4 * hq + 1][e] += p.y * v[e];
                    o[4 * hq + 2][e] += p.z * v[e];
                    o[4 * hq + 3][e] += p.w * v[e];
                }
            }
        }
        // pbuf/abuf are rewritten by the next step
        lds_order();
        if (PROBS) {
            const int kb = (k0 - k_lo) % PK;      // PK is a multiple of 64
#pragma unroll
            for (int blk = 0; blk < 2; ++blk)
#pragma unroll
                for (int r = 0; r < HPL; ++r) sbuf[(grp * HPL + r) * PK + kb + 16 * blk + col] = x[blk][r];
            // a part longer than the buffer writes it out each time it fills
            if (LONG && kb + kDecKB == PK && k0 + kDecKB < k_hi) flush(k0 + kDecKB - PK, PK);
        }
    };

    // two register sets: the loads of step i+1 are issued before step i
    // runs.  They are unconditional (a prefetch past the part's end reads
    // zeros, or its last row over a ring) so the compiler's wait counts stay
    // exact.
    // Steps go in pairs; an odd count ends with a step whose keys are all
    // past the part (scores -inf, probabilities 0, nothing stored).
    load(k_lo, 0);
    for (int k0 = k_lo; k0 < k_hi; k0 += 2 * kDecKB) {
        load(k0 + kDecKB, 1);
        step(k0, 0);
        load(k0 + 2 * kDecKB, 0);
        step(k0 + kDecKB, 1);
    }

    // the rest of the part's raw scores
    if (PROBS) {
        const int last_base = k_lo + (k_hi - 1 - k_lo) / PK * PK;
        flush(last_base, k_hi - last_base);
    }

    // l: sum over the 16 key lanes of each head row; O: sum over the lanes
    // that hold the same dims
#pragma unroll
    for (int r = 0; r < HPL; ++r) l_run[r] = row16_sum(l_run[r]);
#pragma unroll
    for (int hh = 0; hh < GQ; ++hh)
#pragma unroll
        for (int e = 0; e < 8; ++e)
#pragma unroll
            for (int off = CPR; off < 64; off <<= 1) o[hh][e] += __shfl_xor(o[hh][e], off);

    // every head's l to every lane (through LDS), then each head's O/l in
    // half precision with its scale exponent
    if (col == 0) {
#pragma unroll
        for (int r = 0; r < HPL; ++r) abuf[grp * HPL + r] = l_run[r];
    }
    lds_order();
    float linv[GQ];
    int ex[GQ];
#pragma unroll
    for (int hh = 0; hh < GQ; ++hh) {
        const float lv = abuf[hh];
        linv[hh] = lv > 0.f ? 1.f / lv : 0.f;
        float mx = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) mx = fmaxf(mx, fabsf(o[hh][e]));
        // lanes 16j..16j+15 hold every dim of the row (lanes CPR apart repeat)
        ex[hh] = part_scale_exp(row16_max(mx) * linv[hh]);
    }
    // partial of output row (b*n_q + qi)*n_heads + g*G + qh, part s
    constexpr int PS = dec_part_words(HD);
    auto part_of = [&](int v) __attribute__((always_inline)) {
        const int qi = v / G, qh = v - qi * G;
        const size_t row = ((size_t)b * a.n_q + qi) * a.n_heads + g * G + qh;
        return a.part + (row * a.n_splits + s) * PS;
    };
    if (col == 0) {
#pragma unroll
        for (int r = 0; r < HPL; ++r) {
            const int hh = grp * HPL + r;
            if (hh < GV && hh / G < nq_b)
                *reinterpret_cast<float4*>(part_of(hh)) =
                    make_float4(m_run[r], l_run[r], PROBS ? lhalf[hh] : 0.f, (float)ex[hh]);
        }
    }
    if (vr == 0) {
#pragma unroll
        for (int hh = 0; hh < GQ; ++hh) {
            if (hh < GV && hh / G < nq_b) {
                const float sc = __builtin_amdgcn_ldexpf(linv[hh], -ex[hh]);
                uint32_t* dst = reinterpret_cast<uint32_t*>(part_of(hh) + kPartHeadD) + 4 * vc_;
                *reinterpret_cast<u32x4_t*>(dst) =
                    u32x4_t{pack_f16x2(o[hh][0] * sc, o[hh][1] * sc), pack_f16x2(o[hh][2] * sc, o[hh][3] * sc),
                            pack_f16x2(o[hh][4] * sc, o[hh][5] * sc), pack_f16x2(o[hh][6] * sc, o[hh][7] * sc)};
            }
        }
    }
}

// One workgroup per (sequence, head): merge the parts that cover
// [0, ctx) and, when asked, rewrite the raw scores as probabilities
// P_j = 2^(x_j - m) / l.
__device__ __forceinline__ float block_reduce(float v, float* sh, bool is_max) {
    v = is_max ? wave_max(v) : wave_sum(v);
    const int w = threadIdx.x >> 6;
    __syncthreads();                    // sh may still be read from a previous reduction
    if ((threadIdx.x & 63) == 0) sh[w] = v;
    __syncthreads();
    float r = sh[0];
#pragma unroll
    for (int i = 1; i < 4; ++i) r = is_max ? fmaxf(r, sh[i]) : r + sh[i];
    return r;
}

template <int HD>
__global__ __launch_bounds__(256) void decode_combine_kernel(DecodeArgs a) {
    __shared__ float red[4];
    __shared__ float osum[256];
    // output row (b*n_q + qi)*n_heads + h: query qi of sequence b, head h
    const int row = blockIdx.x;
    const int b = row / (a.n_heads * a.n_q);
    const int qi = (row / a.n_heads) % a.n_q;
    const int tid = threadIdx.x;
    if (b >= a.n_seq) return;
    int ctx, nq_b;
    if (!decode_rows(a, b, ctx, nq_b) || qi >= nq_b) return;
    // the packed row of the query (decode: the sequence)
    const size_t orow_id = a.cu_seq ? ((size_t)a.cu_seq[b] + qi) * a.n_heads + row % a.n_heads : (size_t)row;
    float* orow = a.out + orow_id * HD;
    if (ctx < 1) {
        for (int d = tid; d < HD; d += 256) orow[d] = 0.f;
        return;
    }
    constexpr int PS = dec_part_words(HD);
    const int k_first = decode_window_first(ctx, a.window);
    const int k_base = decode_part_base(ctx - nq_b + 1, a.window);
    const int n_parts = min((ctx - k_base + a.split_len - 1) / a.split_len, a.n_splits);
    // output gate factor of this thread's dim, loaded before the merge
    const float gf = a.gate.mode && tid < HD ? gate_factor_bf16(a.gate, orow_id, tid) : 1.f;
    const float* pr = a.part + (size_t)row * a.n_splits * PS;
    float mm = -INFINITY;
    for (int s = tid; s < n_parts; s += 256) mm = fmaxf(mm, pr[(size_t)s * PS]);
    const float m = block_reduce(mm, red, true);
    float ll = 0.f;
    for (int s = tid; s < n_parts; s += 256)
        ll += pr[(size_t)s * PS + 1] * __builtin_amdgcn_exp2f(pr[(size_t)s * PS] - m);
    const float l = block_reduce(ll, red, false);
    const float inv = 1.f / l;
    // the probabilities are normalised by the sum of the half-precision
    // values the parts wrote, so each row sums to 1
    float lh = 0.f;
    if (a.probs)
        for (int s = tid; s < n_parts; s += 256)
            lh += pr[(size_t)s * PS + 2] * __builtin_amdgcn_exp2f(pr[(size_t)s * PS] - m);
    const float inv_h = a.probs ? 1.f / block_reduce(lh, red, false) : 0.f;
    // O: thread -> (dim, phase); phases take every (256/HD)-th part; part s
    // adds its O/l (halves, scaled by 2^-e) with weight l_s 2^(m_s - m) 2^e
    {
        constexpr int PH = 256 / HD;
        const int d = tid % HD, ph = tid / HD;
        auto term = [&](const float4 hdr, uint16_t v) __attribute__((always_inline)) {
            return f16_value(v) * __builtin_amdgcn_ldexpf(hdr.y * __builtin_amdgcn_exp2f(hdr.x - m), (int)hdr.w);
        };
        float acc = 0.f;
        int s = ph;
        for (; s + 3 * PH < n_parts; s += 4 * PH) {
            float4 w[4];
            uint16_t x[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const float* p = pr + (size_t)(s + u * PH) * PS;
                w[u] = *reinterpret_cast<const float4*>(p);
                x[u] = reinterpret_cast<const uint16_t*>(p + kPartHeadD)[d];
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) acc += term(w[u], x[u]);
        }
        for (; s < n_parts; s += PH) {
            const float* p = pr + (size_t)s * PS;
            acc += term(*reinterpret_cast<const float4*>(p), reinterpret_cast<const uint16_t*>(p + kPartHeadD)[d]);
        }
        osum[tid] = acc;
        __syncthreads();
        if (tid < HD) {
            float t = 0.f;
#pragma unroll
            for (int q = 0; q < PH; ++q) t += osum[q * HD + tid];
            orow[tid] = t * inv * gf;
        }
    }
    if (a.probs) {
        // P_j = h_j 2^(m_s - m) / l_h, h_j the half-precision value part s
        // (keys [k_base + s*split_len, ...)) left at 16-bit word j of the
        // row; keys before the window get 0.  The row is widened in place,
        // in blocks of 2048 keys from the top down: float j covers words 2j
        // and 2j+1, which belong to keys at or above j, so a block's writes
        // only reach words of its own keys (read into registers before the
        // barrier) or of blocks already done.  Part bounds are multiples of
        // 8 keys, so 8 consecutive keys share one part.
        float* prow = a.probs + (size_t)row * a.probs_ld;
        const uint16_t* hrow = reinterpret_cast<const uint16_t*>(prow);
        typedef uint32_t u32x4_a4_t __attribute__((ext_vector_type(4), aligned(4)));
        typedef float f32x4_a4_t __attribute__((ext_vector_type(4), aligned(4)));
        constexpr int BLK = 256 * 8;
        for (int lo = (ctx - 1) / BLK * BLK; lo >= 0; lo -= BLK) {
            const int k = lo + 8 * tid;
            float v[8];
            if (k + 8 <= k_base) {
#pragma unroll
                for (int e = 0; e < 8; ++e) v[e] = 0.f;
            } else if (k < ctx) {
                const float f = __builtin_amdgcn_exp2f(pr[(size_t)((k - k_base) / a.split_len) * PS] - m) * inv_h;
                if (k + 8 <= ctx) {
                    const u32x4_a4_t w = *reinterpret_cast<const u32x4_a4_t*>(hrow + k);
#pragma unroll
                    for (int e = 0; e < 8; ++e) v[e] = f16_value((uint16_t)(w[e >> 1] >> (16 * (e & 1)))) * f;
                } else {
#pragma unroll
                    for (int e = 0; e < 8; ++e) v[e] = k + e < ctx ? f16_value(hrow[k + e]) * f : 0.f;
                }
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    if (k + e < k_first) v[e] = 0.f;
            }
            __syncthreads();
            if (k < ctx) {
                if (k + 8 <= ctx) {
                    *reinterpret_cast<f32x4_a4_t*>(prow + k) = f32x4_a4_t{v[0], v[1], v[2], v[3]};
                    *reinterpret_cast<f32x4_a4_t*>(prow + k + 4) = f32x4_a4_t{v[4], v[5], v[6], v[7]};
                } else {
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        if (k + e < ctx) prow[k + e] = v[e];
                }
            }
        }
    }
}

// Importance of each cached position for one decode step, from the
// probabilities the decode call returned: imp[b][j] (+)= sum over heads of
// probs[b][h][j], j < ctx[b] ([ATT] the per-head loop of the decode attention
// adds every head's probability row into one vector, so a position's
// importance is the total probability the heads give it).  Heads are summed in
// order, in float, each thread over 2 consecutive positions (more threads
// keep more of the rows' reads in flight than wider loads per thread); the
// probabilities are read once.
__global__ __launch_bounds__(256) void decode_importance_kernel(ImportanceArgs a) {
    const int b = blockIdx.y;
    if (b >= a.n_seq) return;
    const int ctx = min(min(a.ctx[b], a.max_ctx), a.probs_ld);
    const int j = (blockIdx.x * 256 + threadIdx.x) * 2;
    if (j >= ctx) return;
    const float* pb = a.probs + (size_t)b * a.n_heads * a.probs_ld + j;
    float* dst = a.imp + (size_t)b * a.imp_ld + j;
    const int n = min(2, ctx - j);
    float s[2] = {0.f, 0.f};
    if (n == 2) {
        // sixteen heads' loads in flight at a time, added in head order
        constexpr int U = 16;
        int h = 0;
        for (; h + U <= a.n_heads; h += U) {
            float v[U][2];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                v[u][0] = pb[(size_t)(h + u) * a.probs_ld];
                v[u][1] = pb[(size_t)(h + u) * a.probs_ld + 1];
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                s[0] += v[u][0];
                s[1] += v[u][1];
            }
        }
        for (; h < a.n_heads; ++h)
            for (int e = 0; e < 2; ++e) s[e] += pb[(size_t)h * a.probs_ld + e];
    } else {
        for (int h = 0; h < a.n_heads; ++h) s[0] += pb[(size_t)h * a.probs_ld];
    }
    for (int e = 0; e < n; ++e) dst[e] = a.accumulate ? dst[e] + s[e] : s[e];
}

hipError_t launch_decode_importance(const ImportanceArgs& a, hipStream_t stream) {
    if (a.n_seq <= 0 || a.max_ctx <= 0) return hipSuccess;
    const dim3 grid((unsigned)((a.max_ctx + 511) / 512), (unsigned)a.n_seq);
    decode_importance_kernel<<<grid, dim3(256), 0, stream>>>(a);
    return hipGetLastError();
}

template <int HD, bool PROBS, bool LONG, bool RING>
static void launch_split(const DecodeArgs& a, hipStream_t stream) {
    const dim3 grid((unsigned)((long)a.n_seq * a.n_splits * a.n_kv));
    const int rows = a.group * a.n_q;          // query rows per KV group
    if (rows <= 4)
        decode_split_kernel<HD, 1, PROBS, LONG, RING><<<grid, dim3(64), 0, stream>>>(a);
    else if (rows <= 8)
        decode_split_kernel<HD, 2, PROBS, LONG, RING><<<grid, dim3(64), 0, stream>>>(a);
    else
        decode_split_kernel<HD, 4, PROBS, LONG, RING><<<grid, dim3(64), 0, stream>>>(a);
}

template <int HD, bool RING>
static void launch_split_any(const DecodeArgs& a, hipStream_t stream) {
    if (!a.probs)
        launch_split<HD, false, false, RING>(a, stream);
    else if (a.split_len <= decode_part_limit(a.group, true))
        launch_split<HD, true, false, RING>(a, stream);
    else
        launch_split<HD, true, true, RING>(a, stream);
}

template <int HD>
static void launch_decode_hd(const DecodeArgs& a, hipStream_t stream) {
    if (a.ring)
        launch_split_any<HD, true>(a, stream);
    else
        launch_split_any<HD, false>(a, stream);
    decode_combine_kernel<HD><<<dim3((unsigned)(a.n_seq * a.n_q * a.n_heads)), dim3(256), 0, stream>>>(a);
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
