// Causal grouped-query attention of a prefill chunk over the head-major KV
// cache, bf16 inputs on the gfx950 matrix cores, float32 accumulation.
//
// What is computed (cortiq-engine 0.5.39 src/attention.rs, fn attention_head
// and the batched causal attend of fn qwen_attention_batch; needle-core 0.3.1
// src/v2/batch.rs module docs): for row i of sequence b at position
// p = start[b] + i and query head h of KV group g = h / G,
//   out = softmax_j(scale * q . K[g][j]) V[g][j],  j = 0..p,
// with the softmax's maximum subtracted.
//
// How (gfx950 design, not the pages'):
//  * GQA packing: the G query heads of one KV group read the same keys, so a
//    workgroup takes 128 "rows" = (position, head) pairs of one group, ordered
//    position-major, and streams that group's K/V once for all of them.
//  * The score tile is computed transposed, S^T = K Q^T, with
//    v_mfma_f32_32x32x16_bf16: the A operand is a 32-key slab of K from LDS,
//    the B operand is the lane's own query row held in registers.  In the
//    32x32 result each lane owns one query row (column) and 16 keys, so the
//    row max needs one exchange between the two wave halves and every other
//    softmax step is lane-local.
//  * O^T = V^T P^T reuses the score registers directly as the B operand (the
//    key order inside each 16-key step is the same permutation on both
//    operands); V is written transposed into LDS so the A operand is two
//    8-byte reads.
//  * Online softmax in registers (exp2 with the scale folded in), the
//    rescale of O skipped when no row's maximum moved, probabilities rounded
//    to bf16 for the matrix product and the row sum taken from the rounded
//    values so the weights stay a convex combination.
//  * K/V tiles of 64 keys are double-buffered in LDS, the next tile's global
//    loads are in flight while the current one is multiplied; tiles entirely
//    above a wave's causal limit are skipped, and only tiles that cross the
//    diagonal are masked.
//  * Split-KV: when the chunk has too few row tiles to fill 256 CUs, the key
//    range is split and the parts are merged by a log-sum-exp combine.
//  * blockIdx -> (group, split, row tile, sequence) with the group fastest,
//    so with 8 KV groups every XCD streams one group's K/V from its own L2.
#include "device_common.h"
#include "launch.h"

namespace attn {

constexpr int kTK = 64;                 // keys per tile
constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kPartPad = 4;             // (m, l, pad, pad) before O in a partial
// A row's running maximum (log2 units) is only moved, and O rescaled, when a
// new score exceeds it by more than this; until then probabilities are
// referenced to the old maximum and stay below 2^8.  The softmax is unchanged:
// numerator and row sum share the reference.
constexpr float kRescaleSlack = 8.f;

template <int HD>
struct PrefillSmem {
    static constexpr int KS = HD + 8;   // K row stride in bf16 (16 B pad)
    static constexpr int VS = kTK + 4;  // V^T row stride in bf16: 34 dwords,
                                        // 32 rows land on distinct bank pairs
    uint16_t k[2][kTK * KS];
    uint16_t vt[2][HD * VS];
};

__device__ __forceinline__ f32x16_t mfma32(bf16x8_t a, bf16x8_t b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Sum of the two bfloat16 halves of each packed word, exactly (products by 1).
__device__ __forceinline__ float sum_bf16_pairs(const uint32_t* pk, int n) {
    const bf16x2_t one = __builtin_bit_cast(bf16x2_t, 0x3f803f80u);
    float s0 = 0.f, s1 = 0.f;
#pragma unroll
    for (int q = 0; q < 16; q += 2) {
        s0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pk[q]), one, s0, false);
        s1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pk[q + 1]), one, s1, false);
    }
    return s0 + s1;
}

// QB: 32-row blocks of query rows per wave (1 or 2).  Each wave holds QB rows
// per lane; a K or V^T fragment read from LDS feeds QB matrix products.
template <int HD, int QB>
__global__ __launch_bounds__(kThreads, QB == 1 ? 2 : 1) void prefill_bf16_kernel(PrefillArgs a) {
    using Sm = PrefillSmem<HD>;
    constexpr int KS = Sm::KS;
    constexpr int VS = Sm::VS;
    constexpr int CH = HD / 8;                    // 16-byte chunks per cache row
    constexpr int KCH = kTK * CH / kThreads;      // K chunks per thread
    constexpr int VITEMS = (kTK / 4) * CH;        // (4-key, 8-dim) blocks of V
    constexpr int NDB = HD / 32;                  // 32-dim blocks of O
    constexpr int TILE_ROWS = kWaves * 32 * QB;   // query rows per workgroup
    __shared__ Sm sm;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int hf = lane >> 5;                     // wave half
    const int rl = lane & 31;

    int id = blockIdx.x;
    const int g = id % a.n_kv;
    id /= a.n_kv;
    const int s = id % a.n_splits;
    id /= a.n_splits;
    const int qt = a.n_qtiles - 1 - (id % a.n_qtiles);   // long rows first
    const int b = id / a.n_qtiles;
    if (b >= a.n_seq) return;

    const int G = a.group;
    const int t0 = a.cu_seq[b];
    const int len = min(a.cu_seq[b + 1] - t0, a.max_chunk);
    const int p0 = a.start[b];
    const int rows_b = len * G;
    const int r_tile0 = qt * TILE_ROWS;
    if (len <= 0 || p0 < 0 || r_tile0 >= rows_b) return;

    const int r_last = min(r_tile0 + TILE_ROWS, rows_b) - 1;
    const int n_keys = min(p0 + r_last / G + 1, a.cap);
    const int n_tiles = (n_keys + kTK - 1) / kTK;
    const int per = (n_tiles + a.n_splits - 1) / a.n_splits;
    const int tb = s * per;
    const int te = min(tb + per, n_tiles);

    // this wave's rows: blocks of 32, row = r_tile0 + wave*32*QB + qb*32 + rl
    const int rw0 = r_tile0 + wave * 32 * QB;
    const bool wave_ok = rw0 < rows_b;
    const int pw_lo = p0 + rw0 / G;
    const int pw_hi = p0 + min(rw0 + 32 * QB - 1, rows_b - 1) / G;
    int pos[QB], tq[QB], hq[QB];
    bool ok[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const int r = rw0 + qb * 32 + rl;
        const int i = r / G;
        tq[qb] = t0 + i;
        hq[qb] = g * G + (r - i * G);
        ok[qb] = r < rows_b && tq[qb] >= 0 && tq[qb] < a.n_tok;
        pos[qb] = ok[qb] ? p0 + i : -1;
    }

    bf16x8_t qf[QB][HD / 16];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const uint16_t* qrow =
            reinterpret_cast<const uint16_t*>(a.q) + ((size_t)tq[qb] * a.n_heads + hq[qb]) * HD;
#pragma unroll
        for (int k = 0; k < HD / 16; ++k) {
            uint4 u = make_uint4(0, 0, 0, 0);
            if (ok[qb]) u = *reinterpret_cast<const uint4*>(qrow + 16 * k + 8 * hf);
            qf[qb][k] = __builtin_bit_cast(bf16x8_t, u);
        }
    }

    const size_t kvbase = ((size_t)b * a.n_kv + g) * (size_t)a.cap * HD;
    const uint16_t* kc = reinterpret_cast<const uint16_t*>(a.k_cache) + kvbase;
    const uint16_t* vc = reinterpret_cast<const uint16_t*>(a.v_cache) + kvbase;

    // V^T staging: thread -> (4-key group kq, 8-dim chunk ch), kq fastest so a
    // wave's transposed 8-byte stores spread over the LDS banks
    const int v_kq = tid % (kTK / 4);
    const int v_ch = tid / (kTK / 4);
    uint4 kreg[KCH];
    uint32_t vreg[4][4];
    auto load_tile = [&](int j) {
        const int k0 = j * kTK;
#pragma unroll
        for (int c = 0; c < KCH; ++c) {
            const int idx = c * kThreads + tid;
            const int key = k0 + idx / CH;
            const int ch = idx % CH;
            kreg[c] = key < n_keys ? *reinterpret_cast<const uint4*>(kc + (size_t)key * HD + ch * 8)
                                   : make_uint4(0, 0, 0, 0);
        }
        if (tid < VITEMS) {
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int key = k0 + 4 * v_kq + jj;
                uint4 u = key < n_keys
                              ? *reinterpret_cast<const uint4*>(vc + (size_t)key * HD + v_ch * 8)
                              : make_uint4(0, 0, 0, 0);
                vreg[jj][0] = u.x;
                vreg[jj][1] = u.y;
                vreg[jj][2] = u.z;
                vreg[jj][3] = u.w;
            }
        }
    };
    auto store_tile = [&](int buf) {
#pragma unroll
        for (int c = 0; c < KCH; ++c) {
            const int idx = c * kThreads + tid;
            const int kr = idx / CH;
            const int ch = idx % CH;
            *reinterpret_cast<uint4*>(&sm.k[buf][kr * KS + ch * 8]) = kreg[c];
        }
        if (tid < VITEMS) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int w = e >> 1;
                uint32_t lo, hi;
                if ((e & 1) == 0) {
                    lo = (vreg[0][w] & 0xffffu) | (vreg[1][w] << 16);
                    hi = (vreg[2][w] & 0xffffu) | (vreg[3][w] << 16);
                } else {
                    lo = (vreg[0][w] >> 16) | (vreg[1][w] & 0xffff0000u);
                    hi = (vreg[2][w] >> 16) | (vreg[3][w] & 0xffff0000u);
                }
                *reinterpret_cast<uint2*>(&sm.vt[buf][(v_ch * 8 + e) * VS + 4 * v_kq]) =
                    make_uint2(lo, hi);
            }
        }
    };

    f32x16_t O[QB][NDB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int q = 0; q < 16; ++q) O[qb][db][q] = 0.f;
    float m_run[QB], l_run[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        m_run[qb] = -INFINITY;
        l_run[qb] = 0.f;
    }
    const float sl = a.scale * kLog2e;

    if (tb < te) {
        load_tile(tb);
        store_tile(0);
        __syncthreads();
        for (int j = tb; j < te; ++j) {
            const int buf = (j - tb) & 1;
            if (j + 1 < te) load_tile(j + 1);
            const int k0 = j * kTK;
            if (wave_ok && k0 <= pw_hi) {
                // ---- S^T = K Q^T: 64 keys x the lane's QB rows
                const uint16_t* kl = sm.k[buf];
                f32x16_t S[QB][2];
#pragma unroll
                for (int qb = 0; qb < QB; ++qb)
#pragma unroll
                    for (int q = 0; q < 16; ++q) {
                        S[qb][0][q] = 0.f;
                        S[qb][1][q] = 0.f;
                    }
#pragma unroll
                for (int kk = 0; kk < HD / 16; ++kk) {
                    const bf16x8_t a0 = __builtin_bit_cast(
                        bf16x8_t, *reinterpret_cast<const uint4*>(kl + rl * KS + kk * 16 + hf * 8));
                    const bf16x8_t a1 = __builtin_bit_cast(
                        bf16x8_t,
                        *reinterpret_cast<const uint4*>(kl + (32 + rl) * KS + kk * 16 + hf * 8));
#pragma unroll
                    for (int qb = 0; qb < QB; ++qb) {
                        S[qb][0] = mfma32(a0, qf[qb][kk], S[qb][0]);
                        S[qb][1] = mfma32(a1, qf[qb][kk], S[qb][1]);
                    }
                }
                // ---- causal mask (diagonal tiles only), online softmax
                const bool need_mask = k0 + kTK - 1 > pw_lo;
                uint32_t pk[QB][16];
#pragma unroll
                for (int qb = 0; qb < QB; ++qb) {
                    if (need_mask) {
#pragma unroll
                        for (int q = 0; q < 16; ++q) {
                            const int key = k0 + 8 * (q >> 2) + 4 * hf + (q & 3);
                            if (key > pos[qb]) S[qb][0][q] = -INFINITY;
                            if (key + 32 > pos[qb]) S[qb][1][q] = -INFINITY;
                        }
                    }
                    float mx = S[qb][0][0];
#pragma unroll
                    for (int q = 1; q < 16; ++q) mx = fmaxf(mx, S[qb][0][q]);
#pragma unroll
                    for (int q = 0; q < 16; ++q) mx = fmaxf(mx, S[qb][1][q]);
                    mx = fmaxf(mx, __shfl_xor(mx, 32));
                    const float mt = mx * sl;             // log2 units; -inf stays
                    const bool grow = mt > m_run[qb] + kRescaleSlack;
                    const float m_new = grow ? mt : m_run[qb];
                    const float m_use = m_new == -INFINITY ? 0.f : m_new;
                    if (__any(grow)) {
                        const float alpha = grow ? __builtin_amdgcn_exp2f(m_run[qb] - m_use) : 1.f;
                        l_run[qb] *= alpha;
#pragma unroll
                        for (int db = 0; db < NDB; ++db)
#pragma unroll
                            for (int q = 0; q < 16; ++q) O[qb][db][q] *= alpha;
                    }
                    m_run[qb] = m_new;
                    const float nm = -m_use;
#pragma unroll
                    for (int q = 0; q < 8; ++q) {
                        pk[qb][q] = pack_bf16x2(
                            __builtin_amdgcn_exp2f(__builtin_fmaf(S[qb][0][2 * q], sl, nm)),
                            __builtin_amdgcn_exp2f(__builtin_fmaf(S[qb][0][2 * q + 1], sl, nm)));
                        pk[qb][8 + q] = pack_bf16x2(
                            __builtin_amdgcn_exp2f(__builtin_fmaf(S[qb][1][2 * q], sl, nm)),
                            __builtin_amdgcn_exp2f(__builtin_fmaf(S[qb][1][2 * q + 1], sl, nm)));
                    }
                    // the row sum is taken from the rounded probabilities that
                    // feed the P.V product
                    l_run[qb] += sum_bf16_pairs(pk[qb], 16);
                }
                // ---- O^T += V^T P^T
                const uint16_t* vl = sm.vt[buf];
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
                    for (int tt = 0; tt < 2; ++tt) {
                        const int pq = kb * 8 + tt * 4;
                        bf16x8_t pb[QB];
#pragma unroll
                        for (int qb = 0; qb < QB; ++qb)
                            pb[qb] = __builtin_bit_cast(
                                bf16x8_t, make_uint4(pk[qb][pq], pk[qb][pq + 1], pk[qb][pq + 2],
                                                     pk[qb][pq + 3]));
#pragma unroll
                        for (int db = 0; db < NDB; ++db) {
                            const uint16_t* vp = vl + (db * 32 + rl) * VS + kb * 32 + tt * 16 + hf * 4;
                            const uint2 lo = *reinterpret_cast<const uint2*>(vp);
                            const uint2 hi = *reinterpret_cast<const uint2*>(vp + 8);
                            const bf16x8_t av =
                                __builtin_bit_cast(bf16x8_t, make_uint4(lo.x, lo.y, hi.x, hi.y));
#pragma unroll
                            for (int qb = 0; qb < QB; ++qb) O[qb][db] = mfma32(av, pb[qb], O[qb][db]);
                        }
                    }
                }
            }
            if (j + 1 < te) store_tile(buf ^ 1);
            __syncthreads();
        }
    }

#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const float l_tot = l_run[qb] + __shfl_xor(l_run[qb], 32);
        if (!ok[qb]) continue;
        if (a.n_splits == 1) {
            const float inv = 1.f / l_tot;
            float* orow = a.out + ((size_t)tq[qb] * a.n_heads + hq[qb]) * HD;
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) {
                    float4 v = make_float4(O[qb][db][4 * q4] * inv, O[qb][db][4 * q4 + 1] * inv,
                                           O[qb][db][4 * q4 + 2] * inv, O[qb][db][4 * q4 + 3] * inv);
                    *reinterpret_cast<float4*>(orow + db * 32 + 8 * q4 + 4 * hf) = v;
                }
        } else {
            float* pr = a.part +
                        (((size_t)tq[qb] * a.n_heads + hq[qb]) * a.n_splits + s) * (HD + kPartPad);
            if (hf == 0) *reinterpret_cast<float2*>(pr) = make_float2(m_run[qb], l_tot);
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) {
                    float4 v = make_float4(O[qb][db][4 * q4], O[qb][db][4 * q4 + 1],
                                           O[qb][db][4 * q4 + 2], O[qb][db][4 * q4 + 3]);
                    *reinterpret_cast<float4*>(pr + kPartPad + db * 32 + 8 * q4 + 4 * hf) = v;
                }
        }
    }
}

// Merge split partials (m, l, O) of each row: m* = max m_s,
// l* = sum l_s 2^(m_s - m*), out = sum O_s 2^(m_s - m*) / l*.
template <int HD>
__global__ __launch_bounds__(256) void prefill_combine_kernel(PrefillArgs a) {
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (row >= a.n_tok * a.n_heads) return;
    const int S = a.n_splits;
    const float* pr = a.part + (size_t)row * S * (HD + kPartPad);
    float m = -INFINITY;
    for (int s = 0; s < S; ++s) m = fmaxf(m, pr[(size_t)s * (HD + kPartPad)]);
    const float m_use = m == -INFINITY ? 0.f : m;
    float l = 0.f;
    constexpr int PER = HD / 64;
    float o[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e) o[e] = 0.f;
    for (int s = 0; s < S; ++s) {
        const float* p = pr + (size_t)s * (HD + kPartPad);
        const float w = __builtin_amdgcn_exp2f(p[0] - m_use);
        l += p[1] * w;
#pragma unroll
        for (int e = 0; e < PER; ++e) o[e] += p[kPartPad + lane + 64 * e] * w;
    }
    const float inv = l > 0.f ? 1.f / l : 0.f;
    float* orow = a.out + (size_t)row * HD;
#pragma unroll
    for (int e = 0; e < PER; ++e) orow[lane + 64 * e] = o[e] * inv;
}


// Variant and split choice.  Large chunks (enough 256-row tiles to give every
// CU a workgroup) take 64 rows per wave; otherwise 128-row tiles, with the key
// range split so that about two workgroups per CU are in flight, each part
// keeping at least kMinTilesPerSplit key tiles.
constexpr int kTargetBlocks = 512;
constexpr int kMinTilesPerSplit = 4;
constexpr int kMaxSplits = 32;

PrefillPlan plan_prefill(int n_seq, int n_heads, int n_kv, int head_dim, int n_tok, int max_chunk,
                         int max_end, size_t ws_available) {
    PrefillPlan p{kWaves * 32, 1, 1, 0};
    const long group = n_heads / n_kv;
    const long rows = (long)max_chunk * group;
    const long big_tiles = (rows + kWaves * 64 - 1) / (kWaves * 64);
    if ((long)n_seq * big_tiles * n_kv >= 384) {
        p.rows_per_tile = kWaves * 64;
        p.n_qtiles = (int)big_tiles;
        return p;
    }
    p.n_qtiles = (int)((rows + kWaves * 32 - 1) / (kWaves * 32));
    const long base = (long)n_seq * p.n_qtiles * n_kv;
    const long tiles = ((long)max_end + kTK - 1) / kTK;
    long sp = base > 0 ? (kTargetBlocks + base - 1) / base : 1;
    long by_len = tiles / kMinTilesPerSplit;
    if (by_len < 1) by_len = 1;
    if (sp > by_len) sp = by_len;
    if (sp > kMaxSplits) sp = kMaxSplits;
    if (sp < 1) sp = 1;
    const size_t per = (size_t)n_tok * n_heads * (head_dim + kPartPad) * sizeof(float);
    if (sp > 1 && per > 0) {
        const size_t fit = ws_available / per;
        if ((size_t)sp > fit) sp = (long)fit;
        if (sp < 1) sp = 1;
    }
    p.n_splits = (int)sp;
    p.ws_bytes = sp > 1 ? per * (size_t)sp : 0;
    return p;
}

hipError_t launch_prefill_bf16(const PrefillArgs& a, hipStream_t stream) {
    const long blocks = (long)a.n_seq * a.n_qtiles * a.n_splits * a.n_kv;
    if (blocks <= 0) return hipSuccess;
    const dim3 grid((unsigned)blocks), block(kThreads);
    if (a.rows_per_tile == kWaves * 64) {
        if (a.head_dim == 128) prefill_bf16_kernel<128, 2><<<grid, block, 0, stream>>>(a);
        else prefill_bf16_kernel<64, 2><<<grid, block, 0, stream>>>(a);
    } else {
        if (a.head_dim == 128) prefill_bf16_kernel<128, 1><<<grid, block, 0, stream>>>(a);
        else prefill_bf16_kernel<64, 1><<<grid, block, 0, stream>>>(a);
    }
    return hipGetLastError();
}

hipError_t launch_prefill_combine(const PrefillArgs& a, hipStream_t stream) {
    const long rows = (long)a.n_tok * a.n_heads;
    const long blocks = (rows + 3) / 4;
    if (blocks <= 0) return hipSuccess;
    if (a.head_dim == 128)
        prefill_combine_kernel<128><<<dim3((unsigned)blocks), dim3(256), 0, stream>>>(a);
    else
        prefill_combine_kernel<64><<<dim3((unsigned)blocks), dim3(256), 0, stream>>>(a);
    return hipGetLastError();
}

}  // namespace attn
