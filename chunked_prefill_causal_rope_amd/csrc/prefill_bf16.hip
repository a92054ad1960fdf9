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
//    workgroup takes 256 (large calls) or 128 (small calls) "rows" =
//    (position, head) pairs of one group, ordered position-major, and
//    streams that group's K/V once for all of them.
//  * The score tile is computed transposed, S^T = K Q^T, with
//    v_mfma_f32_32x32x16_bf16: the A operand is a 32-key slab of K from LDS,
//    the B operand is the lane's own query row held in registers.  In the
//    32x32 result each lane owns one query row (column) and 16 keys, so the
//    row max needs one exchange between the two wave halves and every other
//    softmax step is lane-local.
//  * O^T = V^T P^T reuses the score registers directly as the B operand (the
//    key order inside each 16-key step is the same permutation on both
//    operands); V stays in its natural layout in LDS and the A operand is
//    read with the transposing LDS read.
//  * Online softmax in registers (exp2 with the scale folded in), the
//    rescale of O skipped unless a row's maximum grows by more than 2^8,
//    probabilities rounded to bf16 for the matrix product and the row sum
//    taken from the rounded values so the weights stay a convex combination.
//  * 256-row items (prefill_pp_kernel): two waves per SIMD alternate a
//    matrix phase and a softmax phase half a tile apart (ping-pong), so one
//    wave's products overlap the other's exponentials; K/V tiles of 64 keys
//    in three LDS slots.  128-row items (prefill_bf16_ks_kernel): two waves
//    share 32 rows and take the two key halves of every tile.  Tiles
//    entirely above a wave's causal limit are skipped; only tiles that cross
//    the diagonal are masked.
//  * Split-KV: when the chunk has too few row tiles to fill 256 CUs, the key
//    range is split and the parts are merged by a log-sum-exp combine: its
//    own kernel, or (chunk loops) workgroups of the next chunk's launch.
//  * Workgroups besides the attention items: the previous chunk's merge
//    (ahead of them) and the next chunk's RoPE + append (after them).
//  * blockIdx -> (group, split, row tile, sequence) with the group fastest,
//    so with 8 KV groups every XCD streams one group's K/V from its own L2.
#include <algorithm>
#include <climits>
#include <type_traits>

#include "device_common.h"
#include "launch.h"
#include "rope_token.h"

namespace attn {

constexpr int kTK = 64;                 // keys per tile
// A split partial row: (m, l, e, 0) as floats, then O/l * 2^-e as head_dim
// halves (see part_scale_exp).
constexpr int kPartHead = 4;
__host__ __device__ constexpr int part_row_words(int hd) { return kPartHead + hd / 2; }
// A row's running maximum (log2 units) is only moved, and O rescaled, when a
// new score exceeds it by more than this; until then probabilities are
// referenced to the old maximum and stay below 2^8.  The softmax is unchanged:
// numerator and row sum share the reference.
constexpr float kRescaleSlack = 8.f;

template <int HD>
struct alignas(16) PrefillSmem {
    // K rows padded by 16 B: the 32 rows of an A-operand read start on
    // distinct 4-bank groups.  V rows padded by 64 B: the 8 rows of a
    // transposing read (4 keys per 16-lane group, two groups per half-wave)
    // start 16 banks apart.
    static constexpr int KS = HD + 8;
    static constexpr int VS = HD + 32;
    uint16_t k[2][kTK * KS];
    uint16_t v[2][kTK * VS];
};

// Calls f(std::integral_constant<int, i>) for i = I .. N-1, so the body can
// use i in constant expressions (scheduling-group sizes, register indices).
template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (I < N) {
        f(std::integral_constant<int, I>{});
        static_for<I + 1, N>(f);
    }
}

__device__ __forceinline__ f32x16_t mfma32(bf16x8_t a, bf16x8_t b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;

// LDS transposing read: within each 16-lane group, lane j receives element j
// (then j+16, j+32, j+48) of the 64 16-bit values the group's lanes point at,
// 4 per lane in lane order.  Pointing lane a at V[k0 + a/4][d0 + 4(a%4)]
// therefore hands lane j the column V[k0 .. k0+3][d0 + j].
__device__ __forceinline__ u32x2_t lds_read_tr16(const uint16_t* p) {
    const s16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(p));
    return __builtin_bit_cast(u32x2_t, v);
}

// Sum of the two bfloat16 halves of each packed word, exactly (products by 1).
__device__ __forceinline__ float sum_bf16_pairs(const uint32_t* pk) {
    const bf16x2_t one = __builtin_bit_cast(bf16x2_t, 0x3f803f80u);
    float s0 = 0.f, s1 = 0.f;
#pragma unroll
    for (int q = 0; q < 16; q += 2) {
        s0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pk[q]), one, s0, false);
        s1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pk[q + 1]), one, s1, false);
    }
    return s0 + s1;
}

// Scheduling hints for the interleaved sections: each matrix product is
// followed by a few vector-ALU instructions of the independent softmax stream.
#define ATTN_INTERLEAVE(n, mfma, valu)                               \
    do {                                                             \
        _Pragma("unroll") for (int _i = 0; _i < (n); ++_i) {         \
            __builtin_amdgcn_sched_group_barrier(0x008, (mfma), 0);  \
            __builtin_amdgcn_sched_group_barrier(0x002, (valu), 0);  \
        }                                                            \
    } while (0)

// ---------------------------------------------------------------- schedule
// A work item is (sequence b, row tile qt, KV group g, part) and covers one
// part of the row tile's key tiles; workgroup i takes item i.  Without
// splitting there is one part per row tile.  With splitting (few row tiles)
// every workgroup derives the same schedule from cu_seq/start: a row tile of
// n key tiles gets ceil(n / T) parts of equal length, T (at least
// min_tiles_per_split) minimising the estimated duration
// ceil(items / slots) * (T + 2), so the longest sequence is spread over the
// CUs instead of deciding the call's duration alone.  The grid has room for
// the largest item count the schedule can produce; the workgroups past the
// actual count exit.
// Shortest part, in key tiles: a part's start-up (Q and first K/V tiles,
// partial write, its share of the combine) weighs more for the 256-row
// workgroups than for the 128-row key-split ones (measured: c3-shaped calls
// gain ~2 % from 12 over 4 at 256 rows; c1-shaped calls gain ~3 % from 4
// over 6 at 128 rows, 2 and 3 are no better).
#ifndef ATTN_PREFILL_MIN_TILES_128
#define ATTN_PREFILL_MIN_TILES_128 4
#endif
#ifndef ATTN_PREFILL_MIN_TILES_256
#define ATTN_PREFILL_MIN_TILES_256 12
#endif
__host__ __device__ constexpr int min_tiles_per_split(int rows_per_tile) {
    return rows_per_tile == 256 ? ATTN_PREFILL_MIN_TILES_256 : ATTN_PREFILL_MIN_TILES_128;
}
// An item's fixed cost (schedule, Q and first tiles, merge and partial
// write), in key tiles, in the duration estimate: the 128-row key-split
// items merge their halves and run each tile in about half the time.
#ifndef ATTN_PREFILL_ITEM_COST_128
#define ATTN_PREFILL_ITEM_COST_128 4
#endif
#ifndef ATTN_PREFILL_ITEM_COST_256
#define ATTN_PREFILL_ITEM_COST_256 2
#endif
__host__ __device__ constexpr int item_cost_tiles(int rows_per_tile) {
    return rows_per_tile == 256 ? ATTN_PREFILL_ITEM_COST_256 : ATTN_PREFILL_ITEM_COST_128;
}

// First key tile a row tile reads: with a sliding window of W keys its
// first row (position p_first) starts at key p_first - W + 1, and every later
// row of the tile starts at or after it.
__host__ __device__ constexpr int first_key_tile(int p_first, int window) {
    return window > 0 && p_first >= window ? (p_first - window + 1) / kTK : 0;
}

// key tiles of row tile qt of sequence b (0 if the row tile is empty)
__device__ __forceinline__ int group_tiles(const PrefillArgs& a, int b, int qt) {
    const int t0 = a.cu_seq[b];
    const int len = min(a.cu_seq[b + 1] - t0, a.max_chunk);
    const int p0 = a.start[b];
    const int rows_b = len * a.group;
    const int r0 = qt * a.rows_per_tile;
    if (len <= 0 || p0 < 0 || r0 >= rows_b) return 0;
    const int r_last = min(r0 + a.rows_per_tile, rows_b) - 1;
    const int n_keys = a.ring ? p0 + r_last / a.group + 1 : min(p0 + r_last / a.group + 1, a.cap);
    const int n_tiles = (n_keys + kTK - 1) / kTK;
    return n_tiles - min(first_key_tile(p0 + r0 / a.group, a.window), n_tiles);
}

struct PrefillItem {
    int b, qt, g, part, nsp;
};

// Schedule of a split call, computed by every wave alike: lane l holds row
// tile group l = (b, qt) (at most 64 groups).  The part length T minimises
// the estimated duration ceil(items / slots) * (T + 2) (2 tiles for an
// item's start-up) over T = ceil(longest / k) -- on the host when the call
// has one sequence, whose sizes it knows; then item -> group by a prefix
// sum over the groups' item counts.  Lane 0 of workgroup 0 also
// writes, per group, its first item and part count for the combine kernel.
// Wave-wide sum and max of an int: DPP within each 16-lane row, then the
// four row results (no LDS round trips).
template <bool MAX>
__device__ __forceinline__ int wave_reduce_dpp(int x) {
    auto op = [](int u, int v) { return MAX ? max(u, v) : u + v; };
    x = op(x, __builtin_amdgcn_update_dpp(x, x, 0xB1, 0xF, 0xF, false));    // quad_perm 1,0,3,2
    x = op(x, __builtin_amdgcn_update_dpp(x, x, 0x4E, 0xF, 0xF, false));    // quad_perm 2,3,0,1
    x = op(x, __builtin_amdgcn_update_dpp(x, x, 0x141, 0xF, 0xF, false));   // row_half_mirror
    x = op(x, __builtin_amdgcn_update_dpp(x, x, 0x140, 0xF, 0xF, false));   // row_mirror
    return op(op(__builtin_amdgcn_readlane(x, 0), __builtin_amdgcn_readlane(x, 16)),
              op(__builtin_amdgcn_readlane(x, 32), __builtin_amdgcn_readlane(x, 48)));
}

// Part length for the groups' key tiles gt (one per lane): minimise the
// estimated duration ceil(items / slots) * (T + 2) over T = ceil(longest / k).
__device__ __forceinline__ int split_part_length(const PrefillArgs& a, int gt) {
    const int gmax = max(wave_reduce_dpp<true>(gt), 1);
    const long slots = a.slots;
    int best_T = gmax;
    long best_cost = -1;
    int prev_T = 0;
    constexpr int kCand[12] = {1, 2, 3, 4, 6, 8, 12, 16, 24, 32, 48, 64};
    for (int ci = 0; ci < 12; ++ci) {
        const int k = kCand[ci];
        const int T = (gmax + k - 1) / k;
        if (T < min_tiles_per_split(a.rows_per_tile) && k > 1) break;
        if (T == prev_T) continue;
        prev_T = T;
        const int n = wave_reduce_dpp<false>(gt > 0 ? (gt + T - 1) / T : 0) * a.n_kv;
        if (n > a.grid) continue;             // one workgroup per item
        const long cost = (long)((n + slots - 1) / slots) * (T + item_cost_tiles(a.rows_per_tile));
        if (best_cost < 0 || cost < best_cost) {
            best_cost = cost;
            best_T = T;
        }
    }
    return best_T;
}

__device__ PrefillItem split_schedule(const PrefillArgs& a, int item) {
    const int lane = threadIdx.x & 63;
    const int n_groups = a.n_seq * a.n_qtiles;
    const int gt = lane < n_groups ? group_tiles(a, lane / a.n_qtiles, lane % a.n_qtiles) : 0;
    // a single sequence's lengths are host scalars: its part length comes
    // with the launch (checked against the grid, in case the arrays and the
    // host scalars disagree)
    int T = a.part_tiles;
    if (T <= 0 || wave_reduce_dpp<false>(gt > 0 ? (gt + T - 1) / T : 0) * a.n_kv > a.grid)
        T = split_part_length(a, gt);
    const int nsp = gt > 0 ? (gt + T - 1) / T : 0;
    const int cnt = nsp * a.n_kv;
    // exclusive prefix sum of the groups' item counts
    int incl = cnt;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int v = __shfl_up(incl, o);
        if (lane >= o) incl += v;
    }
    const int excl = incl - cnt;
    if (item == 0 && threadIdx.x < 64 && lane < n_groups) {
        a.table[2 * lane] = excl;
        a.table[2 * lane + 1] = nsp;
    }
    const unsigned long long hit = __ballot(cnt > 0 && item >= excl && item < incl);
    if (hit == 0ull) return PrefillItem{0, 0, 0, 0, 0};
    const int src = __builtin_ctzll(hit);
    const int local = item - __shfl(excl, src);
    return PrefillItem{src / a.n_qtiles, src % a.n_qtiles, local % a.n_kv, local / a.n_kv, __shfl(nsp, src)};
}

// Output of one lane's half of a query row (dims db*32 + 8*q4 + 4*hf + 0..3
// of O[db]), after the last key tile: an unsplit row is normalised by its
// row sum l_tot, gated when asked, and stored as float32; a split part leaves
// (m, l) and O/l in half precision (scaled by 2^-e when needed) for the
// combine.  Both wave halves of the row call this.
template <int HD>
__device__ __forceinline__ void write_row(const PrefillArgs& a, f32x16_t (&O)[HD / 32], float m_run, float l_tot,
                                          int t, int h, int hf, int nsp, float* part_row) {
    constexpr int NDB = HD / 32;
    if (nsp <= 1) {
        const float inv = 1.f / l_tot;
        float* orow = a.out + ((size_t)t * a.n_heads + h) * HD;
        if (a.gate.mode) {
            // output gate: all loads issued before any factor is formed
            const size_t grow = (size_t)t * a.n_heads + h;
            const uint16_t* gp = reinterpret_cast<const uint16_t*>(a.gate.p) + grow * (size_t)a.gate.ld;
            if (a.gate.mode == kGateSoftplusHead) {
                const float f = gate_fast(a.gate.mode, bf16_to_f32(gp[0])) * inv;
#pragma unroll
                for (int db = 0; db < NDB; ++db)
#pragma unroll
                    for (int q = 0; q < 16; ++q) O[db][q] *= f;
            } else {
                u32x2_t graw[NDB][4];
                const bool vec = ((a.gate.ld & 3) == 0) && ((reinterpret_cast<uintptr_t>(a.gate.p) & 7) == 0);
#pragma unroll
                for (int db = 0; db < NDB; ++db)
#pragma unroll
                    for (int q4 = 0; q4 < 4; ++q4) {
                        const uint16_t* p = gp + db * 32 + 8 * q4 + 4 * hf;
                        if (vec) {
                            graw[db][q4] = *reinterpret_cast<const u32x2_t*>(p);
                        } else {
                            graw[db][q4] = u32x2_t{(uint32_t)p[0] | ((uint32_t)p[1] << 16),
                                                   (uint32_t)p[2] | ((uint32_t)p[3] << 16)};
                        }
                    }
#pragma unroll
                for (int db = 0; db < NDB; ++db)
#pragma unroll
                    for (int q4 = 0; q4 < 4; ++q4) {
                        O[db][4 * q4] *= gate_fast(a.gate.mode, bf16_lo(graw[db][q4].x)) * inv;
                        O[db][4 * q4 + 1] *= gate_fast(a.gate.mode, bf16_hi(graw[db][q4].x)) * inv;
                        O[db][4 * q4 + 2] *= gate_fast(a.gate.mode, bf16_lo(graw[db][q4].y)) * inv;
                        O[db][4 * q4 + 3] *= gate_fast(a.gate.mode, bf16_hi(graw[db][q4].y)) * inv;
                    }
            }
        } else {
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int q = 0; q < 16; ++q) O[db][q] *= inv;
        }
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const float4 v = make_float4(O[db][4 * q4], O[db][4 * q4 + 1], O[db][4 * q4 + 2],
                                             O[db][4 * q4 + 3]);
                *reinterpret_cast<float4*>(orow + db * 32 + 8 * q4 + 4 * hf) = v;
            }
    } else {
        // partial of the row: O/l in half precision (a part whose keys are
        // all masked for the row has l = 0, O = 0)
        const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
        float mx = 0.f;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int q = 0; q < 16; ++q) mx = fmaxf(mx, fabsf(O[db][q]));
        mx = fmaxf(mx, __shfl_xor(mx, 32)) * inv;
        const int ex = part_scale_exp(mx);
        const float sc = __builtin_amdgcn_ldexpf(inv, -ex);
        if (hf == 0) *reinterpret_cast<float4*>(part_row) = make_float4(m_run, l_tot, (float)ex, 0.f);
        uint32_t* ph = reinterpret_cast<uint32_t*>(part_row + kPartHead);
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const u32x2_t v = {pack_f16x2(O[db][4 * q4] * sc, O[db][4 * q4 + 1] * sc),
                                   pack_f16x2(O[db][4 * q4 + 2] * sc, O[db][4 * q4 + 3] * sc)};
                *reinterpret_cast<u32x2_t*>(ph + (db * 32 + 8 * q4 + 4 * hf) / 2) = v;
            }
    }
}

// Ping-pong kernel for 256-row work items: 8 waves of 32 query rows, two
// per SIMD (waves w and w+4).  Each wave alternates a matrix phase (the
// scores of key tile k on the matrix cores, S^T = K Q^T, together with the
// P.V product of tile k-1) and a softmax phase (mask, row maximum, the rare
// rescale of O, exponentials, row sums of tile k, plus its share of the K/V
// staging).  Waves 4..7 run one phase behind waves 0..3, with a workgroup
// barrier between phases, so on every SIMD one wave's matrix products run
// while the other wave's exponentials and bookkeeping use the vector ALU.
// Three LDS slots per K and V tile give the half-tile offset room: tile j
// sits in slot (j - tb) mod 3, is written during the softmax phases of the
// tile two (K) or one (V) before it, and is overwritten only after both
// wave groups have left the phase that reads it.
template <int HD>
struct alignas(16) PingPongSmem {
    static constexpr int KS = HD + 8;
    static constexpr int VS = HD + 32;
    uint16_t k[3][kTK * KS];
    uint16_t v[3][kTK * VS];
};

#ifndef ATTN_PP_PRIO
#define ATTN_PP_PRIO 1
#endif
// fragment reads in flight ahead of the matrix products (in product steps)
#ifndef ATTN_PP_PREFETCH
#define ATTN_PP_PREFETCH 3
#endif
// staging register sets: one holds the global loads of the next tile's
// share; a second (loads issued two softmax phases ahead) does not fit the
// register budget of two waves per SIMD at a head dimension of 128 and spills
#ifndef ATTN_PP_STAGE_DEPTH
#define ATTN_PP_STAGE_DEPTH 1
#endif
// the staging share is written to LDS after the probabilities, not among them
#ifndef ATTN_PP_LATE_STORE
#define ATTN_PP_LATE_STORE 1
#endif
// the row maximum's exchange between wave halves: v_permlane32_swap (vector
// ALU) rather than an LDS permute, which waits behind the other group's
// fragment reads
#ifndef ATTN_PP_PERMLANE
#define ATTN_PP_PERMLANE 1
#endif
// K/V staging by LDS-DMA loads (head dimension 128): each wave load moves 64
// keys' 16-byte chunk c of a tile straight into LDS, with no staging
// registers, so a tile's loads can be issued two tiles ahead into four LDS
// slots.  A tile is laid out as chunk columns: column c (byte c * kDmaCol)
// holds chunk c of keys 0..63 at 16 bytes per key.  The 64-byte pad per
// column puts the 16 keys of a score-fragment read and the four columns of a
// transposing read on distinct banks.
#ifndef ATTN_PP_DMA
#define ATTN_PP_DMA 1
#endif
// where a softmax phase's tile loads are issued: 1 at its start (measured
// on c4 +4 % over 0, the end of the phase; issuing them at the start of the
// matrix phase before it, one tile further ahead, was slower than either)
#ifndef ATTN_PP_DMA_AT
#define ATTN_PP_DMA_AT 1
#endif
constexpr int kDmaCol = kTK * 16 + 64;
template <int HD>
struct alignas(16) PingPongDmaSmem {
    static constexpr int KS = 0;                  // unused: column layout
    static constexpr int VS = 0;
    static constexpr int kTile = HD / 8 * kDmaCol;
    uint8_t k[4][kTile];
    uint8_t v[4][kTile];
};
// LDS byte address of a shared-memory location (wave-uniform)
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return __builtin_amdgcn_readfirstlane(
        (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p);
}
// One wave load of 16 bytes per lane into LDS at m0 + 16 * lane, from the
// buffer rsrc at byte voff; the compiler sees no LDS write and no counter,
// so the caller waits (vmcnt) before the barrier that publishes the data.
// M0 is a register the compiler reserves and does not allocate; the
// assembly of these kernels uses it only in these loads, each setting it
// in the same asm statement, so it is not listed as a clobber.
__device__ __forceinline__ void dma16(uint32_t m0v, int voff, __amdgpu_buffer_rsrc_t rs) {
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :: "s"(m0v), "v"(voff), "s"(rs) : "memory");
}
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory");
}

// Workgroups past the attention grid finish the next chunk's rows (RoPE and
// cache append), using the kernel's LDS for the token's tables.  The next
// chunk writes cache rows past every key this chunk reads, so the two are
// independent.
template <int HD>
__device__ __forceinline__ void merge_rows(const MergeArgs& a, int bx, int b, int tid);

template <int HD, typename Sm>
__device__ __forceinline__ void next_chunk_role(const PrefillArgs& a, Sm& sm, int r) {
    static_assert(sizeof(RopeTokSmem<HD>) <= sizeof(Sm), "token tables fit the attention LDS");
    const int i = r % a.next_chunk;
    const int hb = (r / a.next_chunk) % a.next_nhb;
    const int b = r / (a.next_chunk * a.next_nhb);
    rope_token_body<uint16_t, HD, 512>(a.next, i, hb, b, reinterpret_cast<RopeTokSmem<HD>&>(sm));
}

// An earlier split chunk's merge, workgroup r of prev_blocks: two merge
// blocks of 256 threads each (threads 0-255 and 256-511).  The merge reads
// partials and writes output rows that this launch's attention does not
// touch.
template <int HD>
__device__ __forceinline__ void prev_merge_role(const PrefillArgs& a, int r) {
    if (a.prev_gx <= 0) return;
    const int f = 2 * r + (int)(threadIdx.x >> 8);
    const int by = f / a.prev_gx;
    if (by < a.prev.n_seq) merge_rows<HD>(a.prev, f - by * a.prev_gx, by, threadIdx.x & 255);
}

// Workgroups besides the attention items.  The grid is [merge roles when
// ATTN_MERGE_FIRST] [next-chunk roles when ATTN_NEXT_FIRST] attention items
// [next-chunk roles] [merge roles]; wg is the workgroup's index past the
// leading roles.  Leading, the merge starts at once beside the first
// attention items instead of after the next-chunk roles (measured on
// 128-token chunks of 32 heads, 128 merge workgroups: 0.62 against 0.64 ms
// per step); the next-chunk roles, 256 workgroups there, are better last
// (0.61 against 0.65 ms leading).
#ifndef ATTN_MERGE_FIRST
#define ATTN_MERGE_FIRST 1
#endif
#ifndef ATTN_NEXT_FIRST
#define ATTN_NEXT_FIRST 0
#endif
__device__ __forceinline__ int attention_wg(const PrefillArgs& a) {
    return (int)blockIdx.x - (ATTN_MERGE_FIRST ? a.prev_blocks : 0) - (ATTN_NEXT_FIRST ? a.next_blocks : 0);
}
template <int HD, typename Sm>
__device__ __forceinline__ void extra_role(const PrefillArgs& a, Sm& sm, int wg) {
    if (wg < 0) {
        const int idx = (int)blockIdx.x - (ATTN_MERGE_FIRST ? a.prev_blocks : 0);
        if (idx < 0) prev_merge_role<HD>(a, (int)blockIdx.x);
        else next_chunk_role<HD>(a, sm, idx);
        return;
    }
    const int r = wg - a.grid;
    if (!ATTN_NEXT_FIRST && r < a.next_blocks) {
        next_chunk_role<HD>(a, sm, r);
        return;
    }
    prev_merge_role<HD>(a, r - (ATTN_NEXT_FIRST ? 0 : a.next_blocks));
}

template <int HD, bool WIN>
__global__ __launch_bounds__(512, 1) void prefill_pp_kernel(PrefillArgs a) {
    constexpr bool DMA = ATTN_PP_DMA && HD == 128;
    using Sm = std::conditional_t<DMA, PingPongDmaSmem<HD>, PingPongSmem<HD>>;
    constexpr int kThreads = 512;
    constexpr int KS = Sm::KS;
    constexpr int VS = Sm::VS;
    constexpr int CH = HD / 8;                    // 16-byte chunks per cache row
    constexpr int NCH = kTK * CH / kThreads;      // K (and V) chunks per thread
    constexpr int NDB = HD / 32;                  // 32-dim blocks of O
    constexpr int NKK = HD / 16;                  // K-steps of a score product
    constexpr int TILE_ROWS = 256;                // query rows per workgroup
    __shared__ Sm sm;
    const int wg = attention_wg(a);
    if (wg < 0 || wg >= a.grid) {
        extra_role<HD>(a, sm, wg);
        return;
    }

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int grp = __builtin_amdgcn_readfirstlane(wave >> 2);   // 0: leads, 1: one phase behind
    const int hf = lane >> 5;                     // wave half
    const int rl = lane & 31;

    const int item = wg;
    PrefillItem itm;
    if (a.split) {
        itm = split_schedule(a, item);
    } else {
        // KV group fastest, long row tiles first
        itm.g = item % a.n_kv;
        itm.qt = a.n_qtiles - 1 - (item / a.n_kv) % a.n_qtiles;
        itm.b = item / (a.n_kv * a.n_qtiles);
        itm.part = 0;
        itm.nsp = 1;
    }
    if (itm.nsp <= 0) return;
    const int b = __builtin_amdgcn_readfirstlane(itm.b), qt = __builtin_amdgcn_readfirstlane(itm.qt),
              g = __builtin_amdgcn_readfirstlane(itm.g), s = __builtin_amdgcn_readfirstlane(itm.part),
              nsp = __builtin_amdgcn_readfirstlane(itm.nsp);

    const int G = a.group;
    const int t0 = a.cu_seq[b];
    const int len = min(a.cu_seq[b + 1] - t0, a.max_chunk);
    const int p0 = a.start[b];
    const int rows_b = len * G;
    const int r_tile0 = qt * TILE_ROWS;
    if (len <= 0 || p0 < 0 || r_tile0 >= rows_b) return;

    const int r_last = min(r_tile0 + TILE_ROWS, rows_b) - 1;
    const int n_keys = WIN && a.ring ? p0 + r_last / G + 1 : min(p0 + r_last / G + 1, a.cap);
    const int n_tiles = (n_keys + kTK - 1) / kTK;
    const int t_first = WIN ? min(first_key_tile(p0 + r_tile0 / G, a.window), n_tiles) : 0;
    const int per = (n_tiles - t_first + nsp - 1) / nsp;
    const int tb = t_first + s * per;
    const int te = min(tb + per, n_tiles);

    const int r = r_tile0 + wave * 32 + rl;
    const int i = r / G;
    const int t = t0 + i;
    const int h = g * G + (r - i * G);
    const bool row_ok = r < rows_b && t >= 0 && t < a.n_tok;
    const int pos = row_ok ? p0 + i : -1;
    const int rw0 = r_tile0 + wave * 32;
    const int pw_lo = __builtin_amdgcn_readfirstlane(p0 + rw0 / G);
    const int win_lo = WIN ? __builtin_amdgcn_readfirstlane(p0 + (rw0 + 31) / G - a.window + 1) : INT_MIN;

    bf16x8_t qf[NKK];
    {
        const uint16_t* qrow =
            reinterpret_cast<const uint16_t*>(a.q) + ((size_t)t * a.n_heads + h) * HD;
#pragma unroll
        for (int k = 0; k < NKK; ++k) {
            u32x4_t u = {0u, 0u, 0u, 0u};
            if (row_ok) u = ld16(qrow + 16 * k + 8 * hf);
            qf[k] = __builtin_bit_cast(bf16x8_t, u);
        }
    }

    const size_t kvbase = ((size_t)b * a.n_kv + g) * (size_t)a.cap * HD;
    const uint16_t* kc = reinterpret_cast<const uint16_t*>(a.k_cache) + kvbase;
    const uint16_t* vc = reinterpret_cast<const uint16_t*>(a.v_cache) + kvbase;

    // staging: thread -> NCH (row, 16-byte chunk) pairs of a tile, buffer
    // loads from a resource over the tile's rows (rows past the last key
    // read as zeros: their scores are masked and their probabilities are 0)
    // SD staging sets: the loads a softmax phase stores were issued SD
    // softmax phases (tiles) earlier
    constexpr int SD = ATTN_PP_STAGE_DEPTH;
    u32x4_t kreg[SD][NCH], vreg[SD][NCH];
    int voff[NCH], kls[NCH], vls[NCH];
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        const int idx = c * kThreads + tid;
        voff[c] = ((idx / CH) * HD + (idx % CH) * 8) * 2;
        kls[c] = (idx / CH) * KS + (idx % CH) * 8;
        vls[c] = (idx / CH) * VS + (idx % CH) * 8;
    }
    const int ring_tiles = a.cap / kTK;
    auto tile_rsrc = [&](const uint16_t* base, int j) __attribute__((always_inline)) {
        const int rows = __builtin_amdgcn_readfirstlane(min(max(n_keys - j * kTK, 0), kTK));
        const int jt = WIN && a.ring ? j % ring_tiles : j;
        return __builtin_amdgcn_make_buffer_rsrc((void*)(base + (size_t)jt * kTK * HD), (short)0, rows * HD * 2,
                                                 kBufferWord3);
    };
    auto load_kv = [&](int jk, int jv, auto set) __attribute__((always_inline)) {
        const auto rk = tile_rsrc(kc, jk);
        const auto rv = tile_rsrc(vc, jv);
#pragma unroll
        for (int c = 0; c < NCH; ++c)
            kreg[set.value][c] =
                __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rk, voff[c], 0, 0));
#pragma unroll
        for (int c = 0; c < NCH; ++c)
            vreg[set.value][c] =
                __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rv, voff[c], 0, 0));
    };
    auto store_k = [&](int slot, auto set) __attribute__((always_inline)) {
#pragma unroll
        for (int c = 0; c < NCH; ++c) st16(&sm.k[slot][kls[c]], kreg[set.value][c]);
    };
    auto store_v = [&](int slot, auto set) __attribute__((always_inline)) {
#pragma unroll
        for (int c = 0; c < NCH; ++c) st16(&sm.v[slot][vls[c]], vreg[set.value][c]);
    };
    constexpr std::integral_constant<int, 0> set0{};
    constexpr std::integral_constant<int, SD - 1> set1{};

    // transposing-read address of this lane inside a V tile (see the
    // full-tile kernel)
    const int tr_off = (4 * hf + ((lane & 15) >> 2)) * VS + 4 * (lane & 3) + 16 * ((lane >> 4) & 1);
    // the same reads in the DMA column layout (byte offsets): a score
    // fragment's lane reads key rl of column 2*kk + hf; a transposing read's
    // lane points at key 4*hf + (lane&15)/4 of column 4*db + 2*((lane>>4)&1)
    // + (lane&3)/2, half (lane&1) of its 16 bytes
    const int kdma_off = hf * kDmaCol + rl * 16;
    const int vdma_off = (2 * ((lane >> 4) & 1) + ((lane & 3) >> 1)) * kDmaCol + (4 * hf + ((lane & 15) >> 2)) * 16 +
                         8 * (lane & 1);
    // DMA staging: wave w loads columns 2w and 2w+1 of each tile; lane i
    // takes key i's chunk
    const uint32_t lds_k = lds_addr(&sm.k[0][0]), lds_v = lds_addr(&sm.v[0][0]);
    const int dma_c0 = 2 * __builtin_amdgcn_readfirstlane(wave);
    auto dma_tile = [&](const uint16_t* base, int j, uint32_t lds_slot) __attribute__((always_inline)) {
        const auto rs = tile_rsrc(base, j);
#pragma unroll
        for (int q = 0; q < 2; ++q)
            dma16(lds_slot + (dma_c0 + q) * kDmaCol, lane * HD * 2 + (dma_c0 + q) * 16, rs);
    };
    constexpr int kSlotBytes = DMA ? PingPongDmaSmem<HD>::kTile : 0;

    f32x16_t O[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int q = 0; q < 16; ++q) O[db][q] = 0.f;
    float m_run = -INFINITY;
    float l_run = 0.f;
    const float sl = a.scale * kLog2e;
    f32x16_t S0, S1;
    uint32_t pk[16];

    // ---- matrix phase: scores of key tile j (slot ks) when SC, and O^T +=
    // V^T P^T of the previous tile (slot vs, probabilities pk) when PV.
    // 2*NKK score products and 4*NDB P.V products, alternated; every
    // fragment is read PFD steps before its product, an order the
    // scheduling groups pin (the reads otherwise drift next to their
    // products and each product waits for a full LDS round trip).
    auto mphase = [&](int ks, int vs, auto SC, auto PV) __attribute__((always_inline)) {
        // phases are kept whole: nothing is scheduled across their bounds
        __builtin_amdgcn_sched_barrier(0);
        if (ATTN_PP_PRIO) __builtin_amdgcn_s_setprio(ATTN_PP_PRIO);
        auto kload = [&](int st) __attribute__((always_inline)) {   // st = (kk, slab)
            if constexpr (DMA) {
                const uint8_t* kb8 = reinterpret_cast<const uint8_t*>(sm.k[ks]) + kdma_off;
                return ld16(kb8 + (st / 2) * 2 * kDmaCol + (st % 2) * 32 * 16);
            } else {
                const uint16_t* kl = reinterpret_cast<const uint16_t*>(sm.k[ks]);
                return ld16(kl + ((st % 2) * 32 + rl) * KS + (st / 2) * 16 + hf * 8);
            }
        };
        auto vfrag = [&](int st) __attribute__((always_inline)) {   // st = (kb, tt, db)
            const int kb = st / (2 * NDB), tt = (st / NDB) % 2, db = st % NDB;
            u32x2_t lo, hi;
            if constexpr (DMA) {
                const uint8_t* vp = reinterpret_cast<const uint8_t*>(sm.v[vs]) + vdma_off + db * 4 * kDmaCol +
                                    (kb * 32 + tt * 16) * 16;
                lo = lds_read_tr16(reinterpret_cast<const uint16_t*>(vp));
                hi = lds_read_tr16(reinterpret_cast<const uint16_t*>(vp + 8 * 16));
            } else {
                const uint16_t* vrow = reinterpret_cast<const uint16_t*>(sm.v[vs]) + tr_off + (kb * 32 + tt * 16) * VS +
                                       db * 32;
                lo = lds_read_tr16(vrow);
                hi = lds_read_tr16(vrow + 8 * VS);
            }
            const u32x4_t vv = {lo.x, lo.y, hi.x, hi.y};
            return vv;
        };
        if (SC.value) {
#pragma unroll
            for (int q = 0; q < 16; ++q) {
                S0[q] = 0.f;
                S1[q] = 0.f;
            }
        }
        constexpr int NS = SC.value ? 2 * NKK : 0;
        constexpr int NP = PV.value ? 4 * NDB : 0;
        constexpr int NT = NS > NP ? NS : NP;
        constexpr int PFD = ATTN_PP_PREFETCH;
        u32x4_t kf[PFD + 1], vf[PFD + 1];
#pragma unroll
        for (int st = 0; st < PFD; ++st) {
            if (st < NS) kf[st] = kload(st);
            if (st < NP) vf[st] = vfrag(st);
        }
        __builtin_amdgcn_sched_group_barrier(0x100, (PFD < NS ? PFD : NS) + 2 * (PFD < NP ? PFD : NP), 0);
        static_for<0, NT>([&](auto ic) __attribute__((always_inline)) {
            constexpr int st = decltype(ic)::value;
            if constexpr (st + PFD < NS) kf[(st + PFD) % (PFD + 1)] = kload(st + PFD);
            if constexpr (st + PFD < NP) vf[(st + PFD) % (PFD + 1)] = vfrag(st + PFD);
            if constexpr (st < NS) {
                if constexpr (st % 2 == 0)
                    S0 = mfma32(__builtin_bit_cast(bf16x8_t, kf[st % (PFD + 1)]), qf[st / 2], S0);
                else
                    S1 = mfma32(__builtin_bit_cast(bf16x8_t, kf[st % (PFD + 1)]), qf[st / 2], S1);
            }
            if constexpr (st < NP) {
                constexpr int kb = st / (2 * NDB), tt = (st / NDB) % 2, db = st % NDB;
                constexpr int pq = kb * 8 + tt * 4;
                const u32x4_t pv = {pk[pq], pk[pq + 1], pk[pq + 2], pk[pq + 3]};
                O[db] = mfma32(__builtin_bit_cast(bf16x8_t, vf[st % (PFD + 1)]), __builtin_bit_cast(bf16x8_t, pv), O[db]);
            }
            constexpr int nrd = (st + PFD < NS ? 1 : 0) + (st + PFD < NP ? 2 : 0);
            if constexpr (nrd > 0) __builtin_amdgcn_sched_group_barrier(0x100, nrd, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, (st < NS ? 1 : 0) + (st < NP ? 1 : 0), 0);
        });
        if (ATTN_PP_PRIO) __builtin_amdgcn_s_setprio(0);
        __builtin_amdgcn_sched_barrier(0);
    };

    // ---- softmax phase of key tile j (scores S0/S1): masks, row maximum,
    // the rare rescale, probabilities rounded to bf16 (pk) and the row sum
    // of the rounded values; then this thread's staging share is written to
    // LDS (K[j+2] into slot ksl, V[j+1] into slot vsl) and the next share's
    // global loads are issued
    auto vphase = [&](int j, int ksl, int vsl, auto set) __attribute__((always_inline)) {
        if constexpr (DMA && ATTN_PP_DMA_AT == 1) {
            dma_tile(kc, min(j + 3, te - 1), lds_k + ksl * kSlotBytes);
            dma_tile(vc, min(j + 2, te - 1), lds_v + vsl * kSlotBytes);
        }
        const int k0 = j * kTK;
        if (k0 + kTK - 1 > pw_lo) {
            const int lim = pos - k0 - 4 * hf;
#pragma unroll
            for (int q = 0; q < 16; ++q) {
                const int off = 8 * (q >> 2) + (q & 3);
                if (off > lim) S0[q] = -INFINITY;
                if (off + 32 > lim) S1[q] = -INFINITY;
            }
        }
        if (WIN && k0 < win_lo) {
            const int llim = pos - a.window + 1 - k0 - 4 * hf;
#pragma unroll
            for (int q = 0; q < 16; ++q) {
                const int off = 8 * (q >> 2) + (q & 3);
                if (off < llim) S0[q] = -INFINITY;
                if (off + 32 < llim) S1[q] = -INFINITY;
            }
        }
        // 32 scores in 16 three-input maxima (two chains, joined at the end)
        float mx0 = __builtin_fmaxf(__builtin_fmaxf(S0[0], S0[1]), S0[2]);
        float mx1 = __builtin_fmaxf(__builtin_fmaxf(S1[0], S1[1]), S1[2]);
#pragma unroll
        for (int q = 3; q < 15; q += 2) {
            mx0 = __builtin_fmaxf(__builtin_fmaxf(mx0, S0[q]), S0[q + 1]);
            mx1 = __builtin_fmaxf(__builtin_fmaxf(mx1, S1[q]), S1[q + 1]);
        }
        float mx = __builtin_fmaxf(__builtin_fmaxf(mx0, S0[15]), __builtin_fmaxf(mx1, S1[15]));
        if (ATTN_PP_PERMLANE) {
            const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
            mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
        } else {
            mx = fmaxf(mx, __shfl_xor(mx, 32));
        }
        const float mt = mx * sl;
        const bool grow = mt > m_run + kRescaleSlack;
        const float m_new = grow ? mt : m_run;
        const float m_use = m_new == -INFINITY ? 0.f : m_new;
        if (__any(grow)) {
            const float alpha = grow ? __builtin_amdgcn_exp2f(m_run - m_use) : 1.f;
            l_run *= alpha;
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int q = 0; q < 16; ++q) O[db][q] *= alpha;
        }
        m_run = m_new;
        const float nm = -m_use;
#pragma unroll
        for (int q = 0; q < 8; ++q)
            pk[q] = pack_bf16x2(__builtin_amdgcn_exp2f(__builtin_fmaf(S0[2 * q], sl, nm)),
                                __builtin_amdgcn_exp2f(__builtin_fmaf(S0[2 * q + 1], sl, nm)));
#pragma unroll
        for (int q = 0; q < 8; ++q)
            pk[8 + q] = pack_bf16x2(__builtin_amdgcn_exp2f(__builtin_fmaf(S1[2 * q], sl, nm)),
                                    __builtin_amdgcn_exp2f(__builtin_fmaf(S1[2 * q + 1], sl, nm)));
        l_run += sum_bf16_pairs(pk);
        // register staging (head dimension 64): this thread's staging share,
        // then the next share's global loads (unconditional, tile index
        // clamped: past the last tile they refill slots that are never read
        // again).  Measured on that path: issuing them at the start of the
        // phase, or reading the next matrix phase's first fragments here, is
        // slower.  The DMA path issues its loads where ATTN_PP_DMA_AT says.
        if (ATTN_PP_LATE_STORE) __builtin_amdgcn_sched_barrier(0);
        if constexpr (DMA) {
            // K[j+3] and V[j+2], two tiles ahead (slots given by the caller)
            if (ATTN_PP_DMA_AT == 0) {
                dma_tile(kc, min(j + 3, te - 1), lds_k + ksl * kSlotBytes);
                dma_tile(vc, min(j + 2, te - 1), lds_v + vsl * kSlotBytes);
            }
        } else {
            store_k(ksl, set);
            store_v(vsl, set);
            load_kv(min(j + 2 + SD, te - 1), min(j + 1 + SD, te - 1), set);
        }
    };

    constexpr std::integral_constant<bool, true> yes{};
    constexpr std::integral_constant<bool, false> no{};
    const int n = te - tb;
    if (DMA && n > 0) {
        // prologue: K[tb..tb+2] and V[tb..tb+1] in slots 0..2 / 0..1; tile
        // tb+k sits in slot k mod 4.  Softmax phase k loads K[tb+k+3] and
        // V[tb+k+2]; the end of matrix phase k waits for the loads of softmax
        // phase k-1 (those of phase k may still be in flight), which every
        // wave does before the barrier after which the first reader starts.
        dma_tile(kc, tb, lds_k);
        dma_tile(vc, tb, lds_v);
        dma_tile(kc, min(tb + 1, te - 1), lds_k + kSlotBytes);
        dma_tile(vc, min(tb + 1, te - 1), lds_v + kSlotBytes);
        dma_tile(kc, min(tb + 2, te - 1), lds_k + 2 * kSlotBytes);
        wait_vmcnt<0>();
        __syncthreads();
        if (grp == 1) __syncthreads();            // the second group starts one phase later
        mphase(0, 0, yes, no);
        __syncthreads();
        int k = 0;
        for (; k < n - 1; ++k) {
            vphase(tb + k, (k + 3) & 3, (k + 2) & 3, set0);
            __syncthreads();
            mphase((k + 1) & 3, k & 3, yes, yes);
            wait_vmcnt<4>();
            __syncthreads();
        }
        vphase(tb + k, (k + 3) & 3, (k + 2) & 3, set0);
        __syncthreads();
        mphase((k + 1) & 3, k & 3, no, yes);
        __syncthreads();
        if (grp == 0) __syncthreads();            // the same barrier count in both groups
        wait_vmcnt<0>();                          // no LDS write outlives the workgroup
    } else if (n > 0) {
        // prologue: K[tb], V[tb], K[tb+1] in slots 0, 0, 1; the staging
        // sets then hold K[tb+2+s] and V[tb+1+s] for the softmax phase s
        load_kv(tb, tb, set0);
        store_k(0, set0);
        store_v(0, set0);
        load_kv(min(tb + 1, te - 1), tb, set0);
        store_k(1, set0);
        load_kv(min(tb + 2, te - 1), min(tb + 1, te - 1), set0);
        if (SD == 2) load_kv(min(tb + 3, te - 1), min(tb + 2, te - 1), set1);
        __syncthreads();
        if (grp == 1) __syncthreads();            // the second group starts one phase later
        mphase(0, 0, yes, no);
        __syncthreads();
        // slots of tile tb+k: K and V in (k mod 3); staging set k mod SD
        int sk = 0;                               // slot of key tile tb+k
        auto step = [&](int k, auto set) __attribute__((always_inline)) {
            const int s1 = sk == 2 ? 0 : sk + 1, s2 = s1 == 2 ? 0 : s1 + 1;
            vphase(tb + k, s2, s1, set);
            __syncthreads();
            mphase(s1, sk, yes, yes);
            __syncthreads();
            sk = s1;
        };
        auto last = [&](auto set) __attribute__((always_inline)) {
            const int s1 = sk == 2 ? 0 : sk + 1, s2 = s1 == 2 ? 0 : s1 + 1;
            vphase(tb + n - 1, s2, s1, set);
            __syncthreads();
            mphase(s1, sk, no, yes);
            __syncthreads();
        };
        int k = 0;
        for (; k + SD <= n - 1; k += SD) {
            step(k, set0);
            if (SD == 2) step(k + 1, set1);
        }
        if (SD == 2 && k < n - 1) {
            step(k, set0);
            last(set1);
        } else {
            last(set0);
        }
        if (grp == 0) __syncthreads();            // the same barrier count in both groups
    }

    const float l_tot = l_run + __shfl_xor(l_run, 32);
    if (!row_ok) return;
    write_row<HD>(a, O, m_run, l_tot, t, h, hf, nsp,
                  a.part + ((size_t)item * TILE_ROWS + (r - r_tile0)) * part_row_words(HD));
}

// Key-split variant for 128-row work items: 8 waves, the waves w and w+4
// hold the same 32 query rows and take the two 32-key halves of every tile
// (kh = wave / 4), each with its own online softmax; the halves merge through
// LDS at the end.  Against 4 waves of 32 rows over whole tiles it has two
// waves per SIMD from one workgroup (one wave's matrix products overlap the
// other's exponentials), the deeper prefetch of the 8-wave layout, and half
// the serial work per wave and tile -- what a small call with one workgroup
// per CU is limited by.
template <int HD, bool WIN>
__global__ __launch_bounds__(512, 1) void prefill_bf16_ks_kernel(PrefillArgs a) {
    using Sm = PrefillSmem<HD>;
    constexpr int kThreads = 512;
    constexpr int PD = 2;                         // staging sets = prefetch depth
    constexpr int KS = Sm::KS;
    constexpr int VS = Sm::VS;
    constexpr int CH = HD / 8;                    // 16-byte chunks per cache row
    constexpr int NCH = kTK * CH / kThreads;      // K (and V) chunks per thread
    constexpr int NDB = HD / 32;                  // 32-dim blocks of O
    constexpr int NKK = HD / 16;                  // K-steps of a score product
    constexpr int TILE_ROWS = 128;                // query rows per workgroup
    __shared__ Sm sm;
    const int wg = attention_wg(a);
    if (wg < 0 || wg >= a.grid) {
        extra_role<HD>(a, sm, wg);
        return;
    }

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int kh = wave >> 2;                     // key half of every tile
    const int wr = wave & 3;                      // row block
    const int hf = lane >> 5;                     // wave half
    const int rl = lane & 31;

    const int item = wg;
    PrefillItem itm;
    if (a.split) {
        itm = split_schedule(a, item);
    } else {
        itm.g = item % a.n_kv;
        itm.qt = a.n_qtiles - 1 - (item / a.n_kv) % a.n_qtiles;
        itm.b = item / (a.n_kv * a.n_qtiles);
        itm.part = 0;
        itm.nsp = 1;
    }
    if (itm.nsp <= 0) return;
    const int b = __builtin_amdgcn_readfirstlane(itm.b), qt = __builtin_amdgcn_readfirstlane(itm.qt),
              g = __builtin_amdgcn_readfirstlane(itm.g), s = __builtin_amdgcn_readfirstlane(itm.part),
              nsp = __builtin_amdgcn_readfirstlane(itm.nsp);

    const int G = a.group;
    const int t0 = a.cu_seq[b];
    const int len = min(a.cu_seq[b + 1] - t0, a.max_chunk);
    const int p0 = a.start[b];
    const int rows_b = len * G;
    const int r_tile0 = qt * TILE_ROWS;
    if (len <= 0 || p0 < 0 || r_tile0 >= rows_b) return;

    const int r_last = min(r_tile0 + TILE_ROWS, rows_b) - 1;
    const int n_keys = WIN && a.ring ? p0 + r_last / G + 1 : min(p0 + r_last / G + 1, a.cap);
    const int n_tiles = (n_keys + kTK - 1) / kTK;
    const int t_first = WIN ? min(first_key_tile(p0 + r_tile0 / G, a.window), n_tiles) : 0;
    const int per = (n_tiles - t_first + nsp - 1) / nsp;
    const int tb = t_first + s * per;
    const int te = min(tb + per, n_tiles);

    const int r = r_tile0 + wr * 32 + rl;
    const int i = r / G;
    const int t = t0 + i;
    const int h = g * G + (r - i * G);
    const bool row_ok = r < rows_b && t >= 0 && t < a.n_tok;
    const int pos = row_ok ? p0 + i : -1;
    const int rw0 = r_tile0 + wr * 32;
    const int pw_lo = p0 + rw0 / G;
    const int win_lo = WIN ? p0 + (rw0 + 31) / G - a.window + 1 : INT_MIN;
    const int koff = 32 * kh;                     // this wave's keys inside a tile

    bf16x8_t qf[NKK];
    {
        const uint16_t* qrow =
            reinterpret_cast<const uint16_t*>(a.q) + ((size_t)t * a.n_heads + h) * HD;
#pragma unroll
        for (int k = 0; k < NKK; ++k) {
            u32x4_t u = {0u, 0u, 0u, 0u};
            if (row_ok) u = ld16(qrow + 16 * k + 8 * hf);
            qf[k] = __builtin_bit_cast(bf16x8_t, u);
        }
    }

    const size_t kvbase = ((size_t)b * a.n_kv + g) * (size_t)a.cap * HD;
    const uint16_t* kc = reinterpret_cast<const uint16_t*>(a.k_cache) + kvbase;
    const uint16_t* vc = reinterpret_cast<const uint16_t*>(a.v_cache) + kvbase;

    // staging as in the full-tile kernel (buffer loads with the tile in
    // scalar registers; rows past the last key read as zeros)
    u32x4_t kreg[PD][NCH], vreg[PD][NCH];
    int voff[NCH];
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        const int idx = c * kThreads + tid;
        voff[c] = ((idx / CH) * HD + (idx % CH) * 8) * 2;
    }
    const int ring_tiles = a.cap / kTK;
    auto tile_rsrc = [&](const uint16_t* base, int j) __attribute__((always_inline)) {
        // the clamp compiles to a vector-ALU instruction; without the
        // readfirstlane the compiler cannot see that the resource is uniform
        // and wraps every load in a loop over distinct resource values
        const int rows = __builtin_amdgcn_readfirstlane(min(max(n_keys - j * kTK, 0), kTK));
        const int jt = WIN && a.ring ? j % ring_tiles : j;
        return __builtin_amdgcn_make_buffer_rsrc((void*)(base + (size_t)jt * kTK * HD), (short)0, rows * HD * 2,
                                                 kBufferWord3);
    };
    auto lds_off = [&](int c, int stride) __attribute__((always_inline)) {
        const int idx = c * kThreads + tid;
        return (idx / CH) * stride + (idx % CH) * 8;
    };
    auto load_k = [&](int j, auto set) __attribute__((always_inline)) {
        const auto rs = tile_rsrc(kc, j);
#pragma unroll
        for (int c = 0; c < NCH; ++c)
            kreg[set.value][c] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rs, voff[c], 0, 0));
    };
    auto load_v = [&](int j, auto set) __attribute__((always_inline)) {
        const auto rs = tile_rsrc(vc, j);
#pragma unroll
        for (int c = 0; c < NCH; ++c)
            vreg[set.value][c] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rs, voff[c], 0, 0));
    };
    auto store_k = [&](int buf, auto set) __attribute__((always_inline)) {
#pragma unroll
        for (int c = 0; c < NCH; ++c) st16(&sm.k[buf][lds_off(c, KS)], kreg[set.value][c]);
    };
    auto store_v = [&](int buf, auto set) __attribute__((always_inline)) {
#pragma unroll
        for (int c = 0; c < NCH; ++c) st16(&sm.v[buf][lds_off(c, VS)], vreg[set.value][c]);
    };
    constexpr std::integral_constant<int, 0> set0{};
    constexpr std::integral_constant<int, 1> set1{};
    // scores of this wave's 32 keys of a tile: S[q] holds key
    // koff + 4*hf + 8*(q/4) + q%4 of its row
    auto scores = [&](const uint16_t* kl, f32x16_t& S) __attribute__((always_inline)) {
#pragma unroll
        for (int q = 0; q < 16; ++q) S[q] = 0.f;
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk)
            S = mfma32(__builtin_bit_cast(bf16x8_t, ld16(kl + (koff + rl) * KS + kk * 16 + hf * 8)), qf[kk], S);
    };

    const int tr_off = (koff + 4 * hf + ((lane & 15) >> 2)) * VS + 4 * (lane & 3) + 16 * ((lane >> 4) & 1);

    f32x16_t O[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int q = 0; q < 16; ++q) O[db][q] = 0.f;
    float m_run = -INFINITY;
    float l_run = 0.f;
    const float sl = a.scale * kLog2e;

    if (tb < te) {
        // the first two K tiles and the first V tile in flight together
        load_k(tb, set0);
        load_v(tb, set0);
        load_k(min(tb + 1, te - 1), set1);
        store_k(0, set0);
        store_v(0, set0);
        store_k(1, set1);
        __syncthreads();
        f32x16_t S;
        scores(sm.k[0], S);
        load_k(min(tb + 2, te - 1), set0);
        load_v(min(tb + 1, te - 1), set0);

        auto tile = [&](int j, auto cur, auto nxt) __attribute__((always_inline)) {
            const int rr = (j - tb) & 1;
            load_k(min(j + 3, te - 1), nxt);
            load_v(min(j + 2, te - 1), nxt);
            const int k0 = j * kTK + koff;        // this wave's first key

            // ---- causal mask (tiles crossing the diagonal), window mask
            if (k0 + 31 > pw_lo) {
                const int lim = pos - k0 - 4 * hf;
#pragma unroll
                for (int q = 0; q < 16; ++q)
                    if (8 * (q >> 2) + (q & 3) > lim) S[q] = -INFINITY;
            }
            if (WIN && k0 < win_lo) {
                const int llim = pos - a.window + 1 - k0 - 4 * hf;
#pragma unroll
                for (int q = 0; q < 16; ++q)
                    if (8 * (q >> 2) + (q & 3) < llim) S[q] = -INFINITY;
            }

            // ---- row max of this wave's keys and the (rare) rescale of O
            float mx = S[0];
#pragma unroll
            for (int q = 1; q < 16; ++q) mx = fmaxf(mx, S[q]);
            mx = fmaxf(mx, __shfl_xor(mx, 32));
            const float mt = mx * sl;
            const bool grow = mt > m_run + kRescaleSlack;
            const float m_new = grow ? mt : m_run;
            const float m_use = m_new == -INFINITY ? 0.f : m_new;
            if (__any(grow)) {
                const float alpha = grow ? __builtin_amdgcn_exp2f(m_run - m_use) : 1.f;
                l_run *= alpha;
#pragma unroll
                for (int db = 0; db < NDB; ++db)
#pragma unroll
                    for (int q = 0; q < 16; ++q) O[db][q] *= alpha;
            }
            m_run = m_new;
            const float nm = -m_use;
            uint32_t pk[8];

            // ---- next tile's scores on the matrix cores while the vector
            // ALU forms this tile's probabilities
            f32x16_t N;
            {
                const uint16_t* kl = sm.k[rr ^ 1];
#pragma unroll
                for (int q = 0; q < 16; ++q) N[q] = 0.f;
                u32x4_t a0 = ld16(kl + (koff + rl) * KS + hf * 8);
#pragma unroll
                for (int kk = 0; kk < NKK; ++kk) {
                    u32x4_t b0 = a0;
                    if (kk + 1 < NKK) b0 = ld16(kl + (koff + rl) * KS + (kk + 1) * 16 + hf * 8);
                    N = mfma32(__builtin_bit_cast(bf16x8_t, a0), qf[kk], N);
#pragma unroll
                    for (int q = kk * 8 / NKK; q < (kk + 1) * 8 / NKK; ++q)
                        pk[q] = pack_bf16x2(__builtin_amdgcn_exp2f(__builtin_fmaf(S[2 * q], sl, nm)),
                                            __builtin_amdgcn_exp2f(__builtin_fmaf(S[2 * q + 1], sl, nm)));
                    a0 = b0;
                }
                ATTN_INTERLEAVE(NKK, 1, 4);
            }

            // the K/V data stored at this tile's end arrived during the
            // previous tile: K[j+2] replaces K[j], V[j+1] replaces V[j-1]
            store_k(rr, cur);
            store_v(rr ^ 1, cur);

            // ---- O^T += V^T P^T over this wave's 32 keys
            {
                const uint16_t* vl = sm.v[rr] + tr_off;
                auto vfrag = [&](int tt, int db) __attribute__((always_inline)) {
                    const uint16_t* vrow = vl + (tt * 16) * VS + db * 32;
                    const u32x2_t lo = lds_read_tr16(vrow);
                    const u32x2_t hi = lds_read_tr16(vrow + 8 * VS);
                    const u32x4_t vv = {lo.x, lo.y, hi.x, hi.y};
                    return vv;
                };
                u32x4_t va = vfrag(0, 0);
#pragma unroll
                for (int st = 0; st < 2 * NDB; ++st) {          // st = (tt, db)
                    const int tt = st / NDB, db = st % NDB;
                    u32x4_t vn = va;
                    if (st + 1 < 2 * NDB) vn = vfrag((st + 1) / NDB, (st + 1) % NDB);
                    const u32x4_t pv = {pk[tt * 4], pk[tt * 4 + 1], pk[tt * 4 + 2], pk[tt * 4 + 3]};
                    O[db] = mfma32(__builtin_bit_cast(bf16x8_t, va), __builtin_bit_cast(bf16x8_t, pv), O[db]);
                    va = vn;
                }
            }
            // the row sum is taken from the rounded probabilities
            {
                const bf16x2_t one = __builtin_bit_cast(bf16x2_t, 0x3f803f80u);
                float s0 = 0.f, s1 = 0.f;
#pragma unroll
                for (int q = 0; q < 8; q += 2) {
                    s0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pk[q]), one, s0, false);
                    s1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pk[q + 1]), one, s1, false);
                }
                l_run += s0 + s1;
            }
            __syncthreads();
            S = N;
        };
        for (int j = tb; j < te; ++j) {
            tile(j, set0, set1);
            if (++j >= te) break;
            tile(j, set1, set0);
        }
    }

    // ---- merge the key halves: waves 4..7 hand (m, l, O) of their rows to
    // waves 0..3 through LDS (the tile buffers are free after the barrier)
    // (per lane: O, then m and l, in a 16-byte-aligned block of NDB*16 + 4
    // floats, read and written 16 bytes at a time; the stride of 4 mod 64
    // words keeps 16 lanes' reads on distinct banks)
    __syncthreads();
    static_assert(4 * 64 * (NDB * 16 + 4) * sizeof(float) <= sizeof(Sm), "exchange fits the tile buffers");
    f32x4_t* xch = reinterpret_cast<f32x4_t*>(&sm) + ((size_t)wr * 64 + lane) * (NDB * 4 + 1);
    if (kh == 1) {
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4)
                xch[db * 4 + q4] = f32x4_t{O[db][4 * q4], O[db][4 * q4 + 1], O[db][4 * q4 + 2], O[db][4 * q4 + 3]};
        xch[NDB * 4] = f32x4_t{m_run, l_run, 0.f, 0.f};
    }
    __syncthreads();
    if (kh == 1) return;
    {
        const f32x4_t ml = xch[NDB * 4];
        const float m1 = ml[0], l1 = ml[1];
        const float mm = fmaxf(m_run, m1);
        const float mu = mm == -INFINITY ? 0.f : mm;
        const float a0 = __builtin_amdgcn_exp2f(m_run - mu), a1 = __builtin_amdgcn_exp2f(m1 - mu);
        l_run = l_run * a0 + l1 * a1;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const f32x4_t x = xch[db * 4 + q4];
#pragma unroll
                for (int e = 0; e < 4; ++e) O[db][4 * q4 + e] = O[db][4 * q4 + e] * a0 + x[e] * a1;
            }
        m_run = mm;
    }

    const float l_tot = l_run + __shfl_xor(l_run, 32);
    if (!row_ok) return;
    write_row<HD>(a, O, m_run, l_tot, t, h, hf, nsp,
                  a.part + ((size_t)item * TILE_ROWS + (r - r_tile0)) * part_row_words(HD));
}

// Merge split partials (m, l, O/l) of each row: m* = max m_s,
// l* = sum l_s 2^(m_s - m*), out = sum (O/l)_s l_s 2^(m_s - m*) / l*.  A row
// is LPR = HD/8 lanes, each over 8 consecutive dims (one 16-byte load of
// halves per part), so a wave merges 64/LPR rows; lane j of a row also reads
// part j's (m, l, e), and the row's maximum and sum are reductions over its
// LPR lanes.  The first parts' values are loaded with the part heads, each
// later batch of four while the previous one is accumulated.  Workgroup
// (x, sequence) takes 4*64/LPR rows of the row tile x / (n_kv * R/RPB) and KV
// group x % n_kv; row tiles that were not split were written by the
// attention kernel.
template <int HD>
struct CombineShape {
    static constexpr int LPR = HD / 8;        // lanes per row
    static constexpr int RPW = 64 / LPR;      // rows per wave
    static constexpr int RPB = 4 * RPW;       // rows per workgroup
};
// Merge block (bx, b) of 256 threads, thread tid (the standalone kernel's
// blockIdx.x, blockIdx.y and threadIdx.x).
template <int HD>
__device__ __forceinline__ void merge_rows(const MergeArgs& a, int bx, int b, int tid) {
    using Sh = CombineShape<HD>;
    constexpr int LPR = Sh::LPR, RPB = Sh::RPB;
    constexpr int PS = part_row_words(HD);
    constexpr int NB = 4;                     // parts per load batch
    const int R = a.rows_per_tile;
    const int g = bx % a.n_kv;
    const int rblk = (bx / a.n_kv) % (R / RPB);
    const int qt = bx / a.n_kv / (R / RPB);
    if (b >= a.n_seq || qt >= a.n_qtiles) return;
    const int first = a.table[2 * (b * a.n_qtiles + qt)];
    const int S = a.table[2 * (b * a.n_qtiles + qt) + 1];
    if (S <= 1) return;
    const int G = a.group;
    const int t0 = a.cu_seq[b];
    const int len = min(a.cu_seq[b + 1] - t0, a.max_chunk);
    const int rows_b = len * G;
    const int lane = tid & 63;
    const int j = lane % LPR;                  // this lane's 8 dims: 8j .. 8j+7
    const int rl = rblk * RPB + (tid / 64) * (64 / LPR) + lane / LPR;
    const int r = qt * R + rl;
    const int i = r / G;
    const int h = g * G + (r - i * G);
    const int t = t0 + i;
    // a row's lanes are one aligned group: they skip together, and the
    // group's shuffles below read only lanes of the same row
    const bool row_ok = r < rows_b && t >= 0 && t < a.n_tok;
    auto prow = [&](int p) { return a.part + ((size_t)(first + p * a.n_kv + g) * R + rl) * PS; };
    auto load_vals = [&](int p) __attribute__((always_inline)) {
        return p < S && row_ok ? *reinterpret_cast<const u32x4_t*>(prow(p) + kPartHead + 4 * j)
                               : u32x4_t{0u, 0u, 0u, 0u};
    };
    // part heads: lane j holds part j (and j + LPR, ... when S > LPR: max only)
    float mp = -INFINITY, lp = 0.f, ep = 0.f;
    u32x4_t xv[NB];
#pragma unroll
    for (int u = 0; u < NB; ++u) xv[u] = load_vals(u);
    if (row_ok) {
        for (int p = j; p < S; p += LPR) {
            const float4 ml = *reinterpret_cast<const float4*>(prow(p));
            if (p < LPR) { mp = ml.x; lp = ml.y; ep = ml.z; }
            else { mp = fmaxf(mp, ml.x); }
        }
    }
    // output gate factors, so their loads overlap the merge: the lane's 8
    // per-element values in one 16-byte load when the rows allow it
    float gf[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) gf[e] = 1.f;
    if (a.gate.mode && row_ok) {
        const size_t grow = (size_t)t * a.n_heads + h;
        const uint16_t* gp = reinterpret_cast<const uint16_t*>(a.gate.p) + grow * (size_t)a.gate.ld;
        if (a.gate.mode == kGateSoftplusHead) {
            const float f = gate_fast(a.gate.mode, bf16_to_f32(gp[0]));
#pragma unroll
            for (int e = 0; e < 8; ++e) gf[e] = f;
        } else if (((a.gate.ld & 7) == 0) && ((reinterpret_cast<uintptr_t>(a.gate.p) & 15) == 0)) {
            const u32x4_t g4 = ld16(gp + 8 * j);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                gf[2 * q] = gate_fast(a.gate.mode, bf16_lo(g4[q]));
                gf[2 * q + 1] = gate_fast(a.gate.mode, bf16_hi(g4[q]));
            }
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) gf[e] = gate_fast(a.gate.mode, bf16_to_f32(gp[8 * j + e]));
        }
    }
    float m = mp;
#pragma unroll
    for (int o = 1; o < LPR; o <<= 1) m = fmaxf(m, __shfl_xor(m, o));
    const float m_use = m == -INFINITY ? 0.f : m;
    // part weight in l: l_p 2^(m_p - m); on the stored values also 2^e_p
    const float wl = j < S ? lp * __builtin_amdgcn_exp2f(mp - m_use) : 0.f;
    const float wo = __builtin_amdgcn_ldexpf(wl, (int)ep);
    float l = wl;
    const int gbase = lane - j;
    float o[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = 0.f;
    auto accum = [&](const u32x4_t& x, float w) __attribute__((always_inline)) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            o[2 * q] += f16_value((uint16_t)x[q]) * w;
            o[2 * q + 1] += f16_value((uint16_t)(x[q] >> 16)) * w;
        }
    };
    if (S <= LPR) {
#pragma unroll
        for (int o2 = 1; o2 < LPR; o2 <<= 1) l += __shfl_xor(l, o2);
        for (int p = 0; p < S; p += NB) {
            u32x4_t nx[NB];
#pragma unroll
            for (int u = 0; u < NB; ++u) nx[u] = load_vals(p + NB + u);
#pragma unroll
            for (int u = 0; u < NB; ++u) {
                const float w = __shfl(wo, gbase + min(p + u, LPR - 1));
                if (p + u < S) accum(xv[u], w);
            }
#pragma unroll
            for (int u = 0; u < NB; ++u) xv[u] = nx[u];
        }
    } else {
        // more parts than lanes: every lane forms each weight itself
        l = 0.f;
        if (row_ok) {
            for (int p = 0; p < S; ++p) {
                const float4 hd4 = *reinterpret_cast<const float4*>(prow(p));
                const float w = hd4.y * __builtin_amdgcn_exp2f(hd4.x - m_use);
                l += w;
                accum(load_vals(p), __builtin_amdgcn_ldexpf(w, (int)hd4.z));
            }
        }
    }
    if (!row_ok) return;
    const float inv = l > 0.f ? 1.f / l : 0.f;
    float* orow = a.out + ((size_t)t * a.n_heads + h) * HD + 8 * j;
    *reinterpret_cast<float4*>(orow) =
        make_float4(o[0] * inv * gf[0], o[1] * inv * gf[1], o[2] * inv * gf[2], o[3] * inv * gf[3]);
    *reinterpret_cast<float4*>(orow + 4) =
        make_float4(o[4] * inv * gf[4], o[5] * inv * gf[5], o[6] * inv * gf[6], o[7] * inv * gf[7]);
}

template <int HD>
__global__ __launch_bounds__(256) void prefill_combine_kernel(MergeArgs a) {
    merge_rows<HD>(a, blockIdx.x, blockIdx.y, threadIdx.x);
}

// Launch plan.  256-row workgroups (8 waves, deeper prefetch) when they
// alone give every CU a workgroup; otherwise 128-row workgroups.  When the
// row tiles are too few for the GPU (an upper bound from host scalars: every
// sequence with max_chunk tokens) and the longest key range spans more than
// min_tiles_per_split tiles, the call splits: a persistent grid of one
// workgroup per CU slot, with the part length chosen on the device from the
// actual lengths (see the schedule above).
#ifndef ATTN_PREFILL_BIG_TILE_BLOCKS
#define ATTN_PREFILL_BIG_TILE_BLOCKS 512
#endif
constexpr int kBigTileBlocks = ATTN_PREFILL_BIG_TILE_BLOCKS;
constexpr int kMaxSplitGroups = 64;      // (sequence, row tile) pairs: one per lane

int device_cus() {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
        cus = 256;
    return cus;
}

PrefillPlan plan_prefill(int n_seq, int n_heads, int n_kv, int head_dim, int n_tok, int max_chunk,
                         int max_end, int window, size_t ws_available) {
    const long group = n_heads / n_kv;
    const long rows = (long)max_chunk * group;
    long tiles = ((long)max_end + kTK - 1) / kTK;
    // a window bounds a row tile's key range by W plus its own positions
    // (at most 256 rows) and the alignment of both ends
    if (window > 0) tiles = std::min(tiles, ((long)window + 256 + 2 * kTK - 2) / kTK + 1);
    const long big = (long)n_seq * ((rows + 255) / 256) * n_kv;
    PrefillPlan p{};
    p.rows_per_tile = big >= kBigTileBlocks / 2 ? 256 : 128;
    p.n_qtiles = (int)((rows + p.rows_per_tile - 1) / p.rows_per_tile);
    const long base = (long)n_seq * p.n_qtiles * n_kv;
    p.split = 0;
    p.grid = (int)base;
    p.ws_bytes = 0;
    p.table_bytes = 0;
    if (base < kBigTileBlocks && tiles > min_tiles_per_split(p.rows_per_tile) &&
        (long)n_seq * p.n_qtiles <= kMaxSplitGroups) {
        const long slots = device_cus();       // one 8-wave workgroup per CU
        const size_t table = ((size_t)n_seq * p.n_qtiles * 2 * sizeof(int) + 255) / 256 * 256;
        // items <= slots + one extra part per row tile (ceil) -- see split_schedule
        const size_t parts = (size_t)(slots + base) * p.rows_per_tile * part_row_words(head_dim) * sizeof(float);
        if (table + parts <= ws_available) {
            p.split = 1;
            p.slots = (int)slots;
            p.grid = (int)(slots + base);
            p.table_bytes = table;
            p.ws_bytes = table + parts;
            p.part_tiles = 0;
            if (n_seq == 1) {
                // the same choice the device would make, from exact sizes:
                // len = n_tok rows starting at max_end - len
                const long len = n_tok < max_chunk ? n_tok : max_chunk;
                const long p0 = max_end - len;
                long gt[kMaxSplitGroups];
                long gmax = 1;
                for (int qt = 0; qt < p.n_qtiles; ++qt) {
                    const long r0 = (long)qt * p.rows_per_tile, rows_b = len * group;
                    gt[qt] = 0;
                    if (len > 0 && p0 >= 0 && r0 < rows_b) {
                        const long r_last = (r0 + p.rows_per_tile < rows_b ? r0 + p.rows_per_tile : rows_b) - 1;
                        const long nk = p0 + r_last / group + 1;
                        const long nt = (nk + kTK - 1) / kTK;
                        gt[qt] = nt - std::min((long)first_key_tile((int)(p0 + r0 / group), window), nt);
                    }
                    if (gt[qt] > gmax) gmax = gt[qt];
                }
                long best_T = gmax, best_cost = -1, prev_T = 0, best_n = 0;
                const int cand[12] = {1, 2, 3, 4, 6, 8, 12, 16, 24, 32, 48, 64};
                for (int k : cand) {
                    const long T = (gmax + k - 1) / k;
                    if (T < min_tiles_per_split(p.rows_per_tile) && k > 1) break;
                    if (T == prev_T) continue;
                    prev_T = T;
                    long n = 0;
                    for (int qt = 0; qt < p.n_qtiles; ++qt) n += gt[qt] > 0 ? (gt[qt] + T - 1) / T : 0;
                    n *= n_kv;
                    if (n > p.grid) continue;
                    const long cost = (n + slots - 1) / slots * (T + item_cost_tiles(p.rows_per_tile));
                    if (best_cost < 0 || cost < best_cost) {
                        best_cost = cost;
                        best_T = T;
                        best_n = n;
                    }
                }
                p.part_tiles = (int)best_T;
                // exactly one workgroup per item: workgroups without an item
                // would still wait for a free slot before they exit
                if (best_n > 0) p.grid = (int)best_n;
            }
        }
    }
    return p;
}

// 256-row work items run the ping-pong kernel, 128-row ones the key-split
// kernel; both are one 8-wave workgroup per CU
template <bool WIN>
static void launch_prefill_win(const PrefillArgs& a, dim3 grid, hipStream_t stream) {
    if (a.rows_per_tile == 256) {
        if (a.head_dim == 128) prefill_pp_kernel<128, WIN><<<grid, dim3(512), 0, stream>>>(a);
        else prefill_pp_kernel<64, WIN><<<grid, dim3(512), 0, stream>>>(a);
    } else {
        if (a.head_dim == 128) prefill_bf16_ks_kernel<128, WIN><<<grid, dim3(512), 0, stream>>>(a);
        else prefill_bf16_ks_kernel<64, WIN><<<grid, dim3(512), 0, stream>>>(a);
    }
}

hipError_t launch_prefill_bf16(const PrefillArgs& a, hipStream_t stream) {
    const long blocks = (long)a.grid + a.next_blocks + a.prev_blocks;
    if (blocks <= 0) return hipSuccess;
    const dim3 grid((unsigned)blocks);
    if (a.window > 0)
        launch_prefill_win<true>(a, grid, stream);
    else
        launch_prefill_win<false>(a, grid, stream);
    return hipGetLastError();
}

MergeArgs merge_args(const PrefillArgs& a) {
    MergeArgs m{};
    m.part = a.part;
    m.table = a.table;
    m.out = a.out;
    m.cu_seq = a.cu_seq;
    m.gate = a.gate;
    m.n_seq = a.n_seq;
    m.n_heads = a.n_heads;
    m.n_kv = a.n_kv;
    m.group = a.group;
    m.max_chunk = a.max_chunk;
    m.n_tok = a.n_tok;
    m.rows_per_tile = a.rows_per_tile;
    m.n_qtiles = a.n_qtiles;
    return m;
}

int merge_blocks_x(const MergeArgs& m, int head_dim) {
    const int rpb = head_dim == 128 ? CombineShape<128>::RPB : CombineShape<64>::RPB;
    return m.n_qtiles * m.n_kv * (m.rows_per_tile / rpb);
}

hipError_t launch_prefill_merge(const MergeArgs& m, int head_dim, hipStream_t stream) {
    if (m.n_seq <= 0) return hipSuccess;
    const dim3 grid((unsigned)merge_blocks_x(m, head_dim), (unsigned)m.n_seq);
    if (head_dim == 128)
        prefill_combine_kernel<128><<<grid, dim3(256), 0, stream>>>(m);
    else
        prefill_combine_kernel<64><<<grid, dim3(256), 0, stream>>>(m);
    return hipGetLastError();
}

hipError_t launch_prefill_combine(const PrefillArgs& a, hipStream_t stream) {
    if (!a.split || a.n_seq <= 0) return hipSuccess;
    return launch_prefill_merge(merge_args(a), a.head_dim, stream);
}

}  // namespace attn
