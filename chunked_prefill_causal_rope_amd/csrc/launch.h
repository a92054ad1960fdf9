// Internal launch interface between the C-ABI layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "device_common.h"

namespace attn {

// Per-head finish (norm + RoPE + rounding) of Q rows, or of K rows into the
// cache with the V rows copied alongside.
struct RopeArgs {
    const void* x;         // rows [n_tok][n_heads][head_dim]
    void* y;               // Q: [n_tok][n_heads][head_dim]; KV: K cache
    const void* v_src;     // KV only: V rows [n_tok][n_heads][head_dim]
    void* v_dst;           // KV only: V cache
    const int32_t* cu_seq;
    const int32_t* start;
    const float* inv_freq;
    const float* norm_w;
    double eps;
    float rope_scale;
    int n_tok, n_heads, head_dim, cap, n_seq, max_chunk, rotary_dim, norm;
    int ring;              // KV: position p in cache row p mod cap (else row p < cap)
    int v_norm;            // KV: V rows scale-less RMS-normalised before the cache
};
hipError_t launch_rope_rows(const RopeArgs& a, int dtype, bool kv, hipStream_t stream);
// Both finishes of a chunk (queries, then keys/values into the cache) in as
// few launches as the layout allows.
hipError_t launch_rope_qkv(const RopeArgs& q, const RopeArgs& kv, int dtype, hipStream_t stream);

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
// The per-token path serves rotary_dim % 8 == 0 at head_dim 64 or 128; its
// arguments for a chunk's queries q and keys/values kv.
bool rope_token_path(const RopeArgs& a);
RopeTokArgs rope_token_args(const RopeArgs& q, const RopeArgs& kv);

// Merge of a split chunk's partials into its output rows: what the merge
// reads (partials, schedule table, batch offsets, gate) and writes (out).
struct MergeArgs {
    const float* part;
    const int* table;
    float* out;
    const int32_t* cu_seq;
    GateRef gate;
    int n_seq, n_heads, n_kv, group, max_chunk, n_tok, rows_per_tile, n_qtiles;
};

// Causal attention of packed chunk rows over the head-major cache.
struct PrefillArgs {
    const void* q;
    const void* k_cache;
    const void* v_cache;
    float* out;
    float* part;           // split calls: partials [item][rows_per_tile][head_dim+4]
    int* table;            // split calls: per (sequence, row tile) first item, part count
    const int32_t* cu_seq;
    const int32_t* start;
    float scale;
    int n_seq, n_heads, n_kv, group, head_dim, cap, n_tok, max_chunk, max_end;
    int window;            // 0: all keys <= p; W: keys p-W+1..p
    int ring;              // key j in cache row j mod cap (needs a window; cap % 64 == 0)
    GateRef gate;          // output gate (mode 0: none)
    // rows per workgroup, row tiles per sequence, split call (persistent
    // grid with device-chosen key-range parts, merged by the combine kernel)
    int rows_per_tile, n_qtiles, split, grid, slots;
    int part_tiles;        // split calls: part length chosen on the host (0: on the device)
    // the next chunk's finish (bf16, per-token path), run by next_blocks
    // workgroups past the attention grid: workgroup grid + r takes token
    // r % next_chunk, head-row block (r / next_chunk) % next_nhb, sequence
    // r / (next_chunk * next_nhb)
    RopeTokArgs next;
    int next_blocks, next_chunk, next_nhb;
    // an earlier split chunk's merge (same head size), run by prev_blocks
    // workgroups past those: each takes two merge blocks of 256 threads,
    // block f = x + prev_gx * sequence
    MergeArgs prev;
    int prev_blocks, prev_gx;
};
// Launch plan of the bf16 prefill, from host scalars only: query rows per
// workgroup (128 or 256), row tiles, whether to split, grid, workspace.
struct PrefillPlan {
    int rows_per_tile, n_qtiles, split, grid, slots, part_tiles;
    size_t ws_bytes, table_bytes;
};
PrefillPlan plan_prefill(int n_seq, int n_heads, int n_kv, int head_dim, int n_tok, int max_chunk,
                         int max_end, int window, size_t ws_available);
hipError_t launch_prefill_bf16(const PrefillArgs& a, hipStream_t stream);
// compute units of the current device (256 if the query fails)
int device_cus();
hipError_t launch_prefill_combine(const PrefillArgs& a, hipStream_t stream);
// the merge of a split chunk on its own launch, and its shape: merge blocks
// per sequence (256 threads each)
MergeArgs merge_args(const PrefillArgs& a);
hipError_t launch_prefill_merge(const MergeArgs& m, int head_dim, hipStream_t stream);
int merge_blocks_x(const MergeArgs& m, int head_dim);

// float32 path (prefill rows and decode rows) -- vector ALU, one wave per row.
struct AttendF32Args {
    const float* q;
    const float* k_cache;
    const float* v_cache;
    float* out;
    float* probs;          // decode only, may be null
    const int32_t* cu_seq; // prefill mode
    const int32_t* start;  // prefill mode
    const int32_t* ctx;    // decode mode
    float scale;
    int decode;
    int n_seq, n_heads, n_kv, group, head_dim, cap, n_tok, max_chunk, max_ctx, probs_ld;
    int window;            // 0: all keys <= p; W: keys p-W+1..p
    int ring;              // key j in cache row j mod cap
    GateRef gate;          // output gate (mode 0: none)
};
hipError_t launch_attend_f32(const AttendF32Args& a, hipStream_t stream);

// bf16 decode: split the key range of each (sequence, KV head), then merge.
struct DecodeArgs {
    const void* q;
    const void* k_cache;
    const void* v_cache;
    float* out;
    float* probs;
    float* part;           // [n_seq*n_heads][n_splits][head_dim+4]
    const int32_t* ctx;
    float scale;
    int n_seq, n_heads, n_kv, group, head_dim, cap, max_ctx, probs_ld;
    int split_len, n_splits;   // parts of split_len keys from the row's first key
    int window;                // 0: all ctx keys; W: the last W
    int ring;                  // key j in cache row j mod cap (needs W <= cap)
    GateRef gate;              // output gate (mode 0: none)
    // A chunk of at most n_q tokens per sequence (a varlen batch, rows packed
    // as for prefill; no probabilities) instead of one query at ctx[b]-1:
    // cu_seq/start non-null, sequence b's queries at start[b] .. start[b] +
    // len_b - 1 attend keys up to their own position.  Decode: null, n_q = 1.
    const int32_t* cu_seq;
    const int32_t* start;
    int n_q;
};
int decode_group_limit();
// Keys one decode row may read, from its part start on: max_ctx, or with a
// window W the W keys plus the alignment of the first part's start.
int decode_key_span(int max_ctx, int window);
// Longest key range one decode part may cover (a multiple of 64).
int decode_part_limit(int group, bool probs);
hipError_t launch_decode_bf16(const DecodeArgs& a, hipStream_t stream);

// attn_decode with its workspace given explicitly (the C entry point and the
// no-allocation variant share it); the smallest workspace it accepts for a
// bf16 call (one part per row).
int decode_impl(const void* q, const void* k_cache, const void* v_cache, int dtype, int n_seq, int n_heads,
                int n_kv, int head_dim, int cap, int ring, const int32_t* ctx, int max_ctx, float scale,
                int window, const void* gate, int gate_mode, int gate_ld, float* out, float* probs,
                int probs_ld, void* workspace, size_t workspace_bytes, void* stream);
size_t decode_min_workspace_bytes(int n_seq, int n_heads, int head_dim);

// Per-position importance of a decode step: sum over heads of the
// probabilities.
struct ImportanceArgs {
    const float* probs;    // [n_seq][n_heads][probs_ld]
    const int32_t* ctx;    // [n_seq]
    float* imp;            // [n_seq][imp_ld]
    int n_seq, n_heads, probs_ld, max_ctx, imp_ld, accumulate;
};
hipError_t launch_decode_importance(const ImportanceArgs& a, hipStream_t stream);

}  // namespace attn
