// C ABI of the library: argument validation, launch geometry, status codes.
// Declared in include/attn.h, which documents every entry point.
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <string.h>

#include <hip/hip_runtime.h>

#include "../../include/attn.h"
#include "launch.h"

// 0: the next chunk's finish always runs as its own launch (timing builds)
#ifndef ATTN_FUSE_NEXT
#define ATTN_FUSE_NEXT 1
#endif

namespace {

// a decode partial row: 4 header floats, then head_dim halves
constexpr int kDecodePartHead = 4;
#ifndef ATTN_DECODE_SPLIT
#define ATTN_DECODE_SPLIT 1024
#endif
constexpr int kDecodeSplit = ATTN_DECODE_SPLIT;   // keys per decode part

bool dtype_ok(int dtype) { return dtype == ATTN_F32 || dtype == ATTN_BF16; }
bool hd_ok(int hd) { return hd == 64 || hd == 128; }

int status_of(hipError_t e) { return e == hipSuccess ? ATTN_OK : ATTN_EDEVICE; }

int check_rope(int dtype, int n_tok, int n_heads, int head_dim, int n_seq, const int32_t* cu_seq,
               const int32_t* start, int max_chunk, const float* inv_freq, int rotary_dim,
               int norm, const float* norm_w) {
    if (!dtype_ok(dtype) || !hd_ok(head_dim)) return ATTN_EUNSUPPORTED;
    if (n_tok < 0 || n_seq < 0 || max_chunk < 0 || n_heads <= 0) return ATTN_EINVAL;
    if (rotary_dim < 0 || (rotary_dim & 1)) return ATTN_EINVAL;
    if (rotary_dim > 0 && !inv_freq) return ATTN_EINVAL;
    if (norm < ATTN_NORM_NONE || norm > ATTN_NORM_1PW) return ATTN_EINVAL;
    if (norm != ATTN_NORM_NONE && !norm_w) return ATTN_EINVAL;
    if (n_seq > 0 && (!cu_seq || !start)) return ATTN_EINVAL;
    if (n_seq > 65535) return ATTN_EINVAL;   // grid z
    return ATTN_OK;
}

// Parts of kDecodeSplit keys, shorter when the group is wide (the kernel
// keeps a part's raw scores on chip; the limit holds with or without
// probabilities so the workspace size never depends on them).
int decode_split_len(int group) {
    const int lim = attn::decode_part_limit(group, true);
    return kDecodeSplit < lim ? kDecodeSplit : lim;
}
int decode_splits_full(int max_ctx, int group) {
    const int len = decode_split_len(group);
    return (max_ctx + len - 1) / len;
}

size_t decode_part_bytes(int n_seq, int n_heads, int head_dim, int splits) {
    return (size_t)n_seq * n_heads * splits * (head_dim / 2 + kDecodePartHead) * sizeof(float);
}

// Chunks of at most kSmallChunk tokens per sequence (a two-position
// speculative verify, a decode step through the prefill call) run on the
// decode kernels: query rows = heads x tokens of a KV group (at most the
// decode group limit), the context split into parts streamed once for all
// of them, instead of row tiles of which a handful of rows would be used.
constexpr int kSmallChunk = 2;
bool small_chunk(int max_chunk, int group) {
    return max_chunk <= kSmallChunk && group * max_chunk <= attn::decode_group_limit();
}
int small_chunk_span(int max_end, int window, int max_chunk) {
    // keys from the first query's window start (rounded down to a step)
    return attn::decode_key_span(max_end, window > 0 ? window + max_chunk - 1 : 0);
}

// Output gate arguments: mode 0 needs nothing; per-element modes read
// head_dim values per row (ld >= head_dim), the per-head mode one (ld >= 1).
bool gate_ok(const void* gate, int mode, int ld, int head_dim) {
    if (mode == attn::kGateNone) return true;
    if (!gate || mode < attn::kGateSigmoid || mode > attn::kGateSoftplus) return false;
    return mode == attn::kGateSoftplusHead ? ld >= 1 : ld >= head_dim;
}

}  // namespace

extern "C" {

const char* attn_version(void) { return "0.1.0"; }

const char* attn_status_string(int status) {
    switch (status) {
        case ATTN_OK: return "ok";
        case ATTN_EINVAL: return "invalid argument";
        case ATTN_ECAPACITY: return "exceeds cache capacity";
        case ATTN_EUNSUPPORTED: return "unsupported configuration";
        case ATTN_EDEVICE: return "device launch failed";
        case ATTN_ESCRATCH: return "exceeds the library's static scratch";
        default: return "unknown status";
    }
}

int attn_rope_inv_freq(int rotary_dim, double base, float* inv_freq) {
    if (rotary_dim <= 0 || (rotary_dim & 1) || !(base > 0.0) || !inv_freq) return ATTN_EINVAL;
    for (int i = 0; i < rotary_dim / 2; ++i)
        inv_freq[i] = (float)(1.0 / pow(base, (double)(2 * i) / (double)rotary_dim));
    return ATTN_OK;
}

int attn_yarn_inv_freq(int rotary_dim, double base, double factor, int orig_max_pos,
                       double beta_fast, double beta_slow, float* inv_freq) {
    if (rotary_dim <= 0 || (rotary_dim & 1) || !(base > 1.0) || !(factor > 0.0) ||
        orig_max_pos <= 0 || !(beta_fast > 0.0) || !(beta_slow > 0.0) || !inv_freq)
        return ATTN_EINVAL;
    const int half = rotary_dim / 2;
    const double two_pi = 6.283185307179586476925286766559;
    auto corr_dim = [&](double rotations) {
        return (double)rotary_dim * log((double)orig_max_pos / (rotations * two_pi)) /
               (2.0 * log(base));
    };
    const double lo_d = fmax(floor(corr_dim(beta_fast)), 0.0);
    const double hi_d = fmin(fmax(ceil(corr_dim(beta_slow)), 0.0), (double)(half - 1));
    const long lo = (long)lo_d;
    const long hi = (long)hi_d;
    const long span = hi > lo ? hi - lo : 0;
    const double denom = (double)(span > 1 ? span : 1);
    for (int i = 0; i < half; ++i) {
        const double f = 1.0 / pow(base, (double)(2 * i) / (double)rotary_dim);
        const double ramp = fmin(fmax((double)(i > lo ? i - lo : 0) / denom, 0.0), 1.0);
        // ramp 0 keeps the original frequency, ramp 1 divides it by factor
        inv_freq[i] = (float)((f / factor) * ramp + f * (1.0 - ramp));
    }
    return ATTN_OK;
}

int attn_rope_apply(const void* x, void* y, int dtype, int n_tok, int n_heads, int head_dim,
                    int n_seq, const int32_t* cu_seq, const int32_t* start, int max_chunk,
                    const float* inv_freq, int rotary_dim, float rope_scale, int norm,
                    const float* norm_w, double eps, void* stream) {
    int st = check_rope(dtype, n_tok, n_heads, head_dim, n_seq, cu_seq, start, max_chunk, inv_freq,
                        rotary_dim, norm, norm_w);
    if (st != ATTN_OK) return st;
    if (n_seq == 0 || n_tok == 0 || max_chunk == 0) return ATTN_OK;
    if (!x || !y) return ATTN_EINVAL;
    attn::RopeArgs a{};
    a.x = x;
    a.y = y;
    a.cu_seq = cu_seq;
    a.start = start;
    a.inv_freq = inv_freq;
    a.norm_w = norm_w;
    a.eps = eps;
    a.rope_scale = rope_scale;
    a.n_tok = n_tok;
    a.n_heads = n_heads;
    a.head_dim = head_dim;
    a.cap = 0;
    a.n_seq = n_seq;
    a.max_chunk = max_chunk;
    a.rotary_dim = rotary_dim < head_dim ? rotary_dim : head_dim;
    a.norm = norm;
    return status_of(attn::launch_rope_rows(a, dtype, false, (hipStream_t)stream));
}

int attn_kv_append(void* k_cache, void* v_cache, int dtype, int n_seq, int n_kv, int head_dim,
                   int cap, int ring, const void* k_new, const void* v_new, int n_tok,
                   const int32_t* cu_seq, const int32_t* start, int max_chunk, int max_end,
                   const float* inv_freq, int rotary_dim, float rope_scale, int norm,
                   const float* norm_w, double eps, int v_norm, void* stream) {
    int st = check_rope(dtype, n_tok, n_kv, head_dim, n_seq, cu_seq, start, max_chunk, inv_freq,
                        rotary_dim, norm, norm_w);
    if (st != ATTN_OK) return st;
    if (cap <= 0 || max_end < 0 || (ring != 0 && ring != 1) || (v_norm != 0 && v_norm != 1))
        return ATTN_EINVAL;
    if (!ring && max_end > cap) return ATTN_ECAPACITY;
    // a wrapped ring gives two positions of one chunk, p and p + cap, the
    // same row when the chunk is longer than the ring
    if (ring && max_end > cap && max_chunk > cap) return ATTN_ECAPACITY;
    if (n_seq == 0 || n_tok == 0 || max_chunk == 0) return ATTN_OK;
    if (!k_cache || !v_cache || !k_new || !v_new) return ATTN_EINVAL;
    attn::RopeArgs a{};
    a.x = k_new;
    a.y = k_cache;
    a.v_src = v_new;
    a.v_dst = v_cache;
    a.cu_seq = cu_seq;
    a.start = start;
    a.inv_freq = inv_freq;
    a.norm_w = norm_w;
    a.eps = eps;
    a.rope_scale = rope_scale;
    a.n_tok = n_tok;
    a.n_heads = n_kv;
    a.head_dim = head_dim;
    a.cap = cap;
    a.ring = ring && max_end > cap;
    a.v_norm = v_norm;
    a.n_seq = n_seq;
    a.max_chunk = max_chunk;
    a.rotary_dim = rotary_dim < head_dim ? rotary_dim : head_dim;
    a.norm = norm;
    return status_of(attn::launch_rope_rows(a, dtype, true, (hipStream_t)stream));
}

}  // extern "C"

namespace {

// Validation and launch arguments of attn_rope_qkv; *empty when the call has
// no work (and nothing to launch).
int rope_qkv_build(const void* q, void* q_out, int n_heads, void* k_cache, void* v_cache,
                   const void* k_new, const void* v_new, int n_kv, int cap, int ring, int dtype, int n_tok,
                   int head_dim, int n_seq, const int32_t* cu_seq, const int32_t* start, int max_chunk,
                   int max_end, const float* inv_freq, int rotary_dim, float rope_scale, int norm,
                   const float* q_norm_w, const float* k_norm_w, double eps, int v_norm,
                   attn::RopeArgs& aq, attn::RopeArgs& ak, bool& empty) {
    empty = true;
    int st = check_rope(dtype, n_tok, n_heads, head_dim, n_seq, cu_seq, start, max_chunk, inv_freq,
                        rotary_dim, norm, q_norm_w);
    if (st != ATTN_OK) return st;
    st = check_rope(dtype, n_tok, n_kv, head_dim, n_seq, cu_seq, start, max_chunk, inv_freq,
                    rotary_dim, norm, k_norm_w);
    if (st != ATTN_OK) return st;
    if (cap <= 0 || max_end < 0 || (ring != 0 && ring != 1) || (v_norm != 0 && v_norm != 1))
        return ATTN_EINVAL;
    if (!ring && max_end > cap) return ATTN_ECAPACITY;
    if (ring && max_end > cap && max_chunk > cap) return ATTN_ECAPACITY;   // as attn_kv_append
    if (n_seq == 0 || n_tok == 0 || max_chunk == 0) return ATTN_OK;
    if (!q || !q_out || !k_cache || !v_cache || !k_new || !v_new) return ATTN_EINVAL;
    empty = false;
    aq = attn::RopeArgs{};
    aq.x = q;
    aq.y = q_out;
    aq.norm_w = q_norm_w;
    aq.n_heads = n_heads;
    aq.cap = 0;
    ak = attn::RopeArgs{};
    ak.x = k_new;
    ak.y = k_cache;
    ak.v_src = v_new;
    ak.v_dst = v_cache;
    ak.norm_w = k_norm_w;
    ak.n_heads = n_kv;
    ak.cap = cap;
    ak.ring = ring && max_end > cap;
    ak.v_norm = v_norm;
    for (attn::RopeArgs* a : {&aq, &ak}) {
        a->cu_seq = cu_seq;
        a->start = start;
        a->inv_freq = inv_freq;
        a->eps = eps;
        a->rope_scale = rope_scale;
        a->n_tok = n_tok;
        a->head_dim = head_dim;
        a->n_seq = n_seq;
        a->max_chunk = max_chunk;
        a->rotary_dim = rotary_dim < head_dim ? rotary_dim : head_dim;
        a->norm = norm;
    }
    return ATTN_OK;
}

// The next chunk's finish, when it rides in a prefill launch.
struct NextFinish {
    const attn::RopeArgs* q;
    const attn::RopeArgs* kv;
    int dtype;
};

// What a pending record holds: the merge a split chunk still owes, and the
// workspace bytes its partials occupy until then.
struct PendingState {
    attn::MergeArgs m;
    const char* ws_lo;
    const char* ws_hi;
};
constexpr int kPendingWords = sizeof(((attn_prefill_pending*)nullptr)->state) / sizeof(uint64_t);
static_assert(sizeof(PendingState) <= sizeof(uint64_t) * (kPendingWords - 1),
              "pending state fits the record beside its check word");

// The record's last word checks the rest (FNV-1a over head_dim and the state
// words), so a record the library did not write -- uninitialised memory with
// active set -- is refused instead of launching a merge on stray pointers.
uint64_t pending_check(const attn_prefill_pending& r) {
    uint64_t h = 1469598103934665603ull;
    auto mix = [&](uint64_t w) {
        for (int i = 0; i < 8; ++i) {
            h ^= (w >> (8 * i)) & 0xffu;
            h *= 1099511628211ull;
        }
    };
    mix((uint64_t)(uint32_t)r.head_dim);
    for (int i = 0; i < kPendingWords - 1; ++i) mix(r.state[i]);
    return h;
}
void pending_write(attn_prefill_pending* r, int head_dim, const PendingState& st) {
    memset(r->state, 0, sizeof(r->state));
    memcpy(r->state, &st, sizeof(st));
    r->head_dim = head_dim;
    r->state[kPendingWords - 1] = pending_check(*r);
    r->active = 1;
}
// a record the library wrote and that owes a merge: its state in *st
bool pending_read(const attn_prefill_pending& r, PendingState* st) {
    if (r.active != 1 || !hd_ok(r.head_dim) || r.state[kPendingWords - 1] != pending_check(r)) return false;
    memcpy(st, r.state, sizeof(*st));
    return true;
}

// An earlier chunk's merge to run in this call, and where to leave this
// chunk's own (deferred mode when `pending` is set).
struct MergeDefer {
    const PendingState* prev;     // null: none owed
    int prev_hd;
    attn_prefill_pending* pending;
};

int prefill_chunk_impl(const void* q, const void* k_cache, const void* v_cache, int dtype,
                       int n_seq, int n_heads, int n_kv, int head_dim, int cap, int ring, int n_tok,
                       const int32_t* cu_seq, const int32_t* start, int max_chunk, int max_end,
                       float scale, int window, const void* gate, int gate_mode, int gate_ld,
                       float* out, void* workspace, size_t workspace_bytes, const NextFinish* next,
                       const MergeDefer* defer, hipStream_t s);

}  // namespace

extern "C" {

int attn_rope_qkv(const void* q, void* q_out, int n_heads, void* k_cache, void* v_cache,
                  const void* k_new, const void* v_new, int n_kv, int cap, int ring, int dtype, int n_tok,
                  int head_dim, int n_seq, const int32_t* cu_seq, const int32_t* start, int max_chunk,
                  int max_end, const float* inv_freq, int rotary_dim, float rope_scale, int norm,
                  const float* q_norm_w, const float* k_norm_w, double eps, int v_norm,
                  void* stream) {
    attn::RopeArgs aq, ak;
    bool empty;
    const int st = rope_qkv_build(q, q_out, n_heads, k_cache, v_cache, k_new, v_new, n_kv, cap, ring, dtype,
                                  n_tok, head_dim, n_seq, cu_seq, start, max_chunk, max_end, inv_freq,
                                  rotary_dim, rope_scale, norm, q_norm_w, k_norm_w, eps, v_norm, aq, ak, empty);
    if (st != ATTN_OK || empty) return st;
    return status_of(attn::launch_rope_qkv(aq, ak, dtype, (hipStream_t)stream));
}

size_t attn_prefill_workspace_bytes(int n_seq, int n_heads, int n_kv, int head_dim, int n_tok,
                                    int max_chunk, int max_end) {
    if (n_seq <= 0 || n_heads <= 0 || n_kv <= 0 || n_heads % n_kv || n_tok <= 0 || max_chunk <= 0 ||
        max_end <= 0 || !hd_ok(head_dim))
        return 0;
    size_t ws = attn::plan_prefill(n_seq, n_heads, n_kv, head_dim, n_tok, max_chunk, max_end, 0,
                                   (size_t)-1).ws_bytes;
    if (small_chunk(max_chunk, n_heads / n_kv)) {
        const int splits = decode_splits_full(small_chunk_span(max_end, 0, max_chunk), n_heads / n_kv * max_chunk);
        const size_t need = decode_part_bytes(n_seq * max_chunk, n_heads, head_dim, splits);
        if (need > ws) ws = need;
    }
    return ws;
}

int attn_prefill_chunk(const void* q, const void* k_cache, const void* v_cache, int dtype,
                       int n_seq, int n_heads, int n_kv, int head_dim, int cap, int ring, int n_tok,
                       const int32_t* cu_seq, const int32_t* start, int max_chunk, int max_end,
                       float scale, int window, const void* gate, int gate_mode, int gate_ld,
                       float* out, void* workspace, size_t workspace_bytes, void* stream) {
    return prefill_chunk_impl(q, k_cache, v_cache, dtype, n_seq, n_heads, n_kv, head_dim, cap, ring, n_tok,
                              cu_seq, start, max_chunk, max_end, scale, window, gate, gate_mode, gate_ld, out,
                              workspace, workspace_bytes, nullptr, nullptr, (hipStream_t)stream);
}

int attn_prefill_chunk_rope_next(const void* q, const void* k_cache, const void* v_cache, int dtype,
                                 int n_seq, int n_heads, int n_kv, int head_dim, int cap, int ring, int n_tok,
                                 const int32_t* cu_seq, const int32_t* start, int max_chunk, int max_end,
                                 float scale, int window, const void* gate, int gate_mode, int gate_ld,
                                 float* out, void* workspace, size_t workspace_bytes,
                                 const attn_rope_qkv_args* next, void* stream) {
    if (!next) return ATTN_EINVAL;
    attn::RopeArgs aq, ak;
    bool empty;
    const int st = rope_qkv_build(next->q, next->q_out, next->n_heads, next->k_cache, next->v_cache, next->k_new,
                                  next->v_new, next->n_kv, next->cap, next->ring, next->dtype, next->n_tok,
                                  next->head_dim, next->n_seq, next->cu_seq, next->start, next->max_chunk,
                                  next->max_end, next->inv_freq, next->rotary_dim, next->rope_scale, next->norm,
                                  next->q_norm_w, next->k_norm_w, next->eps, next->v_norm, aq, ak, empty);
    if (st != ATTN_OK) return st;
    const NextFinish nf{&aq, &ak, next->dtype};
    return prefill_chunk_impl(q, k_cache, v_cache, dtype, n_seq, n_heads, n_kv, head_dim, cap, ring, n_tok,
                              cu_seq, start, max_chunk, max_end, scale, window, gate, gate_mode, gate_ld, out,
                              workspace, workspace_bytes, empty ? nullptr : &nf, nullptr, (hipStream_t)stream);
}

int attn_prefill_chunk_deferred(const void* q, const void* k_cache, const void* v_cache, int dtype,
                                int n_seq, int n_heads, int n_kv, int head_dim, int cap, int ring, int n_tok,
                                const int32_t* cu_seq, const int32_t* start, int max_chunk, int max_end,
                                float scale, int window, const void* gate, int gate_mode, int gate_ld,
                                float* out, void* workspace, size_t workspace_bytes,
                                const attn_rope_qkv_args* next, const attn_prefill_pending* prev,
                                attn_prefill_pending* pending, void* stream) {
    if (!pending) return ATTN_EINVAL;
    // prev may be the record this call rewrites: take its state first
    PendingState pv{};
    MergeDefer d{nullptr, 0, pending};
    if (prev && prev->active) {
        if (!pending_read(*prev, &pv)) return ATTN_EINVAL;
        d.prev = &pv;
        d.prev_hd = prev->head_dim;
    }
    attn::RopeArgs aq, ak;
    bool empty = true;
    if (next) {
        const int st = rope_qkv_build(next->q, next->q_out, next->n_heads, next->k_cache, next->v_cache,
                                      next->k_new, next->v_new, next->n_kv, next->cap, next->ring, next->dtype,
                                      next->n_tok, next->head_dim, next->n_seq, next->cu_seq, next->start,
                                      next->max_chunk, next->max_end, next->inv_freq, next->rotary_dim,
                                      next->rope_scale, next->norm, next->q_norm_w, next->k_norm_w, next->eps,
                                      next->v_norm, aq, ak, empty);
        if (st != ATTN_OK) return st;
    }
    const NextFinish nf{&aq, &ak, next ? next->dtype : 0};
    return prefill_chunk_impl(q, k_cache, v_cache, dtype, n_seq, n_heads, n_kv, head_dim, cap, ring, n_tok,
                              cu_seq, start, max_chunk, max_end, scale, window, gate, gate_mode, gate_ld, out,
                              workspace, workspace_bytes, next && !empty ? &nf : nullptr, &d, (hipStream_t)stream);
}

int attn_prefill_finish(const attn_prefill_pending* pending, void* stream) {
    if (!pending) return ATTN_EINVAL;
    if (!pending->active) return ATTN_OK;
    PendingState pv;
    if (!pending_read(*pending, &pv)) return ATTN_EINVAL;
    return status_of(attn::launch_prefill_merge(pv.m, pending->head_dim, (hipStream_t)stream));
}

size_t attn_decode_workspace_bytes(int n_seq, int n_heads, int n_kv, int head_dim, int max_ctx) {
    if (n_seq <= 0 || n_heads <= 0 || n_kv <= 0 || n_heads % n_kv || max_ctx <= 0 ||
        !hd_ok(head_dim))
        return 0;
    return decode_part_bytes(n_seq, n_heads, head_dim, decode_splits_full(max_ctx, n_heads / n_kv));
}

}  // extern "C"

namespace {

// Byte ranges [p, p + n) that share a byte.
bool overlap(const void* a, size_t na, const void* b, size_t nb) {
    if (!a || !b || !na || !nb) return false;
    const char* x = static_cast<const char*>(a);
    const char* y = static_cast<const char*>(b);
    return x < y + nb && y < x + na;
}

// The work of one pipelined call that may run concurrently -- this chunk's
// attention, the next chunk's finish and an earlier chunk's merge -- touches
// disjoint rows outside the caches: no buffer one of them writes overlaps a
// buffer another one reads or writes.  The cache rows are the caller's
// chunk-order precondition.
bool pipeline_disjoint(const void* q, int dtype, int n_tok, int n_heads, int head_dim, const void* gate,
                       int gate_ld, const float* out, const void* workspace, size_t workspace_bytes,
                       const NextFinish* next, const PendingState* pv, int prev_hd) {
    if (!next && !pv) return true;
    const size_t esz = dtype == ATTN_BF16 ? 2 : 4;
    const size_t rows = (size_t)(n_tok > 0 ? n_tok : 0) * (size_t)n_heads;
    struct Span {
        const void* p;
        size_t n;
    };
    // this chunk: read (q, gate) and written (out, workspace)
    const Span q_in{q, rows * head_dim * esz};
    const Span g_in{gate, gate && rows ? ((rows - 1) * (size_t)gate_ld + head_dim) * esz : 0};
    const Span o_w{out, rows * head_dim * sizeof(float)};
    const Span ws_w{workspace, workspace ? workspace_bytes : 0};
    const Span mine[] = {q_in, g_in, o_w, ws_w};
    auto hits = [&](const Span& x, const Span* set, int n) {
        for (int i = 0; i < n; ++i)
            if (overlap(x.p, x.n, set[i].p, set[i].n)) return true;
        return false;
    };
    Span nx_w{nullptr, 0}, nx_in[3] = {};
    if (next) {
        const size_t ne = next->dtype == ATTN_BF16 ? 2 : 4;
        const attn::RopeArgs& a = *next->q;
        const attn::RopeArgs& k = *next->kv;
        nx_w = {a.y, (size_t)a.n_tok * a.n_heads * a.head_dim * ne};
        nx_in[0] = {a.x, (size_t)a.n_tok * a.n_heads * a.head_dim * ne};
        nx_in[1] = {k.x, (size_t)k.n_tok * k.n_heads * k.head_dim * ne};
        nx_in[2] = {k.v_src, (size_t)k.n_tok * k.n_heads * k.head_dim * ne};
        // its query rows are written while this chunk reads and writes its own
        if (hits(nx_w, mine, 4)) return false;
        // this chunk's writes against what it reads
        if (hits(o_w, nx_in, 3) || hits(ws_w, nx_in, 3)) return false;
    }
    if (pv) {
        // the earlier chunk's output rows, written by its merge
        const Span pw{pv->m.out, (size_t)pv->m.n_tok * pv->m.n_heads * prev_hd * sizeof(float)};
        if (hits(pw, mine, 4) || hits(pw, nx_in, 3) || overlap(pw.p, pw.n, nx_w.p, nx_w.n)) return false;
    }
    return true;
}

int prefill_chunk_impl(const void* q, const void* k_cache, const void* v_cache, int dtype,
                       int n_seq, int n_heads, int n_kv, int head_dim, int cap, int ring, int n_tok,
                       const int32_t* cu_seq, const int32_t* start, int max_chunk, int max_end,
                       float scale, int window, const void* gate, int gate_mode, int gate_ld,
                       float* out, void* workspace, size_t workspace_bytes, const NextFinish* next,
                       const MergeDefer* defer, hipStream_t s) {
    if (!dtype_ok(dtype) || !hd_ok(head_dim)) return ATTN_EUNSUPPORTED;
    if (n_seq < 0 || n_tok < 0 || max_chunk < 0 || max_end < 0 || n_heads <= 0 || n_kv <= 0 ||
        cap <= 0 || n_heads % n_kv != 0 || !isfinite(scale) || window < 0 || (ring != 0 && ring != 1))
        return ATTN_EINVAL;
    // A ring that has wrapped still holds every key the chunk reads only if
    // the window plus the chunk's other rows fit in it (the chunk is written
    // before it attends).  Until it wraps it is a plain cache.
    const bool wrapped = ring && max_end > cap;
    if (!wrapped && max_end > cap) return ATTN_ECAPACITY;
    if (wrapped && (window <= 0 || (long)window + max_chunk - 1 > cap)) return ATTN_ECAPACITY;
    if (wrapped && dtype == ATTN_BF16 && cap % 64 != 0) return ATTN_EUNSUPPORTED;
    if (!gate_ok(gate, gate_mode, gate_ld, head_dim)) return ATTN_EINVAL;
    // an earlier chunk's partials stay in its workspace until its merge runs
    const PendingState* pv = defer ? defer->prev : nullptr;
    if (pv && workspace && workspace_bytes && (const char*)workspace < pv->ws_hi &&
        pv->ws_lo < (const char*)workspace + workspace_bytes)
        return ATTN_EINVAL;
    if (!pipeline_disjoint(q, dtype, n_tok, n_heads, head_dim, gate, gate_ld, out, workspace, workspace_bytes,
                           next, pv, defer ? defer->prev_hd : 0))
        return ATTN_EINVAL;
    // after validation, nothing but the launches can fail: the next chunk's
    // finish runs after this chunk's attention unless it rides in its launch
    auto finish_next = [&](hipError_t e) {
        if (e == hipSuccess && next) e = attn::launch_rope_qkv(*next->q, *next->kv, next->dtype, s);
        return status_of(e);
    };
    // deferred mode: the earlier chunk's merge on a launch of its own (when it
    // does not ride in this chunk's attention launch), and this chunk's record
    auto prev_alone = [&]() { return pv ? attn::launch_prefill_merge(pv->m, defer->prev_hd, s) : hipSuccess; };
    auto owe_nothing = [&]() {
        if (defer) {
            defer->pending->active = 0;
            defer->pending->head_dim = head_dim;
        }
    };
    if (n_seq == 0 || n_tok == 0 || max_chunk == 0) {
        owe_nothing();
        return finish_next(prev_alone());
    }
    const attn::GateRef gref{gate, gate_mode, gate_ld, dtype == ATTN_BF16};
    if (!q || !k_cache || !v_cache || !out || !cu_seq || !start) return ATTN_EINVAL;
    if (n_seq > 65535) return ATTN_EINVAL;
    const int group = n_heads / n_kv;
    if (dtype == ATTN_F32) {
        attn::AttendF32Args a{};
        a.q = (const float*)q;
        a.k_cache = (const float*)k_cache;
        a.v_cache = (const float*)v_cache;
        a.out = out;
        a.cu_seq = cu_seq;
        a.start = start;
        a.scale = scale;
        a.decode = 0;
        a.n_seq = n_seq;
        a.n_heads = n_heads;
        a.n_kv = n_kv;
        a.group = group;
        a.head_dim = head_dim;
        a.cap = cap;
        a.n_tok = n_tok;
        a.max_chunk = max_chunk;
        a.window = window;
        a.ring = wrapped;
        a.gate = gref;
        owe_nothing();
        hipError_t e = prev_alone();
        if (e == hipSuccess) e = attn::launch_attend_f32(a, s);
        return finish_next(e);
    }
    if (small_chunk(max_chunk, group) && workspace &&
        workspace_bytes >= decode_part_bytes(n_seq * max_chunk, n_heads, head_dim, 1)) {
        const int span = small_chunk_span(max_end, window, max_chunk);
        int splits = decode_splits_full(span, group * max_chunk);
        const size_t fit = workspace_bytes / decode_part_bytes(n_seq * max_chunk, n_heads, head_dim, 1);
        if ((size_t)splits > fit) splits = (int)fit;
        int split_len = (span + splits - 1) / splits;
        split_len = (split_len + 63) / 64 * 64;
        splits = (span + split_len - 1) / split_len;
        if ((long)n_seq * splits * n_kv > 0x7fffffffL) return ATTN_EINVAL;
        attn::DecodeArgs d{};
        d.q = q;
        d.k_cache = k_cache;
        d.v_cache = v_cache;
        d.out = out;
        d.probs = nullptr;
        d.part = (float*)workspace;
        d.ctx = nullptr;
        d.scale = scale;
        d.n_seq = n_seq;
        d.n_heads = n_heads;
        d.n_kv = n_kv;
        d.group = group;
        d.head_dim = head_dim;
        d.cap = cap;
        d.max_ctx = max_end;
        d.probs_ld = 0;
        d.split_len = split_len;
        d.n_splits = splits;
        d.window = window;
        d.ring = wrapped;
        d.gate = gref;
        d.cu_seq = cu_seq;
        d.start = start;
        d.n_q = max_chunk;
        owe_nothing();
        hipError_t e = prev_alone();
        if (e == hipSuccess) e = attn::launch_decode_bf16(d, s);
        return finish_next(e);
    }
    attn::PrefillArgs a{};
    a.q = q;
    a.k_cache = k_cache;
    a.v_cache = v_cache;
    a.out = out;
    a.cu_seq = cu_seq;
    a.start = start;
    a.scale = scale;
    a.n_seq = n_seq;
    a.n_heads = n_heads;
    a.n_kv = n_kv;
    a.group = group;
    a.head_dim = head_dim;
    a.cap = cap;
    a.n_tok = n_tok;
    a.max_chunk = max_chunk;
    a.max_end = max_end;
    a.window = window;
    a.ring = wrapped;
    a.gate = gref;
    const attn::PrefillPlan plan = attn::plan_prefill(n_seq, n_heads, n_kv, head_dim, n_tok,
                                                      max_chunk, max_end, window,
                                                      workspace ? workspace_bytes : 0);
    a.rows_per_tile = plan.rows_per_tile;
    a.n_qtiles = plan.n_qtiles;
    a.split = plan.split;
    a.grid = plan.grid;
    a.slots = plan.slots;
    a.part_tiles = plan.part_tiles;
    a.table = plan.split ? (int*)workspace : nullptr;
    a.part = plan.split ? (float*)((char*)workspace + plan.table_bytes) : nullptr;
    const long blocks = (long)n_seq * a.n_qtiles * n_kv;
    if (blocks > 0x7fffffffL) return ATTN_EINVAL;
    // the next chunk's finish rides in this launch on the per-token path
    // (bf16, the same head size, neither cache wrapped): one workgroup of 512
    // threads per (token, block of 512 / (head_dim / 8) head rows, sequence).
    // Those workgroups carry the attention kernel's registers and LDS, one per
    // CU, so only a finish that fits one such wave rides along (measured: a
    // 128-token chunk of 40 heads, 256 workgroups, gains 10 % per step; 2048 or
    // 4096 of them lose 1-3 % against the standalone launch's small workgroups)
    bool fuse = ATTN_FUSE_NEXT && next && next->dtype == ATTN_BF16 && next->q->head_dim == head_dim &&
                attn::rope_token_path(*next->q) && !next->kv->ring && !wrapped;
    if (fuse) {
        const int nhb_rows = 512 / (head_dim / 8);
        const int nhb = (next->q->n_heads + next->kv->n_heads + nhb_rows - 1) / nhb_rows;
        const long nb = (long)next->q->max_chunk * nhb * next->q->n_seq;
        fuse = nb <= attn::device_cus();
        if (fuse) {
            a.next = attn::rope_token_args(*next->q, *next->kv);
            a.next_chunk = next->q->max_chunk;
            a.next_nhb = nhb;
            a.next_blocks = (int)nb;
        }
    }
    // an earlier chunk's merge of the same head size rides in this launch when
    // it needs at most half the CUs' worth of workgroups: there it takes the
    // attention kernel's footprint, one workgroup of two merge blocks per CU,
    // where its own launch runs eight blocks per CU (measured: 128 merge
    // workgroups per call gain 3-5 % per step, 2560 lose 2 %)
    bool ride = pv && defer->prev_hd == head_dim;
    if (ride) {
        const int gx = attn::merge_blocks_x(pv->m, head_dim);
        const long nb = ((long)gx * pv->m.n_seq + 1) / 2;
        ride = nb <= attn::device_cus() / 2;
        if (ride) {
            a.prev = pv->m;
            a.prev_gx = gx;
            a.prev_blocks = (int)nb;
        }
    }
    hipError_t e = ride ? hipSuccess : prev_alone();
    if (e == hipSuccess) e = attn::launch_prefill_bf16(a, s);
    if (defer) {
        // this chunk's merge is owed to a later launch
        owe_nothing();
        if (plan.split) {
            const PendingState st{attn::merge_args(a), (const char*)workspace,
                                  (const char*)workspace + plan.ws_bytes};
            pending_write(defer->pending, head_dim, st);
        }
    } else if (e == hipSuccess && plan.split) {
        e = attn::launch_prefill_combine(a, s);
    }
    return fuse ? status_of(e) : finish_next(e);
}

}  // namespace

namespace attn {

int decode_impl(const void* q, const void* k_cache, const void* v_cache, int dtype, int n_seq,
                int n_heads, int n_kv, int head_dim, int cap, int ring, const int32_t* ctx,
                int max_ctx, float scale, int window, const void* gate, int gate_mode, int gate_ld,
                float* out, float* probs, int probs_ld, void* workspace,
                size_t workspace_bytes, void* stream) {
    if (!dtype_ok(dtype) || !hd_ok(head_dim)) return ATTN_EUNSUPPORTED;
    if (n_seq < 0 || max_ctx < 0 || n_heads <= 0 || n_kv <= 0 || cap <= 0 ||
        n_heads % n_kv != 0 || !isfinite(scale) || window < 0 || (ring != 0 && ring != 1))
        return ATTN_EINVAL;
    // a wrapped ring holds the last cap keys: enough for a window of at most cap
    const bool wrapped = ring && max_ctx > cap;
    if (!wrapped && max_ctx > cap) return ATTN_ECAPACITY;
    if (wrapped && (window <= 0 || window > cap)) return ATTN_ECAPACITY;
    if (!gate_ok(gate, gate_mode, gate_ld, head_dim)) return ATTN_EINVAL;
    const attn::GateRef gref{gate, gate_mode, gate_ld, dtype == ATTN_BF16};
    if (n_seq == 0 || max_ctx == 0) return ATTN_OK;
    if (!q || !k_cache || !v_cache || !out || !ctx) return ATTN_EINVAL;
    if (probs && probs_ld < max_ctx) return ATTN_EINVAL;
    hipStream_t s = (hipStream_t)stream;
    const int group = n_heads / n_kv;
    if (dtype == ATTN_F32) {
        attn::AttendF32Args a{};
        a.q = (const float*)q;
        a.k_cache = (const float*)k_cache;
        a.v_cache = (const float*)v_cache;
        a.out = out;
        a.probs = probs;
        a.ctx = ctx;
        a.scale = scale;
        a.decode = 1;
        a.n_seq = n_seq;
        a.n_heads = n_heads;
        a.n_kv = n_kv;
        a.group = group;
        a.head_dim = head_dim;
        a.cap = cap;
        a.n_tok = n_seq;
        a.max_ctx = max_ctx;
        a.probs_ld = probs_ld;
        a.window = window;
        a.ring = wrapped;
        a.gate = gref;
        return status_of(attn::launch_attend_f32(a, s));
    }
    if (group > attn::decode_group_limit()) return ATTN_EUNSUPPORTED;
    const size_t per = decode_part_bytes(n_seq, n_heads, head_dim, 1);
    if (!workspace || workspace_bytes < per) return ATTN_EINVAL;
    // a window bounds the keys any row reads
    const int span = attn::decode_key_span(max_ctx, window);
    int splits = decode_splits_full(span, group);
    const size_t fit = workspace_bytes / per;
    if ((size_t)splits > fit) splits = (int)fit;
    int split_len = (span + splits - 1) / splits;
    split_len = (split_len + 63) / 64 * 64;
    splits = (span + split_len - 1) / split_len;
    attn::DecodeArgs a{};
    a.q = q;
    a.k_cache = k_cache;
    a.v_cache = v_cache;
    a.out = out;
    a.probs = probs;
    a.part = (float*)workspace;
    a.ctx = ctx;
    a.scale = scale;
    a.n_seq = n_seq;
    a.n_heads = n_heads;
    a.n_kv = n_kv;
    a.group = group;
    a.head_dim = head_dim;
    a.cap = cap;
    a.max_ctx = max_ctx;
    a.probs_ld = probs ? probs_ld : 0;
    a.split_len = split_len;
    a.n_splits = splits;
    a.window = window;
    a.ring = wrapped;
    a.gate = gref;
    a.n_q = 1;
    if ((long)n_seq * splits * n_kv > 0x7fffffffL) return ATTN_EINVAL;
    return status_of(attn::launch_decode_bf16(a, s));
}

size_t decode_min_workspace_bytes(int n_seq, int n_heads, int head_dim) {
    return decode_part_bytes(n_seq, n_heads, head_dim, 1);
}

}  // namespace attn

extern "C" {

int attn_decode(const void* q, const void* k_cache, const void* v_cache, int dtype, int n_seq,
                int n_heads, int n_kv, int head_dim, int cap, int ring, const int32_t* ctx,
                int max_ctx, float scale, int window, const void* gate, int gate_mode, int gate_ld,
                float* out, float* probs, int probs_ld, void* workspace,
                size_t workspace_bytes, void* stream) {
    return attn::decode_impl(q, k_cache, v_cache, dtype, n_seq, n_heads, n_kv, head_dim, cap, ring, ctx,
                             max_ctx, scale, window, gate, gate_mode, gate_ld, out, probs, probs_ld,
                             workspace, workspace_bytes, stream);
}

int attn_decode_importance(const float* probs, int n_seq, int n_heads, int probs_ld,
                           const int32_t* ctx, int max_ctx, float* imp, int imp_ld, int accumulate,
                           void* stream) {
    if (n_seq < 0 || n_heads <= 0 || max_ctx < 0) return ATTN_EINVAL;
    if (n_seq == 0 || max_ctx == 0) return ATTN_OK;
    if (!probs || !ctx || !imp || probs_ld < max_ctx || imp_ld < max_ctx) return ATTN_EINVAL;
    attn::ImportanceArgs a{};
    a.probs = probs;
    a.ctx = ctx;
    a.imp = imp;
    a.n_seq = n_seq;
    a.n_heads = n_heads;
    a.probs_ld = probs_ld;
    a.max_ctx = max_ctx;
    a.imp_ld = imp_ld;
    a.accumulate = accumulate ? 1 : 0;
    return status_of(attn::launch_decode_importance(a, (hipStream_t)stream));
}

}  // extern "C"
