/*
 * attn.h -- C ABI of the MI355X (gfx950) library for causal grouped-query
 * attention with RoPE over a head-major KV cache.
 *
 * Sources (page title, then the item on it):
 *   [ATT] cortiq-engine 0.5.39, src/attention.rs
 *   [NDL] needle-core 0.3.1, src/v2/batch.rs
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Pointers marked "device" are HIP device pointers; "host" pointers are
 *   ordinary host memory.  The caller owns every buffer; the library allocates
 *   nothing, keeps no global mutable state and enqueues work only on `stream`
 *   (a hipStream_t passed as void*; NULL is the default stream).  Calls return
 *   as soon as the work is enqueued.
 * - dtype: ATTN_F32 or ATTN_BF16.  It is the element type of the raw and
 *   rotated Q, of the new K/V rows and of the K/V cache.  Attention outputs
 *   and probabilities are always float32.
 * - Varlen batch descriptor (prefill, RoPE, append): n_seq sequences whose
 *   tokens are packed back to back in token-major tensors of n_tok rows.
 *   cu_seq [n_seq+1] (device, int32) gives each sequence's first packed row;
 *   start [n_seq] (device, int32) gives the absolute position of that row
 *   ([ATT] fn qwen_attention_batch: the position a call is configured with is
 *   where its chunk starts).  Token i of sequence b is packed row
 *   cu_seq[b]+i at position start[b]+i.  max_chunk (host) bounds every
 *   sequence's token count; max_end (host) bounds every start[b]+len_b.  The
 *   host checks sizes from these host scalars; the device arrays are trusted
 *   to agree with them, and kernels skip any row outside [0, n_tok) or any
 *   position outside [0, cap) (below 0 with a ring) so a disagreeing array
 *   can never write out of bounds.
 * - Ring cache (ring = 1, on the calls that take `ring`): position p lives in
 *   cache row p mod cap, overwriting position p - cap ([NDL] the per-chunk
 *   loop keeps a ring of window positions: writing p+1 overwrites the slot of
 *   p+1-window).  The pages write and attend one position at a time over a
 *   ring of exactly the window; here a chunk is written whole before it
 *   attends, which reads the same keys when cap >= window + max_chunk - 1 --
 *   the attention calls check that bound.  While every position is below cap
 *   a ring is an ordinary cache.  ring = 0: row p, p < cap.
 * - Layouts (row-major, innermost last):
 *     Q, output            [n_tok][n_heads][head_dim]
 *     new K, new V         [n_tok][n_kv][head_dim]
 *     K cache, V cache     [n_seq][n_kv][cap][head_dim]  (head-major: each
 *                          KV head's rows are one contiguous [cap][head_dim]
 *                          slice, [ATT] fn multi_head_attention notes)
 *   Query head h reads KV head h / (n_heads / n_kv) ([ATT] fn
 *   multi_head_attention, fn attend_all_heads).
 * - Errors: every call returns an attn_status; nothing else crosses the ABI.
 *   Empty work (n_seq == 0, n_tok == 0 or max_chunk == 0) returns ATTN_OK and
 *   launches nothing.  There is no fallback path: a configuration without a
 *   kernel returns ATTN_EUNSUPPORTED.
 */
#ifndef ATTN_H
#define ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { ATTN_F32 = 0, ATTN_BF16 = 1 } attn_dtype;

typedef enum {
    ATTN_OK = 0,
    ATTN_EINVAL = -1,      /* bad argument: null pointer, non-positive size,
                              n_heads % n_kv != 0, odd rotary_dim, ... */
    ATTN_ECAPACITY = -2,   /* max_end (or max_ctx) exceeds the cache capacity */
    ATTN_EUNSUPPORTED = -3,/* head_dim not 64/128, unknown dtype, or a GQA
                              group wider than the kernel supports */
    ATTN_EDEVICE = -4,     /* a HIP launch failed (hipGetLastError) */
    ATTN_ESCRATCH = -5     /* the call needs more than the library's static
                              scratch (attn_decode_noalloc only) */
} attn_status;

typedef enum {
    ATTN_NORM_NONE = 0,
    ATTN_NORM_W = 1,       /* x * r * w        ("Qwen" style)  */
    ATTN_NORM_1PW = 2      /* x * r * (1 + w)  ("Gemma" style) */
} attn_norm;

/*
 * Output gates, applied to the normalised attention output as it is written
 * (attn_prefill_chunk, attn_decode).  The gate has the call's dtype; the
 * value for output row (token t, head h), dim d, is
 *   gate[(t * n_heads + h) * gate_ld + d]      (per element), or
 *   gate[(t * n_heads + h) * gate_ld]          (per head),
 * t the packed row (prefill) or the sequence (decode).  gate_ld = head_dim
 * for a [n_tok][n_heads][head_dim] gate; 2 * head_dim with gate = the raw
 * query projection + head_dim reads the Qwen3.5 layout, each head's rows
 * [q(head_dim); gate(head_dim)] ([ATT] QwenAttnCfg.output_gate, the gate
 * split).
 */
typedef enum {
    ATTN_GATE_NONE = 0,
    ATTN_GATE_SIGMOID = 1,      /* out *= 1 / (1 + exp(-g)), per element ([ATT] fn apply_gate) */
    ATTN_GATE_SOFTPLUS_HEAD = 2,/* out *= softplus(g), one g per head   ([ATT] fn apply_projected_gate) */
    ATTN_GATE_SOFTPLUS = 3      /* out *= softplus(g), per element; softplus(x) = max(x, 0) +
                                   log(1 + exp(-|x|)) ([ATT] fn softplus) */
} attn_gate;

/*
 * RoPE inverse-frequency table.  [ATT] fn rope_inv_freq:
 *   inv_freq[i] = 1 / base^(2i / rotary_dim),  i < rotary_dim / 2,
 * evaluated in double and rounded once to float.
 * inv_freq: host, float[rotary_dim/2], written.
 * Errors: EINVAL if rotary_dim is not positive and even, base <= 0, or
 * inv_freq is NULL.
 */
int attn_rope_inv_freq(int rotary_dim, double base, float *inv_freq);

/*
 * YaRN inverse-frequency table.  [ATT] fn yarn_inv_freq ("Hugging Face
 * compatible"; rotary_dim is the rotary dimension, not the head width):
 *   cd(r)  = rotary_dim * ln(orig_max_pos / (2 pi r)) / (2 ln base)
 *   low    = max(floor(cd(beta_fast)), 0)
 *   high   = clamp(ceil(cd(beta_slow)), 0, rotary_dim/2 - 1)
 *   ramp_i = clamp(max(i - low, 0) / max(high - low, 1), 0, 1)
 *   inv_freq[i] = (f_i / factor) * ramp_i + f_i * (1 - ramp_i),
 * with f_i the plain RoPE frequency; double arithmetic, one rounding to float.
 * inv_freq: host, float[rotary_dim/2], written.
 * Errors: EINVAL if rotary_dim is not positive and even, base <= 1,
 * factor <= 0, orig_max_pos <= 0, beta_fast/beta_slow <= 0, or a NULL table.
 */
int attn_yarn_inv_freq(int rotary_dim, double base, double factor, int orig_max_pos,
                       double beta_fast, double beta_slow, float *inv_freq);

/*
 * Finish the query rows: optional per-head RMS norm, then RoPE, then rounding
 * to dtype.  [ATT] fn finish_projection (qk-norm before RoPE, partial RoPE on
 * the first rotary_dim dims), fn rmsnorm_head, fn rope_rotate_scaled:
 *   r = 1 / sqrt(mean(x^2) + eps);  x <- x*r*w  or  x*r*(1+w)
 *   x_i     <- (x_i cos t - x_{i+h} sin t) * rope_scale
 *   x_{i+h} <- (x_i sin t + x_{i+h} cos t) * rope_scale,
 *   h = rotary_dim / 2, t = position * inv_freq[i];
 * dims at or past rotary_dim are normed but neither rotated nor scaled.  The
 * norm, angle and rotation are computed in double; each stored element is
 * rounded once to dtype (ties to even).
 *   x        device [n_tok][n_heads][head_dim], read
 *   y        device [n_tok][n_heads][head_dim], written (y == x is allowed)
 *   inv_freq device float[rotary_dim/2]; rotary_dim 0 disables RoPE;
 *            rotary_dim > head_dim is clamped to head_dim ([ATT] uses
 *            rotary_dim.min(head_dim))
 *   norm_w   device float[head_dim], shared by all heads; NULL iff norm is
 *            ATTN_NORM_NONE
 * Errors: EINVAL (sizes, odd rotary_dim, NULL pointers, bad norm),
 * EUNSUPPORTED (dtype, head_dim), EDEVICE.
 */
int attn_rope_apply(const void *x, void *y, int dtype, int n_tok, int n_heads, int head_dim,
                    int n_seq, const int32_t *cu_seq, const int32_t *start, int max_chunk,
                    const float *inv_freq, int rotary_dim, float rope_scale, int norm,
                    const float *norm_w, double eps, void *stream);

/*
 * Append a chunk's keys and values to the head-major cache: each K row gets
 * the same finish as attn_rope_apply (norm, RoPE, rounding) and is written to
 * k_cache[b][g][start[b]+i][:]; each V row is copied bit for bit to
 * v_cache[b][g][start[b]+i][:].  Every row of the chunk is written by this
 * call, i.e. before any of the chunk's positions attends ([NDL] module docs,
 * "What has to stay sequential"; [ATT] fn qwen_attention_batch appends every
 * position of the chunk before the batched attend).  Rows outside
 * [start[b], start[b]+len_b) are not touched.
 *   k_cache, v_cache device [n_seq][n_kv][cap][head_dim], updated
 *   ring             0: position p in row p; 1: row p mod cap (see above)
 *   k_new, v_new     device [n_tok][n_kv][head_dim], read
 *   norm_w           the k-norm weight, device float[head_dim] or NULL
 *   v_norm           1: each V row is scale-less RMS-normalised first,
 *                    v / sqrt(mean(v^2) + eps), in double and rounded once
 *                    ([ATT] fn vnorm_head, Gemma-4); 0: copied bit for bit
 * Errors: ECAPACITY if max_end > cap without a ring, or with a ring that has
 * wrapped (max_end > cap) and max_chunk > cap (two positions of one chunk
 * would share a row); EINVAL (ring or v_norm not 0/1); otherwise as
 * attn_rope_apply.
 */
int attn_kv_append(void *k_cache, void *v_cache, int dtype, int n_seq, int n_kv, int head_dim,
                   int cap, int ring, const void *k_new, const void *v_new, int n_tok,
                   const int32_t *cu_seq, const int32_t *start, int max_chunk, int max_end,
                   const float *inv_freq, int rotary_dim, float rope_scale, int norm,
                   const float *norm_w, double eps, int v_norm, void *stream);

/*
 * attn_rope_apply on the queries and attn_kv_append on the keys and values of
 * the same chunk, in one call: the same results as the two calls (the
 * queries' finish, then every K/V row of the chunk in the cache before any
 * position attends), with one launch where the layout allows (rotary_dim a
 * multiple of 8, head_dim 64 or 128) -- a token's cos/sin table then serves
 * its query and key heads alike.  Arguments as in the two calls:
 *   q, q_out  device [n_tok][n_heads][head_dim] (q_out == q is allowed)
 *   k_cache, v_cache, k_new, v_new, n_kv, cap, ring, v_norm   as attn_kv_append
 *   q_norm_w, k_norm_w   the two norm weights (NULL iff norm is NONE)
 * Errors: the union of the two calls' errors (ECAPACITY as attn_kv_append).
 */
int attn_rope_qkv(const void *q, void *q_out, int n_heads, void *k_cache, void *v_cache,
                  const void *k_new, const void *v_new, int n_kv, int cap, int ring, int dtype,
                  int n_tok,
                  int head_dim, int n_seq, const int32_t *cu_seq, const int32_t *start,
                  int max_chunk, int max_end, const float *inv_freq, int rotary_dim,
                  float rope_scale, int norm, const float *q_norm_w, const float *k_norm_w,
                  double eps, int v_norm, void *stream);

/*
 * Causal attention for the rows of a chunk whose keys and values are already
 * in the cache (call attn_kv_append first).  For row i of sequence b at
 * position p = start[b]+i and query head h, with g = h / (n_heads/n_kv):
 *   s_j = scale * <q, K[b][g][j]>,  j = 0..p   (keys <= p only)
 *   out = sum_j softmax(s)_j V[b][g][j],  max-subtracted softmax
 * [ATT] fn attention_head, the batched causal fallback of fn
 * qwen_attention_batch (limit s0+bi+1), gpu::chunk_attend's signature;
 * [NDL] module docs (position p attends keys <= p).
 * bf16: products on bf16 matrix cores with float32 accumulation, softmax in
 * float32, probabilities rounded to bf16 for the P.V product; f32: float32
 * vector arithmetic.
 *   q        device [n_tok][n_heads][head_dim] (rotated), read
 *   out      device float[n_tok][n_heads][head_dim], written
 *   scale    the score scale, normally 1/sqrt(head_dim)
 *   ring     0: key j in cache row j; 1: row j mod cap.  A ring with
 *            max_end > cap needs 0 < window and window + max_chunk - 1 <= cap
 *            (ECAPACITY otherwise) and, for bf16, cap a multiple of 64
 *            (EUNSUPPORTED otherwise)
 *   window   0: every key <= p; W > 0: a sliding window, keys
 *            max(0, p-W+1)..p only ([ATT] QwenAttnCfg.window: a row reads
 *            just the most recent W positions).
 *   gate, gate_mode, gate_ld   output gate (see attn_gate; NULL/0 for none)
 *   workspace device scratch of workspace_bytes (may be NULL/0); with less
 *            than attn_prefill_workspace_bytes() the key range is split into
 *            fewer parts (never an error).  Contents need no initialisation
 *            and are clobbered.  Calls that share a workspace must be ordered
 *            on one stream.
 * Errors: ECAPACITY if max_end > cap without a ring (see ring); EINVAL
 * (window < 0, ring not 0/1, a gate mode without a gate or with gate_ld too
 * small, ...), EUNSUPPORTED, EDEVICE.
 */
int attn_prefill_chunk(const void *q, const void *k_cache, const void *v_cache, int dtype,
                       int n_seq, int n_heads, int n_kv, int head_dim, int cap, int ring,
                       int n_tok,
                       const int32_t *cu_seq, const int32_t *start, int max_chunk, int max_end,
                       float scale, int window, const void *gate, int gate_mode, int gate_ld,
                       float *out, void *workspace, size_t workspace_bytes, void *stream);

/*
 * attn_rope_qkv's arguments, as a struct, for attn_prefill_chunk_rope_next.
 */
typedef struct attn_rope_qkv_args {
    const void *q;
    void *q_out;
    int n_heads;
    void *k_cache;
    void *v_cache;
    const void *k_new;
    const void *v_new;
    int n_kv;
    int cap;
    int ring;
    int dtype;
    int n_tok;
    int head_dim;
    int n_seq;
    const int32_t *cu_seq;
    const int32_t *start;
    int max_chunk;
    int max_end;
    const float *inv_freq;
    int rotary_dim;
    float rope_scale;
    int norm;
    const float *q_norm_w;
    const float *k_norm_w;
    double eps;
    int v_norm;
} attn_rope_qkv_args;

/*
 * One step of a chunk loop: attn_prefill_chunk on this chunk, then
 * attn_rope_qkv(*next) on the next chunk -- the same results as the two calls
 * in that order.  The pages' chunk loop keeps sequential only that a chunk's
 * rows are in the cache before the chunk attends ([NDL] module docs, "What has
 * to stay sequential"; [ATT] fn qwen_attention_batch appends the chunk, then
 * attends); the next chunk's finish writes cache rows past every key this
 * chunk reads, so with bf16, the same head_dim, rotary_dim a multiple of 8
 * and neither cache wrapped (ring == 0 or max_end <= cap on both) it runs in
 * this chunk's attention launch, in the workgroups past the attention items
 * (one launch fewer per chunk).  Otherwise the two run one after the other.
 *   next     the next chunk's attn_rope_qkv arguments (not NULL)
 * Precondition of the single launch (the caller's chunk order): every cache
 * row next writes lies past every key this chunk reads, i.e. each sequence's
 * next chunk starts at or after the end of this one.  The call serves a loop
 * that has the next chunk's projected rows while this chunk attends (one
 * layer over a projected prompt); a caller that projects the next chunk only
 * after this one has passed every layer uses the two separate calls.
 * Outside the caches the two calls' buffers must not overlap where either
 * writes: next->q_out against this call's q, gate, out and workspace, and
 * this call's out and workspace against next->q, k_new and v_new (each as
 * the rows its sizes span).
 * Errors: those of either call, checked before anything is launched; EINVAL
 * for buffers that overlap as above.
 */
int attn_prefill_chunk_rope_next(const void *q, const void *k_cache, const void *v_cache, int dtype,
                                 int n_seq, int n_heads, int n_kv, int head_dim, int cap, int ring,
                                 int n_tok,
                                 const int32_t *cu_seq, const int32_t *start, int max_chunk,
                                 int max_end, float scale, int window, const void *gate,
                                 int gate_mode, int gate_ld, float *out, void *workspace,
                                 size_t workspace_bytes, const attn_rope_qkv_args *next,
                                 void *stream);

/*
 * A split chunk's merge left for a later launch, recorded by
 * attn_prefill_chunk_deferred and run by the next such call (as its prev) or
 * by attn_prefill_finish.  active is 1 while that chunk's output rows wait for
 * their merge, 0 when nothing is owed; head_dim and state belong to the
 * library (device pointers and sizes of that chunk's call, and a check word
 * over them: an active record the library did not write is refused with
 * EINVAL) and must not be changed.  Host memory, owned by the caller.
 */
typedef struct attn_prefill_pending {
    int active;
    int head_dim;
    uint64_t state[16];
} attn_prefill_pending;

/*
 * attn_prefill_chunk_rope_next with the split merge of each chunk moved into a
 * later launch: the merge of log-sum-exp partials is the same computation as
 * in attn_prefill_chunk (it exists because the max-subtracted softmax of [ATT]
 * fn attention_head lets parts of a key range be combined exactly), run
 * elsewhere.  When this chunk splits, its attention leaves the partials in
 * `workspace` and *pending records the merge owed: this chunk's rows of `out`
 * are final only once it has run.  The merge *prev owes (an earlier chunk's
 * record; NULL or inactive for none) runs in this call: in this chunk's
 * attention launch, in workgroups of its own ahead of the attention items,
 * when this chunk takes the bf16 prefill kernels with prev's head_dim, otherwise on a launch
 * of its own first (a merge too large for the attention launch's spare
 * workgroups takes that launch too).  When both ride, a loop of such calls is
 * one launch per chunk where attn_prefill_chunk + attn_rope_qkv take three.
 *   next     the next chunk's attn_rope_qkv arguments, or NULL (as in
 *            attn_prefill_chunk_rope_next, with its precondition)
 *   prev     an earlier chunk's record, or NULL; read before *pending is
 *            written (the two may be the same record)
 *   pending  written (not NULL): this chunk's merge, or active = 0
 * prev's partials stay in prev's workspace until its merge runs, so this
 * call's workspace must not overlap it (alternate two workspaces), and prev's
 * output rows, batch arrays and gate values must stay valid until then; after
 * the last chunk, run attn_prefill_finish on its record.  The results are
 * those of the same chunks through attn_prefill_chunk.
 * The buffers must not overlap as for attn_prefill_chunk_rope_next, and
 * prev's output rows (written by its merge) must overlap none of this call's
 * q, gate, out and workspace nor next's q, q_out, k_new and v_new.
 * Errors: those of attn_prefill_chunk and attn_rope_qkv, checked before
 * anything is launched; EINVAL for a NULL pending, an invalid prev record,
 * overlapping workspaces or buffers that overlap as above.
 */
int attn_prefill_chunk_deferred(const void *q, const void *k_cache, const void *v_cache, int dtype,
                                int n_seq, int n_heads, int n_kv, int head_dim, int cap, int ring,
                                int n_tok,
                                const int32_t *cu_seq, const int32_t *start, int max_chunk,
                                int max_end, float scale, int window, const void *gate,
                                int gate_mode, int gate_ld, float *out, void *workspace,
                                size_t workspace_bytes, const attn_rope_qkv_args *next,
                                const attn_prefill_pending *prev, attn_prefill_pending *pending,
                                void *stream);

/*
 * Runs the merge a record owes, on `stream` (nothing for an inactive record).
 * Errors: EINVAL for NULL or an invalid record; EDEVICE.
 */
int attn_prefill_finish(const attn_prefill_pending *pending, void *stream);

/*
 * Workspace, in bytes, that lets attn_prefill_chunk split the key range as far
 * as it chooses for these sizes (the split is this library's own scheduling,
 * not a step of the pages: [ATT] fn attention_head's max-subtracted softmax is
 * what lets parts of the key range be merged exactly).  0 when the call would
 * not split, or for invalid sizes (non-positive sizes, n_heads % n_kv != 0,
 * head_dim not 64/128).  Enough for any window.  Host only; no device call.
 */
size_t attn_prefill_workspace_bytes(int n_seq, int n_heads, int n_kv, int head_dim, int n_tok,
                                    int max_chunk, int max_end);

/*
 * Decode: one query per sequence (chunk = 1) at position ctx[b]-1, whose K/V
 * row is already in the cache (append it first with attn_kv_append,
 * start[b] = ctx[b]-1).  Row (b, h) attends keys 0..ctx[b]-1 of KV head
 * h/(n_heads/n_kv), as attn_prefill_chunk; optionally it also returns the
 * attention probabilities ([ATT] fn attention_head returns (out, probs); the
 * probabilities feed importance accounting).  The key range of each sequence
 * is split across workgroups and the parts are merged with a log-sum-exp
 * combine.
 *   q      device [n_seq][n_heads][head_dim] (rotated), read
 *   ctx    device int32[n_seq], 1 <= ctx[b] <= max_ctx (values above max_ctx
 *          are clamped to it; a row with ctx[b] < 1 gets zeros)
 *   ring   0: key j in cache row j; 1: row j mod cap.  A ring with
 *          max_ctx > cap needs 0 < window <= cap (ECAPACITY otherwise)
 *   window 0: all ctx[b] keys; W > 0: only the last W (a sliding window,
 *          [ATT] the decode loop starts at stored - window); the
 *          probabilities of the keys before it are written as 0
 *   gate, gate_mode, gate_ld   output gate of row (b, h) (see attn_gate);
 *          the probabilities are not gated
 *   out    device float[n_seq][n_heads][head_dim], written
 *   probs  NULL, or device float[n_seq][n_heads][probs_ld]; row (b, h) gets
 *          ctx[b] entries summing to 1, entries past ctx[b] are not written.
 *          Any probs_ld >= max_ctx works; a multiple of 32 starts every row
 *          on a 128-byte line, which the 16-byte stores of the kernels use.
 *          bf16: the row's first ctx[b] entries also hold the intermediate
 *          unnormalised values in half precision, so each probability
 *          carries a relative error below 2^-10 (2^-11 from its own
 *          rounding, 2^-11 from the sum of rounded values that normalises
 *          it) plus, for values below half precision's normal range, an
 *          absolute one below 2^-24 of the row's largest; f32: float
 *          throughout
 *   workspace device scratch, clobbered, no initialisation needed.  bf16
 *          needs at least n_seq*n_heads*(2*head_dim+16) bytes (one part per
 *          row, EINVAL below that); attn_decode_workspace_bytes() gives the
 *          size for the full split, and a smaller one means fewer, longer
 *          parts.  f32 needs none.
 * Errors: ECAPACITY if max_ctx > cap without a ring (see ring); EINVAL
 * (probs_ld < max_ctx, window < 0, ring not 0/1, a bad gate, ...), EUNSUPPORTED (bf16
 * with more than 16 query heads per KV head), EDEVICE.
 */
int attn_decode(const void *q, const void *k_cache, const void *v_cache, int dtype, int n_seq,
                int n_heads, int n_kv, int head_dim, int cap, int ring, const int32_t *ctx,
                int max_ctx, float scale, int window, const void *gate, int gate_mode,
                int gate_ld, float *out, float *probs, int probs_ld,
                void *workspace, size_t workspace_bytes, void *stream);

/*
 * Workspace, in bytes, for attn_decode to split every row's key range as far
 * as it chooses (parts of up to 1024 keys, fewer keys per part for groups of
 * more than 4 query heads per KV head): per (sequence, head, part) a 16-byte
 * header (running maximum, row sum, sum of the rounded probabilities, scale
 * exponent) and head_dim half-precision values.  Arguments as attn_decode;
 * max_ctx bounds every ctx[b].  Returns 0 for invalid sizes (non-positive
 * sizes, n_heads % n_kv != 0, head_dim not 64/128).  Host only; no device
 * call.  A smaller workspace is accepted (fewer, longer parts) down to the
 * one-part minimum attn_decode documents.
 */
size_t attn_decode_workspace_bytes(int n_seq, int n_heads, int n_kv, int head_dim, int max_ctx);

/*
 * attn_decode for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same computation, arguments and results as attn_decode, with the split
 * partials in a static scratch array that the library holds on each GPU it
 * runs on (ATTN_NOALLOC_SCRATCH_BYTES per GPU, kept until the process ends)
 * instead of a caller workspace.  Nothing is allocated by the call.  The
 * call uses as many key-range parts as fit in the scratch (the full split of
 * attn_decode_workspace_bytes() when that fits, so the results equal
 * attn_decode's with that workspace).  Every call on one GPU shares that
 * GPU's scratch: calls that overlap on one GPU (different streams, or other
 * threads) race on it and must be ordered by the caller.  No part of the
 * scratch needs to start at zero.
 * Errors: as attn_decode; ATTN_ESCRATCH (before any device call) when even
 * one part per row does not fit: n_seq * n_heads * (2 * head_dim + 16)
 * bytes above ATTN_NOALLOC_SCRATCH_BYTES.
 */
#define ATTN_NOALLOC_SCRATCH_BYTES (32u << 20)
int attn_decode_noalloc(const void *q, const void *k_cache, const void *v_cache, int dtype, int n_seq,
                        int n_heads, int n_kv, int head_dim, int cap, int ring, const int32_t *ctx,
                        int max_ctx, float scale, int window, const void *gate, int gate_mode,
                        int gate_ld, float *out, float *probs, int probs_ld, void *stream);

/*
 * Importance of each cached position after a decode step ([ATT] the decode
 * attention adds every head's probability row into one vector before the
 * cache accumulates it for eviction; a position's importance is the total
 * probability the step's heads give it):
 *   imp[b][j] = (accumulate ? imp[b][j] : 0) + sum_h probs[b][h][j],
 * for j < min(ctx[b], max_ctx); entries past that are not written.  Heads are
 * summed in order in float.
 *   probs  device float[n_seq][n_heads][probs_ld], as attn_decode returned
 *          them, read
 *   ctx    device int32[n_seq], the same array attn_decode used
 *   imp    device float[n_seq][imp_ld], read (when accumulating) and written
 * Ownership: the caller's buffers; nothing is allocated.  The call is
 * ordered after attn_decode on the same stream.
 * Errors: EINVAL (null pointer, probs_ld or imp_ld < max_ctx, n_heads <= 0,
 * negative sizes), EDEVICE.  n_seq == 0 or max_ctx == 0: ATTN_OK, no launch.
 */
int attn_decode_importance(const float *probs, int n_seq, int n_heads, int probs_ld,
                           const int32_t *ctx, int max_ctx, float *imp, int imp_ld,
                           int accumulate, void *stream);

/*
 * Measured roofline denominators (not a step of the pages: the throughput of
 * the attention calls is stated as a fraction of the part's peaks, and these
 * two kernels measure what the part sustains next to the published figures).
 *
 * attn_calibrate_mfma: n_workgroups workgroups of 4 waves, each wave issuing
 *   iters rounds of four independent 32x32x16 bf16 matrix products
 *   (32768 FLOP each); total work n_workgroups * 4 * iters * 4 * 32768 FLOP.
 *   random_operands 0: small constant operands with few distinct bits (the
 *   highest rate the part sustains); 1: hashed random bfloat16 operands, a
 *   different set per accumulator (the rate for data like the attention
 *   kernels': the clock under load falls with the operands' switching).
 *   out: device float[n_workgroups * 4], one value per wave, written.
 * attn_calibrate_read: a streaming read of `bytes` (a multiple of 16, src
 *   16-byte aligned) with nontemporal 16-byte loads by n_workgroups
 *   workgroups of 256 threads, each reading its own contiguous share.
 *   out: device uint32[n_workgroups * 4], one value per wave, written.
 * The caller times the launch on `stream` (e.g. with events).  Errors: EINVAL
 * for non-positive sizes, NULL pointers, misaligned reads, random_operands
 * other than 0/1; EDEVICE.
 */
int attn_calibrate_mfma(int n_workgroups, int iters, int random_operands, float *out, void *stream);
int attn_calibrate_read(const void *src, size_t bytes, int n_workgroups, uint32_t *out, void *stream);

/* Static, human-readable name of a status code. */
const char *attn_status_string(int status);

/* Library version, "major.minor.patch". */
const char *attn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_H */
