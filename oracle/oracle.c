/*
 * oracle.c -- plain, slow CPU oracle for causal grouped-query attention with
 * RoPE over a head-major KV cache.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code with
 * the HIP library and never consumes anything that library produced.
 *
 * Everything is computed in double precision with straight loops, in the order
 * the source pages describe.  Sources (page title, then the item on it):
 *   [ATT]  cortiq-engine 0.5.39, src/attention.rs
 *   [NDL]  needle-core 0.3.1, src/v2/batch.rs
 *
 * Readings taken where the pages leave a step open are listed next to the
 * function that takes them.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifndef M_PI
#define M_PI 3.14159265358979323846
#endif

/* ------------------------------------------------------------------------ */
/* Frequency tables                                                          */
/* ------------------------------------------------------------------------ */

/*
 * [ATT] fn rope_inv_freq: one inverse frequency per rotated pair,
 *   f_i = 1 / base^(2i/d),  i < d/2,  d = rotary dimension.
 * Reading: evaluated in double and rounded once to float (the page stores the
 * table as f32, and the device receives an f32 table).
 */
void orc_rope_inv_freq(int rd, double base, float *out)
{
    for (int i = 0; i < rd / 2; i++) {
        double f = 1.0 / pow(base, (2.0 * i) / (double)rd);
        out[i] = (float)f;
    }
}

/*
 * YaRN "by parts" frequency table, Hugging Face flavour ([ATT] fn
 * yarn_inv_freq; the rotary dimension d plays the role of the head width).
 *
 * A rotated pair i turns L0 * f_i / (2 pi) times over the original context L0.
 * The pair whose count equals r sits at the fractional index
 *     c(r) = d * ln(L0 / (2 pi r)) / (2 ln base).
 * Pairs that turn at least beta_fast times (index <= c(beta_fast)) keep their
 * frequency; pairs that turn fewer than beta_slow times are interpolated, i.e.
 * divided by the scaling factor s; between the two bounds a linear ramp
 *     gamma_i = clamp((i - lo) / max(hi - lo, 1), 0, 1),
 *     lo = max(floor(c(beta_fast)), 0),
 *     hi = min(max(ceil(c(beta_slow)), 0), d/2 - 1),
 * blends the two:  f'_i = f_i * (1 - gamma_i) + (f_i / s) * gamma_i.
 * Reading: the bounds are the integer ones the page forms (floor, ceil, the
 * clamp of hi to the last pair, the ramp's width at least 1); double
 * arithmetic, one rounding to float at the end.  The bounds are returned
 * through *lo_out / *hi_out when non-NULL.
 */
static double yarn_corr_index(int rd, double base, int orig_max_pos, double rotations)
{
    return (double)rd * log((double)orig_max_pos / (2.0 * M_PI * rotations)) / (2.0 * log(base));
}

void orc_yarn_inv_freq(int rd, double base, double factor, int orig_max_pos,
                       double beta_fast, double beta_slow, float *out,
                       int *lo_out, int *hi_out)
{
    int n_pairs = rd / 2;
    double lo = fmax(floor(yarn_corr_index(rd, base, orig_max_pos, beta_fast)), 0.0);
    double hi = fmax(ceil(yarn_corr_index(rd, base, orig_max_pos, beta_slow)), 0.0);
    hi = fmin(hi, (double)(n_pairs > 0 ? n_pairs - 1 : 0));
    double width = fmax(hi - lo, 1.0);
    for (int i = 0; i < n_pairs; i++) {
        double f = 1.0 / pow(base, (2.0 * i) / (double)rd);
        double gamma = fmin(fmax(((double)i - lo) / width, 0.0), 1.0);
        out[i] = (float)(f * (1.0 - gamma) + (f / factor) * gamma);
    }
    if (lo_out)
        *lo_out = (int)lo;
    if (hi_out)
        *hi_out = (int)hi;
}

/* ------------------------------------------------------------------------ */
/* Storage rounding                                                          */
/* ------------------------------------------------------------------------ */

/*
 * Round a double to the nearest bfloat16 value, ties to even (8 significant
 * bits, exponent range of float).  Written from the format's definition:
 * scale so that the bfloat16 quantum becomes 1, round to the nearest integer
 * (the default rounding mode is to-nearest-even), scale back.
 */
double orc_round_bf16(double x)
{
    if (x == 0.0 || isnan(x) || isinf(x))
        return x;
    int e;
    (void)frexp(x, &e);           /* |x| = m * 2^e, 0.5 <= m < 1 */
    int q = e - 8;                /* quantum exponent for 8 significant bits */
    if (q < -133)                 /* bfloat16 subnormal quantum is 2^-133 */
        q = -133;
    double r = nearbyint(ldexp(x, -q));
    double y = ldexp(r, q);
    double max_finite = ldexp(255.0, 120); /* (2 - 2^-7) * 2^127 */
    if (fabs(y) > max_finite)
        return copysign(INFINITY, x);
    return y;
}

/* store_dtype: 0 = float32, 1 = bfloat16 */
static double round_store(double x, int store_dtype)
{
    if (store_dtype == 1)
        return orc_round_bf16(x);
    return (double)(float)x;
}

void orc_round_array(double *x, long n, int store_dtype)
{
    for (long i = 0; i < n; i++)
        x[i] = round_store(x[i], store_dtype);
}

/* ------------------------------------------------------------------------ */
/* Per-head finish: qk-norm, then RoPE                                       */
/* ------------------------------------------------------------------------ */

/*
 * [ATT] fn rmsnorm_head: r = 1/sqrt(sum(x^2)/n + eps); x <- x*r*w ("Qwen"
 * style, norm_style 1) or x*r*(1+w) ("Gemma" style, norm_style 2).
 */
static void rmsnorm_head(double *x, int hd, const float *w, int norm_style, double eps)
{
    double ss = 0.0;
    for (int d = 0; d < hd; d++)
        ss += x[d] * x[d];
    double r = 1.0 / sqrt(ss / (double)hd + eps);
    for (int d = 0; d < hd; d++) {
        double wd = (double)w[d];
        double g = norm_style == 2 ? 1.0 + wd : wd;
        x[d] = x[d] * r * g;
    }
}

/*
 * [ATT] fn rope_rotate_scaled: half-split pairs (i, i+h), h = rd/2,
 *   x_i     <- (x_i cos t - x_{i+h} sin t) * s
 *   x_{i+h} <- (x_i sin t + x_{i+h} cos t) * s,   t = position * f_i.
 * Dims at or past rd pass through unchanged and unscaled ([ATT] fn
 * finish_projection, partial RoPE).  Reading: the angle is formed in double
 * from the f32 table entry (the page forms it in f32).
 */
static void rope_head(double *x, int rd, long pos, const float *inv_freq, double s)
{
    int h = rd / 2;
    for (int i = 0; i < h; i++) {
        double t = (double)pos * (double)inv_freq[i];
        double c = cos(t), sn = sin(t);
        double a = x[i], b = x[i + h];
        x[i] = (a * c - b * sn) * s;
        x[i + h] = (a * sn + b * c) * s;
    }
}

/*
 * Finish the rows of one projection for a set of tokens: optional per-head
 * norm, then RoPE, then the storage rounding of the tensor that is kept
 * (rotated Q, or the K cache row).  x: [n_tok][n_heads][hd], in place.
 * pos[t] is the absolute position of token t.  norm_style 0 = no norm.
 * [ATT] fn finish_projection: norm before RoPE; RoPE on the first rd dims.
 * Tokens are independent; they are shared out over n_threads threads.
 */
typedef struct {
    double *x;
    int n_tok, n_heads, hd, rd, norm_style, store_dtype, n_threads, tid;
    const int64_t *pos;
    const float *inv_freq, *norm_w;
    double rope_scale, eps;
} finish_job;

static void *finish_worker(void *arg)
{
    finish_job *jb = (finish_job *)arg;
    for (int t = jb->tid; t < jb->n_tok; t += jb->n_threads) {
        for (int h = 0; h < jb->n_heads; h++) {
            double *row = jb->x + ((long)t * jb->n_heads + h) * jb->hd;
            if (jb->norm_style != 0)
                rmsnorm_head(row, jb->hd, jb->norm_w, jb->norm_style, jb->eps);
            rope_head(row, jb->rd, (long)jb->pos[t], jb->inv_freq, jb->rope_scale);
            for (int d = 0; d < jb->hd; d++)
                row[d] = round_store(row[d], jb->store_dtype);
        }
    }
    return NULL;
}

void orc_finish_heads(double *x, int n_tok, int n_heads, int hd, const int64_t *pos,
                      const float *inv_freq, int rd, double rope_scale, int norm_style,
                      const float *norm_w, double eps, int store_dtype, int n_threads)
{
    if (rd > hd)
        rd = hd;
    if (n_threads < 1)
        n_threads = 1;
    if (n_threads > n_tok)
        n_threads = n_tok > 0 ? n_tok : 1;
    finish_job jobs[64];
    pthread_t th[64];
    if (n_threads > 64)
        n_threads = 64;
    for (int i = 0; i < n_threads; i++) {
        finish_job j = {x, n_tok, n_heads, hd, rd, norm_style, store_dtype, n_threads, i,
                        pos, inv_freq, norm_w, rope_scale, eps};
        jobs[i] = j;
    }
    int started = 0;
    for (int i = 1; i < n_threads; i++) {
        if (pthread_create(&th[i], NULL, finish_worker, &jobs[i]) != 0)
            break;
        started = i;
    }
    for (int i = started + 1; i < n_threads; i++)
        finish_worker(&jobs[i]);
    finish_worker(&jobs[0]);
    for (int i = 1; i <= started; i++)
        pthread_join(th[i], NULL);
}

/* ------------------------------------------------------------------------ */
/* Attention                                                                 */
/* ------------------------------------------------------------------------ */

/*
 * One query row against one KV group, keys 0..p inclusive:
 *   s_j = scale * <q, K_j>,  m = max s,  e_j = exp(s_j - m),  l = sum e_j,
 *   P_j = e_j / l,  O = sum_j P_j V_j.
 * [ATT] fn attention_head (max-subtracted softmax, probabilities returned);
 * [NDL] module docs: a row at position p sees keys 0..p.
 * Readings: no weight is skipped (the page skips |P| < 1e-12); the softmax is
 * normalised before the P.V sum, as in fn attention_head.
 */
static void attend_row(const double *q, const double *kc, const double *vc, int hd, long nkeys,
                       double scale, double *out, double *probs, double *scratch)
{
    double m = -INFINITY;
    for (long j = 0; j < nkeys; j++) {
        const double *k = kc + j * hd;
        double acc = 0.0;
        for (int d = 0; d < hd; d++)
            acc += q[d] * k[d];
        scratch[j] = acc * scale;
        if (scratch[j] > m)
            m = scratch[j];
    }
    double l = 0.0;
    for (long j = 0; j < nkeys; j++) {
        scratch[j] = exp(scratch[j] - m);
        l += scratch[j];
    }
    for (long j = 0; j < nkeys; j++)
        scratch[j] /= l;
    for (int d = 0; d < hd; d++)
        out[d] = 0.0;
    for (long j = 0; j < nkeys; j++) {
        const double *v = vc + j * hd;
        double p = scratch[j];
        for (int d = 0; d < hd; d++)
            out[d] += p * v[d];
    }
    if (probs)
        memcpy(probs, scratch, (size_t)nkeys * sizeof(double));
}

typedef struct {
    const double *q, *kc, *vc;
    int n_tok, nh, nkv, hd;
    long cap;
    const int64_t *qpos;
    double scale;
    double *out, *probs;
    long probs_ld;
    long window;
    int n_threads, tid;
    int status;
} attend_job;

static void *attend_worker(void *arg)
{
    attend_job *jb = (attend_job *)arg;
    long max_keys = 0;
    for (int t = 0; t < jb->n_tok; t++)
        if (jb->qpos[t] + 1 > max_keys)
            max_keys = (long)jb->qpos[t] + 1;
    double *scratch = (double *)malloc((size_t)(max_keys > 0 ? max_keys : 1) * sizeof(double));
    if (!scratch) {
        jb->status = -1;
        return NULL;
    }
    int group = jb->nh / jb->nkv; /* query heads per KV head */
    long rows = (long)jb->n_tok * jb->nh;
    for (long r = jb->tid; r < rows; r += jb->n_threads) {
        int t = (int)(r / jb->nh), h = (int)(r % jb->nh);
        int g = h / group; /* [ATT] GQA mapping: query head h reads KV head h/(nh/nkv) */
        const double *q = jb->q + r * jb->hd;
        const double *kc = jb->kc + (long)g * jb->cap * jb->hd;
        const double *vc = jb->vc + (long)g * jb->cap * jb->hd;
        double *pr = jb->probs ? jb->probs + r * jb->probs_ld : NULL;
        /* sliding window ([ATT] QwenAttnCfg.window: only the most recent W
         * positions are read; the decode loop starts at stored - window): keys
         * first..p, probabilities of the keys before it are 0 */
        long first = 0;
        if (jb->window > 0 && (long)jb->qpos[t] + 1 > jb->window)
            first = (long)jb->qpos[t] + 1 - jb->window;
        if (pr)
            for (long j = 0; j < first; j++)
                pr[j] = 0.0;
        attend_row(q, kc + first * jb->hd, vc + first * jb->hd, jb->hd, (long)jb->qpos[t] + 1 - first,
                   jb->scale, jb->out + r * jb->hd, pr ? pr + first : NULL, scratch);
    }
    free(scratch);
    jb->status = 0;
    return NULL;
}

/*
 * Attention for the rows of one sequence.
 *   q     [n_tok][nh][hd]   rotated queries
 *   kc,vc [nkv][cap][hd]    the sequence's cache; rows 0..max(qpos) are read
 *   qpos  [n_tok]           absolute position of each query row; row t attends
 *                           keys 0..qpos[t]
 *   out   [n_tok][nh][hd]
 *   probs NULL or [n_tok][nh][probs_ld]; row (t,h) gets qpos[t]+1 entries
 * Returns 0, or -1 on bad arguments / allocation failure.
 */
int orc_attend_window(const double *q, const double *kc, const double *vc, int n_tok, int nh,
                      int nkv, int hd, long cap, const int64_t *qpos, double scale, double *out,
                      double *probs, long probs_ld, long window, int n_threads);

int orc_attend(const double *q, const double *kc, const double *vc, int n_tok, int nh, int nkv,
               int hd, long cap, const int64_t *qpos, double scale, double *out, double *probs,
               long probs_ld, int n_threads)
{
    return orc_attend_window(q, kc, vc, n_tok, nh, nkv, hd, cap, qpos, scale, out, probs, probs_ld,
                             0, n_threads);
}

/*
 * The same with a sliding window: window > 0 limits row t to the keys
 * max(0, qpos[t] + 1 - window) .. qpos[t]; 0 means the whole prefix.
 */
int orc_attend_window(const double *q, const double *kc, const double *vc, int n_tok, int nh,
                      int nkv, int hd, long cap, const int64_t *qpos, double scale, double *out,
                      double *probs, long probs_ld, long window, int n_threads)
{
    if (window < 0)
        return -1;
    if (n_tok < 0 || nh <= 0 || nkv <= 0 || hd <= 0 || nh % nkv != 0)
        return -1;
    for (int t = 0; t < n_tok; t++)
        if (qpos[t] < 0 || qpos[t] >= cap || (probs && qpos[t] + 1 > probs_ld))
            return -1;
    if (n_tok == 0)
        return 0;
    if (n_threads < 1)
        n_threads = 1;
    long rows = (long)n_tok * nh;
    if (n_threads > rows)
        n_threads = (int)rows;
    attend_job *jobs = (attend_job *)calloc((size_t)n_threads, sizeof(attend_job));
    pthread_t *th = (pthread_t *)calloc((size_t)n_threads, sizeof(pthread_t));
    if (!jobs || !th) {
        free(jobs);
        free(th);
        return -1;
    }
    int rc = 0;
    for (int i = 0; i < n_threads; i++) {
        attend_job j = {q, kc, vc, n_tok, nh, nkv, hd, cap, qpos, scale, out, probs, probs_ld,
                        window, n_threads, i, 0};
        jobs[i] = j;
    }
    int started = 0;
    for (int i = 1; i < n_threads; i++) {
        if (pthread_create(&th[i], NULL, attend_worker, &jobs[i]) != 0)
            break;
        started = i;
    }
    /* Rows of threads that failed to start are done by the calling thread. */
    for (int i = started + 1; i < n_threads; i++) {
        jobs[i].tid = i;
        attend_worker(&jobs[i]);
    }
    attend_worker(&jobs[0]);
    for (int i = 1; i <= started; i++)
        pthread_join(th[i], NULL);
    for (int i = 0; i < n_threads; i++)
        if (jobs[i].status != 0)
            rc = -1;
    free(jobs);
    free(th);
    return rc;
}

/*
 * Importance of each cached position for one decode step ([ATT] the
 * per-head loop of the decode attention adds every head's probability row
 * into one vector, so a position's importance is the total probability the
 * heads give it): imp[j] = sum over heads h of probs[h][j], j < ctx, heads in
 * order, in double.  probs [nh][probs_ld].  Returns 0, or -1 on bad
 * arguments.
 */
int orc_head_importance(const double *probs, int nh, long ctx, long probs_ld, double *imp)
{
    if (nh <= 0 || ctx < 0 || probs_ld < ctx)
        return -1;
    for (long j = 0; j < ctx; j++) {
        double s = 0.0;
        for (int h = 0; h < nh; h++)
            s += probs[(long)h * probs_ld + j];
        imp[j] = s;
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* V-norm and output gates                                                   */
/* ------------------------------------------------------------------------ */

/*
 * [ATT] fn vnorm_head (Gemma-4): a V head is RMS-normalised, without a
 * weight, ahead of the cache write: x <- x / sqrt(mean(x^2) + eps) -- no
 * weight, no "+1".  x: rows of hd values, in place, then the storage rounding.
 * Reading: evaluated in double and rounded once, like the qk-norm.
 */
void orc_vnorm_heads(double *x, long rows, int hd, double eps, int store_dtype)
{
    for (long r = 0; r < rows; r++) {
        double *row = x + r * hd;
        double ss = 0.0;
        for (int d = 0; d < hd; d++)
            ss += row[d] * row[d];
        double inv = 1.0 / sqrt(ss / (double)hd + eps);
        for (int d = 0; d < hd; d++)
            row[d] = round_store(row[d] * inv, store_dtype);
    }
}

/* [ATT] fn softplus: max(x, 0) + log(1 + exp(-|x|)) */
static double softplus(double x)
{
    return fmax(x, 0.0) + log1p(exp(-fabs(x)));
}

/*
 * Output gates on the attention output out [rows][hd], rows = (token, head)
 * pairs, gate row r at gate + r * gate_ld:
 *   mode 1: out *= 1 / (1 + exp(-g_d))     ([ATT] fn apply_gate: the
 *           Qwen3.5 output gate, the second half of each head's q rows)
 *   mode 2: out *= softplus(g_0)           ([ATT] fn apply_projected_gate,
 *           per-head gain broadcast across head_dim)
 *   mode 3: out *= softplus(g_d)           (the same, per element)
 * Returns 0, or -1 on a bad mode.
 */
int orc_output_gate(double *out, const double *gate, long rows, int hd, long gate_ld, int mode)
{
    if (mode < 1 || mode > 3)
        return -1;
    for (long r = 0; r < rows; r++) {
        const double *g = gate + r * gate_ld;
        double *o = out + r * hd;
        for (int d = 0; d < hd; d++) {
            double f;
            if (mode == 1)
                f = 1.0 / (1.0 + exp(-g[d]));
            else if (mode == 2)
                f = softplus(g[0]);
            else
                f = softplus(g[d]);
            o[d] *= f;
        }
    }
    return 0;
}
