/*
 * Sanitizer driver for the CPU oracle (test infrastructure): every oracle
 * function on small inputs, built with AddressSanitizer and
 * UndefinedBehaviorSanitizer by tests/test_sanitizers_cpu.py.  Besides
 * running clean under the sanitizers, it checks a few invariants the
 * pages fix (rows of probabilities sum to 1, position 0 returns V0, RoPE at
 * position 0 is the identity) so the calls are exercised on real paths.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

void orc_rope_inv_freq(int rd, double base, float *out);
void orc_yarn_inv_freq(int rd, double base, double factor, int orig_max_pos, double beta_fast,
                       double beta_slow, float *out, int *lo_out, int *hi_out);
double orc_round_bf16(double x);
void orc_round_array(double *x, long n, int store_dtype);
void orc_finish_heads(double *x, int n_tok, int n_heads, int hd, const int64_t *pos,
                      const float *inv_freq, int rd, double rope_scale, int norm_style,
                      const float *norm_w, double eps, int store_dtype, int n_threads);
int orc_attend_window(const double *q, const double *kc, const double *vc, int n_tok, int nh,
                      int nkv, int hd, long cap, const int64_t *qpos, double scale, double *out,
                      double *probs, long probs_ld, long window, int n_threads);
int orc_attend(const double *q, const double *kc, const double *vc, int n_tok, int nh, int nkv,
               int hd, long cap, const int64_t *qpos, double scale, double *out, double *probs,
               long probs_ld, int n_threads);
int orc_head_importance(const double *probs, int nh, long ctx, long probs_ld, double *imp);
void orc_vnorm_heads(double *x, long rows, int hd, double eps, int store_dtype);
int orc_output_gate(double *out, const double *gate, long rows, int hd, long gate_ld, int mode);

static int failures = 0;
#define CHECK(c, msg)                                  \
    do {                                               \
        if (!(c)) {                                    \
            fprintf(stderr, "FAILED: %s\n", msg);      \
            failures++;                                \
        }                                              \
    } while (0)

static double lcg(unsigned long long *s)
{
    *s = *s * 6364136223846793005ULL + 1442695040888963407ULL;
    return ((double)(*s >> 11) / 9007199254740992.0) * 2.0 - 1.0;
}

int main(void)
{
    unsigned long long seed = 12345;
    enum { T = 9, NH = 4, NKV = 2, HD = 16, RD = 12 };
    float f[HD / 2], fy[HD / 2], w[HD];
    int lo = -1, hi = -1;
    orc_rope_inv_freq(RD, 1e4, f);
    CHECK(f[0] == 1.0f, "rope table starts at 1");
    orc_yarn_inv_freq(RD, 1e4, 4.0, 64, 32.0, 1.0, fy, &lo, &hi);
    CHECK(lo >= 0 && hi <= RD / 2 - 1, "yarn bounds inside the table");
    CHECK(orc_round_bf16(1.0 + 1.0 / 512.0) == 1.0, "bf16 tie rounds to even");
    double *q = malloc(sizeof(double) * T * NH * HD), *k = malloc(sizeof(double) * T * NKV * HD);
    double *v = malloc(sizeof(double) * T * NKV * HD), *x0 = malloc(sizeof(double) * T * NH * HD);
    for (int i = 0; i < T * NH * HD; i++) q[i] = x0[i] = lcg(&seed);
    for (int i = 0; i < T * NKV * HD; i++) {
        k[i] = lcg(&seed);
        v[i] = lcg(&seed);
    }
    for (int i = 0; i < HD; i++) w[i] = 1.0f + 0.1f * (float)lcg(&seed);
    int64_t pos[T];
    for (int t = 0; t < T; t++) pos[t] = t;
    orc_round_array(q, T * NH * HD, 1);
    orc_finish_heads(x0, 1, NH, HD, pos, f, RD, 1.0, 0, NULL, 1e-6, 0, 2);
    /* position 0: RoPE is the identity (up to the float rounding) */
    for (int i = 0; i < NH * HD; i++) CHECK(x0[i] == (double)(float)x0[i], "float storage");
    orc_finish_heads(q, T, NH, HD, pos, fy, RD, 1.1, 1, w, 1e-6, 1, 3);
    orc_finish_heads(k, T, NKV, HD, pos, fy, RD, 1.1, 2, w, 1e-6, 1, 3);
    orc_vnorm_heads(v, T * NKV, HD, 1e-6, 1);
    /* head-major cache [nkv][T][hd] */
    double *kc = malloc(sizeof(double) * NKV * T * HD), *vc = malloc(sizeof(double) * NKV * T * HD);
    for (int t = 0; t < T; t++)
        for (int g = 0; g < NKV; g++)
            for (int d = 0; d < HD; d++) {
                kc[((long)g * T + t) * HD + d] = k[((long)t * NKV + g) * HD + d];
                vc[((long)g * T + t) * HD + d] = v[((long)t * NKV + g) * HD + d];
            }
    double *out = malloc(sizeof(double) * T * NH * HD), *probs = malloc(sizeof(double) * T * NH * T);
    CHECK(orc_attend(q, kc, vc, T, NH, NKV, HD, T, pos, 0.25, out, probs, T, 4) == 0, "attend");
    for (int t = 0; t < T; t++)
        for (int h = 0; h < NH; h++) {
            double s = 0.0;
            for (int j = 0; j <= t; j++) s += probs[((long)t * NH + h) * T + j];
            CHECK(fabs(s - 1.0) < 1e-12, "probability rows sum to 1");
        }
    for (int h = 0; h < NH; h++)
        for (int d = 0; d < HD; d++)
            CHECK(out[(long)h * HD + d] == vc[(long)(h / (NH / NKV)) * T * HD + d], "position 0 returns V0");
    CHECK(orc_attend_window(q, kc, vc, T, NH, NKV, HD, T, pos, 0.25, out, probs, T, 3, 2) == 0, "window");
    CHECK(orc_attend_window(q, kc, vc, T, NH, NKV, HD, T, pos, 0.25, out, NULL, 0, -1, 2) == -1, "bad window");
    double imp[T];
    CHECK(orc_head_importance(probs + (long)(T - 1) * NH * T, NH, T, T, imp) == 0, "importance");
    double sum = 0.0;
    for (int j = 0; j < T; j++) sum += imp[j];
    CHECK(fabs(sum - NH) < 1e-12, "importances sum to the head count");
    double *gate = malloc(sizeof(double) * T * NH * HD);
    for (int i = 0; i < T * NH * HD; i++) gate[i] = lcg(&seed) * 4.0;
    for (int mode = 1; mode <= 3; mode++)
        CHECK(orc_output_gate(out, gate, T * NH, HD, HD, mode) == 0, "output gate");
    CHECK(orc_output_gate(out, gate, T * NH, HD, HD, 7) != 0, "bad gate mode");
    free(q); free(k); free(v); free(x0); free(kc); free(vc); free(out); free(probs); free(gate);
    if (failures) return 1;
    printf("oracle sanitizer check ok\n");
    return 0;
}
