/*
 * Sanitizer driver for the library's host code (test infrastructure): the
 * frequency tables, the workspace planners and every entry point's
 * argument validation, built with AddressSanitizer and
 * UndefinedBehaviorSanitizer on the host side by
 * tests/test_sanitizers_cpu.py.  No call here reaches a kernel launch: every
 * device pointer is a placeholder that validation rejects or never touches.
 */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "attn.h"

static int failures = 0;
#define EXPECT(call, want)                                                       \
    do {                                                                         \
        int got_ = (call);                                                       \
        if (got_ != (want)) {                                                    \
            fprintf(stderr, "FAILED line %d: %s -> %d, want %d\n", __LINE__,    \
                    #call, got_, (int)(want));                                   \
            failures++;                                                          \
        }                                                                        \
    } while (0)

int main(void)
{
    void *P = (void *)(uintptr_t)4096;     /* placeholder device pointer */
    const int32_t *I = (const int32_t *)P;
    float tab[64];
    EXPECT(attn_rope_inv_freq(128, 1e4, tab), ATTN_OK);
    EXPECT(attn_rope_inv_freq(7, 1e4, tab), ATTN_EINVAL);
    EXPECT(attn_yarn_inv_freq(128, 1e6, 4.0, 32768, 32.0, 1.0, tab), ATTN_OK);
    EXPECT(attn_yarn_inv_freq(128, 1e6, 0.0, 32768, 32.0, 1.0, tab), ATTN_EINVAL);
    EXPECT(attn_rope_apply(P, P, ATTN_BF16, 4, 4, 96, 1, I, I, 4, (const float *)P, 64, 1.f, 0, NULL, 1e-6, NULL),
           ATTN_EUNSUPPORTED);
    EXPECT(attn_rope_apply(P, P, ATTN_BF16, 4, 4, 128, 1, I, I, 4, (const float *)P, 63, 1.f, 0, NULL, 1e-6, NULL),
           ATTN_EINVAL);
    EXPECT(attn_kv_append(P, P, ATTN_BF16, 1, 2, 128, 256, 0, P, P, 16, I, I, 16, 300, (const float *)P, 128, 1.f,
                          0, NULL, 1e-6, 0, NULL), ATTN_ECAPACITY);
    EXPECT(attn_kv_append(P, P, ATTN_BF16, 1, 2, 128, 256, 1, P, P, 257, I, I, 257, 600, (const float *)P, 128,
                          1.f, 0, NULL, 1e-6, 0, NULL), ATTN_ECAPACITY);
    EXPECT(attn_rope_qkv(P, P, 8, P, P, P, P, 2, 256, 3, ATTN_BF16, 16, 128, 1, I, I, 16, 64, (const float *)P,
                         128, 1.f, 0, NULL, NULL, 1e-6, 0, NULL), ATTN_EINVAL);
    EXPECT(attn_prefill_chunk(P, P, P, ATTN_BF16, 1, 8, 2, 128, 256, 0, 16, I, I, 16, 257, 0.088f, 0, NULL, 0,
                              0, (float *)P, NULL, 0, NULL), ATTN_ECAPACITY);
    EXPECT(attn_prefill_chunk(P, P, P, ATTN_BF16, 1, 6, 4, 128, 256, 0, 16, I, I, 16, 64, 0.088f, 0, NULL, 0, 0,
                              (float *)P, NULL, 0, NULL), ATTN_EINVAL);
    EXPECT(attn_prefill_chunk(P, P, P, ATTN_BF16, 1, 8, 2, 128, 200, 1, 16, I, I, 16, 300, 0.088f, 100, NULL, 0,
                              0, (float *)P, NULL, 0, NULL), ATTN_EUNSUPPORTED);
    EXPECT(attn_prefill_chunk(P, P, P, ATTN_BF16, 0, 8, 2, 128, 256, 0, 16, I, I, 16, 64, 0.088f, 0, NULL, 0, 0,
                              (float *)P, NULL, 0, NULL), ATTN_OK);
    EXPECT(attn_decode(P, P, P, ATTN_BF16, 4, 64, 2, 128, 4096, 0, I, 4096, 0.088f, 0, NULL, 0, 0, (float *)P,
                       NULL, 0, P, 1 << 30, NULL), ATTN_EUNSUPPORTED);
    EXPECT(attn_decode(P, P, P, ATTN_BF16, 4, 32, 8, 128, 4096, 0, I, 4097, 0.088f, 0, NULL, 0, 0, (float *)P,
                       NULL, 0, P, 1 << 30, NULL), ATTN_ECAPACITY);
    EXPECT(attn_decode(P, P, P, ATTN_BF16, 4, 32, 8, 128, 4096, 0, I, 4096, 0.088f, 0, NULL, 0, 0, (float *)P,
                       (float *)P, 100, P, 1 << 30, NULL), ATTN_EINVAL);
    EXPECT(attn_decode_noalloc(P, P, P, ATTN_BF16, 4096, 32, 8, 128, 4096, 0, I, 4096, 0.088f, 0, NULL, 0, 0,
                               (float *)P, NULL, 0, NULL), ATTN_ESCRATCH);
    EXPECT(attn_decode_importance((const float *)P, 4, 32, 100, I, 4096, (float *)P, 4096, 1, NULL),
           ATTN_EINVAL);
    EXPECT(attn_calibrate_read(P, 15, 8, (uint32_t *)P, NULL), ATTN_EINVAL);
    EXPECT(attn_calibrate_mfma(0, 8, 1, (float *)P, NULL), ATTN_EINVAL);
    EXPECT(attn_calibrate_mfma(4, 8, 2, (float *)P, NULL), ATTN_EINVAL);
    /* the deferred chunk step: records it did not write are refused; with
       nothing to attend and nothing owed it launches nothing */
    {
        attn_prefill_pending rec, bad;
        memset(&rec, 0, sizeof(rec));
        memset(&bad, 0, sizeof(bad));
        bad.active = 1;
        bad.head_dim = 96;
        EXPECT(attn_prefill_chunk_deferred(P, P, P, ATTN_BF16, 1, 8, 2, 128, 256, 0, 16, I, I, 16, 64, 0.088f, 0,
                                           NULL, 0, 0, (float *)P, NULL, 0, NULL, NULL, NULL, NULL),
               ATTN_EINVAL);
        EXPECT(attn_prefill_chunk_deferred(P, P, P, ATTN_BF16, 1, 8, 2, 128, 256, 0, 16, I, I, 16, 64, 0.088f, 0,
                                           NULL, 0, 0, (float *)P, NULL, 0, NULL, &bad, &rec, NULL),
               ATTN_EINVAL);
        EXPECT(attn_prefill_chunk_deferred(P, P, P, ATTN_BF16, 1, 8, 2, 128, 256, 0, 16, I, I, 16, 257, 0.088f, 0,
                                           NULL, 0, 0, (float *)P, NULL, 0, NULL, NULL, &rec, NULL),
               ATTN_ECAPACITY);
        rec.active = 1;
        EXPECT(attn_prefill_chunk_deferred(P, P, P, ATTN_BF16, 0, 8, 2, 128, 256, 0, 16, I, I, 16, 64, 0.088f, 0,
                                           NULL, 0, 0, (float *)P, NULL, 0, NULL, NULL, &rec, NULL),
               ATTN_OK);
        EXPECT(rec.active, 0);
        EXPECT(attn_prefill_finish(&rec, NULL), ATTN_OK);
        EXPECT(attn_prefill_finish(&bad, NULL), ATTN_EINVAL);
        bad.head_dim = 128;       /* a valid size, but not a record the library wrote */
        EXPECT(attn_prefill_finish(&bad, NULL), ATTN_EINVAL);
        EXPECT(attn_prefill_chunk_deferred(P, P, P, ATTN_BF16, 1, 8, 2, 128, 256, 0, 16, I, I, 16, 64, 0.088f, 0,
                                           NULL, 0, 0, (float *)P, NULL, 0, NULL, &bad, &rec, NULL),
               ATTN_EINVAL);
        EXPECT(attn_prefill_finish(NULL, NULL), ATTN_EINVAL);
    }
    /* planners: sizes from host scalars only */
    size_t ws = attn_prefill_workspace_bytes(1, 32, 8, 128, 128, 128, 4096);
    if (!(ws > 256 && (ws - 256) % (128 * (16 + 2 * 128)) == 0)) {
        fprintf(stderr, "FAILED: prefill workspace %zu\n", ws);
        failures++;
    }
    if (attn_prefill_workspace_bytes(8, 40, 8, 128, 2048, 256, 8192) == 0) {
        fprintf(stderr, "FAILED: varlen prefill workspace\n");
        failures++;
    }
    if (attn_decode_workspace_bytes(64, 32, 8, 128, 32768) != (size_t)64 * 32 * 32 * (16 + 2 * 128)) {
        fprintf(stderr, "FAILED: decode workspace\n");
        failures++;
    }
    for (int s = -6; s <= 1; s++)
        if (!attn_status_string(s) || !strlen(attn_status_string(s))) failures++;
    if (failures) return 1;
    printf("library host sanitizer check ok (%s)\n", attn_version());
    return 0;
}
