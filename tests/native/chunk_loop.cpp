// Native client of the C ABI (test infrastructure): a bf16 chunked prefill of
// one prompt driven from C++ with hipMalloc'd buffers and no PyTorch --
// attn_rope_qkv on the first chunk, then per chunk attn_prefill_chunk_deferred
// (attend it, finish the next chunk, merge the previous one's split parts)
// with two alternating workspaces, and attn_prefill_finish after the last.
// Checked against the CPU oracle (oracle/oracle.c, linked): the key cache bit
// for bit against the oracle's finished and rounded keys, every output row
// within 2e-2 of the oracle row's RMS.  The inputs come from a seeded
// splitmix64 generator here, fed to both sides.  Built as a shared library
// whose one entry point, chunk_loop_check, returns 0 on success and writes a
// one-line report.
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include "attn.h"

extern "C" {
void orc_rope_inv_freq(int rd, double base, float* out);
void orc_finish_heads(double* x, int n_tok, int n_heads, int hd, const int64_t* pos, const float* inv_freq,
                      int rd, double rope_scale, int norm_style, const float* norm_w, double eps,
                      int store_dtype, int n_threads);
int orc_attend(const double* q, const double* kc, const double* vc, int n_tok, int nh, int nkv, int hd,
               long cap, const int64_t* qpos, double scale, double* out, double* probs, long probs_ld,
               int n_threads);
}

namespace {

constexpr int kStoreBf16 = 1;

#define CHECK_HIP(x)                                                                          \
    do {                                                                                      \
        hipError_t e_ = (x);                                                                  \
        if (e_ != hipSuccess) {                                                               \
            std::fprintf(stderr, "%s:%d %s: %s\n", __FILE__, __LINE__, #x, hipGetErrorString(e_)); \
            return 2;                                                                         \
        }                                                                                     \
    } while (0)
#define CHECK_ATTN(x)                                                                         \
    do {                                                                                      \
        int s_ = (x);                                                                         \
        if (s_ != ATTN_OK) {                                                                  \
            std::fprintf(stderr, "%s:%d %s: %s\n", __FILE__, __LINE__, #x, attn_status_string(s_)); \
            return 3;                                                                         \
        }                                                                                     \
    } while (0)

// splitmix64 (Steele, Lea and Flood), mapped to roughly N(0, 1) by a sum of
// four uniforms
struct Rng {
    uint64_t s;
    uint64_t next() {
        uint64_t z = (s += 0x9e3779b97f4a7c15ull);
        z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
        z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
        return z ^ (z >> 31);
    }
    double normalish() {
        double u = 0.0;
        for (int i = 0; i < 4; ++i) u += (double)(next() >> 11) * (1.0 / 9007199254740992.0);
        return (u - 2.0) * std::sqrt(3.0);
    }
};

// round to bfloat16 (nearest even) and back, for the inputs both sides read
uint16_t to_bf16(float f) {
    uint32_t u;
    std::memcpy(&u, &f, 4);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}
double from_bf16(uint16_t h) {
    uint32_t u = (uint32_t)h << 16;
    float f;
    std::memcpy(&f, &u, 4);
    return f;
}

}  // namespace

extern "C" int chunk_loop_check(char* report, int report_len) {
    const int T = 700, chunk = 128, nh = 32, nkv = 8, hd = 128, rd = 128, cap = 768;
    const double base = 1e4;
    const float scale = 1.f / std::sqrt((float)hd);
    const int n_chunks = (T + chunk - 1) / chunk;

    // inputs, rounded to bf16
    Rng rng{20260601ull};
    std::vector<uint16_t> q((size_t)T * nh * hd), k((size_t)T * nkv * hd), v((size_t)T * nkv * hd);
    for (auto& x : q) x = to_bf16((float)rng.normalish());
    for (auto& x : k) x = to_bf16((float)rng.normalish());
    for (auto& x : v) x = to_bf16((float)rng.normalish());
    std::vector<float> inv_freq(rd / 2);
    CHECK_ATTN(attn_rope_inv_freq(rd, base, inv_freq.data()));

    // device buffers
    void *dq, *dk, *dv, *dqr, *dkc, *dvc, *dout, *dfreq, *dws[2];
    int32_t* dbatch;
    CHECK_HIP(hipMalloc(&dq, q.size() * 2));
    CHECK_HIP(hipMalloc(&dk, k.size() * 2));
    CHECK_HIP(hipMalloc(&dv, v.size() * 2));
    CHECK_HIP(hipMalloc(&dqr, q.size() * 2));
    CHECK_HIP(hipMalloc(&dkc, (size_t)nkv * cap * hd * 2));
    CHECK_HIP(hipMalloc(&dvc, (size_t)nkv * cap * hd * 2));
    CHECK_HIP(hipMalloc(&dout, (size_t)T * nh * hd * 4));
    CHECK_HIP(hipMalloc(&dfreq, inv_freq.size() * 4));
    CHECK_HIP(hipMalloc(&dbatch, (size_t)n_chunks * 3 * sizeof(int32_t)));
    size_t wsb = 16;
    for (int c = 0; c < n_chunks; ++c) {
        const int len = std::min(chunk, T - c * chunk);
        const size_t b = attn_prefill_workspace_bytes(1, nh, nkv, hd, len, len, c * chunk + len);
        if (b > wsb) wsb = b;
    }
    CHECK_HIP(hipMalloc(&dws[0], wsb));
    CHECK_HIP(hipMalloc(&dws[1], wsb));
    CHECK_HIP(hipMemcpy(dq, q.data(), q.size() * 2, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(dk, k.data(), k.size() * 2, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(dv, v.data(), v.size() * 2, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(dfreq, inv_freq.data(), inv_freq.size() * 4, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemset(dkc, 0, (size_t)nkv * cap * hd * 2));
    CHECK_HIP(hipMemset(dvc, 0, (size_t)nkv * cap * hd * 2));
    // per chunk: cu_seq = {0, len}, start = {first position}
    std::vector<int32_t> batch((size_t)n_chunks * 3);
    for (int c = 0; c < n_chunks; ++c) {
        batch[3 * c] = 0;
        batch[3 * c + 1] = std::min(chunk, T - c * chunk);
        batch[3 * c + 2] = c * chunk;
    }
    CHECK_HIP(hipMemcpy(dbatch, batch.data(), batch.size() * sizeof(int32_t), hipMemcpyHostToDevice));

    auto rope_args = [&](int c) {
        const int len = batch[3 * c + 1], p0 = batch[3 * c + 2];
        attn_rope_qkv_args r{};
        r.q = (const char*)dq + (size_t)p0 * nh * hd * 2;
        r.q_out = (char*)dqr + (size_t)p0 * nh * hd * 2;
        r.n_heads = nh;
        r.k_cache = dkc;
        r.v_cache = dvc;
        r.k_new = (const char*)dk + (size_t)p0 * nkv * hd * 2;
        r.v_new = (const char*)dv + (size_t)p0 * nkv * hd * 2;
        r.n_kv = nkv;
        r.cap = cap;
        r.ring = 0;
        r.dtype = ATTN_BF16;
        r.n_tok = len;
        r.head_dim = hd;
        r.n_seq = 1;
        r.cu_seq = dbatch + 3 * c;
        r.start = dbatch + 3 * c + 2;
        r.max_chunk = len;
        r.max_end = p0 + len;
        r.inv_freq = (const float*)dfreq;
        r.rotary_dim = rd;
        r.rope_scale = 1.f;
        r.norm = ATTN_NORM_NONE;
        r.eps = 1e-6;
        r.v_norm = 0;
        return r;
    };

    // the chunk loop
    {
        const attn_rope_qkv_args r0 = rope_args(0);
        CHECK_ATTN(attn_rope_qkv(r0.q, r0.q_out, r0.n_heads, r0.k_cache, r0.v_cache, r0.k_new, r0.v_new, r0.n_kv,
                                 r0.cap, r0.ring, r0.dtype, r0.n_tok, r0.head_dim, r0.n_seq, r0.cu_seq, r0.start,
                                 r0.max_chunk, r0.max_end, r0.inv_freq, r0.rotary_dim, r0.rope_scale, r0.norm,
                                 r0.q_norm_w, r0.k_norm_w, r0.eps, r0.v_norm, nullptr));
    }
    attn_prefill_pending rec[2];
    std::memset(rec, 0, sizeof(rec));
    int owed = 0;
    for (int c = 0; c < n_chunks; ++c) {
        const int len = batch[3 * c + 1], p0 = batch[3 * c + 2];
        attn_rope_qkv_args nxt{};
        if (c + 1 < n_chunks) nxt = rope_args(c + 1);
        CHECK_ATTN(attn_prefill_chunk_deferred(
            (const char*)dqr + (size_t)p0 * nh * hd * 2, dkc, dvc, ATTN_BF16, 1, nh, nkv, hd, cap, 0, len,
            dbatch + 3 * c, dbatch + 3 * c + 2, len, p0 + len, scale, 0, nullptr, 0, 0,
            (float*)dout + (size_t)p0 * nh * hd, dws[c % 2], wsb, c + 1 < n_chunks ? &nxt : nullptr,
            c > 0 ? &rec[(c - 1) % 2] : nullptr, &rec[c % 2], nullptr));
        owed += rec[c % 2].active;
    }
    CHECK_ATTN(attn_prefill_finish(&rec[(n_chunks - 1) % 2], nullptr));
    CHECK_HIP(hipDeviceSynchronize());

    std::vector<float> out((size_t)T * nh * hd);
    std::vector<uint16_t> kc((size_t)nkv * cap * hd);
    CHECK_HIP(hipMemcpy(out.data(), dout, out.size() * 4, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(kc.data(), dkc, kc.size() * 2, hipMemcpyDeviceToHost));

    // the oracle: finished and rounded Q and K, the cache, causal attention
    std::vector<int64_t> pos(T);
    for (int t = 0; t < T; ++t) pos[t] = t;
    std::vector<float> ofreq(rd / 2);
    orc_rope_inv_freq(rd, base, ofreq.data());
    std::vector<double> oq(q.size()), ok(k.size()), ov(v.size());
    for (size_t i = 0; i < q.size(); ++i) oq[i] = from_bf16(q[i]);
    for (size_t i = 0; i < k.size(); ++i) ok[i] = from_bf16(k[i]);
    for (size_t i = 0; i < v.size(); ++i) ov[i] = from_bf16(v[i]);
    orc_finish_heads(oq.data(), T, nh, hd, pos.data(), ofreq.data(), rd, 1.0, 0, nullptr, 1e-6, kStoreBf16, 8);
    orc_finish_heads(ok.data(), T, nkv, hd, pos.data(), ofreq.data(), rd, 1.0, 0, nullptr, 1e-6, kStoreBf16, 8);
    std::vector<double> okc((size_t)nkv * cap * hd, 0.0), ovc((size_t)nkv * cap * hd, 0.0);
    for (int t = 0; t < T; ++t)
        for (int g = 0; g < nkv; ++g)
            for (int d = 0; d < hd; ++d) {
                okc[((size_t)g * cap + t) * hd + d] = ok[((size_t)t * nkv + g) * hd + d];
                ovc[((size_t)g * cap + t) * hd + d] = ov[((size_t)t * nkv + g) * hd + d];
            }
    std::vector<double> oref((size_t)T * nh * hd);
    if (orc_attend(oq.data(), okc.data(), ovc.data(), T, nh, nkv, hd, cap, pos.data(), (double)scale, oref.data(),
                   nullptr, 0, 8) != 0) {
        std::fprintf(stderr, "oracle attend failed\n");
        return 4;
    }

    // the key cache: bit for bit
    long key_mismatch = 0;
    for (int g = 0; g < nkv; ++g)
        for (int t = 0; t < T; ++t)
            for (int d = 0; d < hd; ++d) {
                const size_t i = ((size_t)g * cap + t) * hd + d;
                if (from_bf16(kc[i]) != okc[i]) ++key_mismatch;
            }
    // outputs: every row within 2e-2 of its RMS
    double worst = 0.0;
    for (int r = 0; r < T * nh; ++r) {
        double ss = 0.0, e = 0.0;
        for (int d = 0; d < hd; ++d) {
            const double x = oref[(size_t)r * hd + d];
            ss += x * x;
            e = std::fmax(e, std::fabs((double)out[(size_t)r * hd + d] - x));
        }
        const double rms = std::sqrt(ss / hd);
        worst = std::fmax(worst, e / rms);
    }
    std::snprintf(report, (size_t)report_len,
                  "%d chunks, %d merges deferred, key cache mismatches %ld, worst row err/rms %.3e", n_chunks,
                  owed, key_mismatch, worst);
    for (void* p : {dq, dk, dv, dqr, dkc, dvc, dout, dfreq, dws[0], dws[1], (void*)dbatch}) (void)hipFree(p);
    return key_mismatch == 0 && worst <= 2e-2 && owed > 0 ? 0 : 1;
}
