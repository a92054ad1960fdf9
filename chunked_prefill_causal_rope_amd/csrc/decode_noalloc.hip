// attn_decode without a caller workspace: the split partials live in a
// file-scope device array of this library (ATTN_NOALLOC_SCRATCH_BYTES per
// GPU, zero when the library is loaded), for callers that cannot allocate
// device memory.  The array's device address is taken once per device with
// hipGetSymbolAddress; host code never uses the array's name as an address.
#include <atomic>
#include <mutex>

#include <hip/hip_runtime.h>

#include "../../include/attn.h"
#include "launch.h"

namespace attn {

static __device__ __align__(256) unsigned char scratch[ATTN_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
static std::atomic<void*> g_scratch_ptr[kMaxDevices];
static std::mutex g_scratch_mu;

// Device address of this device's copy of the scratch array (current device),
// or nullptr when it cannot be obtained.
static void* scratch_address(int dev) {
    if (dev < 0 || dev >= kMaxDevices) return nullptr;
    void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (p) return p;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (!p) {
        void* addr = nullptr;
        if (hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch)) != hipSuccess || !addr) return nullptr;
        p = addr;
        g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
    return p;
}

}  // namespace attn

extern "C" {

int attn_decode_noalloc(const void* q, const void* k_cache, const void* v_cache, int dtype, int n_seq,
                        int n_heads, int n_kv, int head_dim, int cap, int ring, const int32_t* ctx,
                        int max_ctx, float scale, int window, const void* gate, int gate_mode,
                        int gate_ld, float* out, float* probs, int probs_ld, void* stream) {
    // f32 uses no scratch; bf16 needs at least one part per row in it
    if (dtype == ATTN_BF16 && n_seq > 0 && n_heads > 0 && (head_dim == 64 || head_dim == 128) &&
        attn::decode_min_workspace_bytes(n_seq, n_heads, head_dim) > (size_t)ATTN_NOALLOC_SCRATCH_BYTES)
        return ATTN_ESCRATCH;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return ATTN_EDEVICE;
    void* ws = attn::scratch_address(dev);
    if (!ws) return ATTN_EDEVICE;
    return attn::decode_impl(q, k_cache, v_cache, dtype, n_seq, n_heads, n_kv, head_dim, cap, ring, ctx,
                             max_ctx, scale, window, gate, gate_mode, gate_ld, out, probs, probs_ld, ws,
                             (size_t)ATTN_NOALLOC_SCRATCH_BYTES, stream);
}

}  // extern "C"
