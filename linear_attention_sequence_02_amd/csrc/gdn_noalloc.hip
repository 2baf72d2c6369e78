// gdn_prefill_noalloc: gdn_prefill for callers that cannot allocate device
// memory (code under graph capture, tight serving loops, harnesses that forbid
// hipMalloc). The bf16 prefill's segment workspace lives in a file-scope device
// array instead of a caller-supplied buffer.
//
// Every GPU the library runs on holds its own copy of `scratch` (kScratchBytes)
// from the moment the library's code object is loaded on it until the process
// ends. All calls on one GPU share that copy and leave the last call's
// contents in it: two calls that overlap on one GPU (different streams, or
// different host threads without ordering) race on it. The workspace needs no
// clearing: every byte a call reads was written earlier in the same call.
//
// In host code the array's name is only a host-side stand-in, so the device
// address is looked up once per device with hipGetSymbolAddress (with that
// device current) and cached; only that address is ever passed to kernels.
#include "../../include/gdn.h"
#include "gdn_internal.h"

#include <mutex>

namespace {

constexpr size_t kScratchBytes = GDN_PREFILL_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device (looked up on the first call per device).
hipError_t scratch_on_current_device(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (p == nullptr) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

}  // namespace

extern "C" {

gdn_status_t gdn_prefill_noalloc(const void* q, const void* k, const void* v, const float* g, const float* beta,
                                 const float* initial_state, const int32_t* cu_seqlens, int32_t num_seqs,
                                 int64_t total_tokens, int32_t num_qk_heads, int32_t num_v_heads, int32_t d_k,
                                 int32_t d_v, float scale, gdn_dtype_t dtype, void* out, float* final_state,
                                 void* stream) {
    const size_t need = gdn_prefill_workspace_size(total_tokens, num_seqs, num_qk_heads, num_v_heads, d_k, d_v,
                                                   dtype);
    if (need > kScratchBytes) return GDN_ERR_SCRATCH_LIMIT;
    void* ws = nullptr;
    if (need > 0) {
        if (scratch_on_current_device(&ws) != hipSuccess) return GDN_ERR_HIP;
    }
    // The rest (argument checks, kernels) is gdn_prefill's, with the static array as its workspace.
    return gdn_prefill(q, k, v, g, beta, initial_state, cu_seqlens, num_seqs, total_tokens, num_qk_heads,
                       num_v_heads, d_k, d_v, scale, dtype, out, final_state, ws, need > 0 ? kScratchBytes : 0,
                       stream);
}

}  // extern "C"
