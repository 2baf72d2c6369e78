// C ABI of libgdn (declarations and contracts in include/gdn.h).
//
// Host side only: argument validation, workspace accounting and kernel
// dispatch on the caller's stream. No allocation, no host synchronisation.
#include "../../include/gdn.h"
#include "gdn_internal.h"

#include <stdint.h>

namespace {

bool fp32_head_size_ok(int32_t d) { return d == 16 || d == 32 || d == 64 || d == 128; }

gdn_status_t check_heads(int32_t hqk, int32_t hv, int32_t dk, int32_t dv, gdn_dtype_t dt) {
    if (hqk <= 0 || hv <= 0 || dk <= 0 || dv <= 0) return GDN_ERR_INVALID_ARG;
    if (hv % hqk != 0) return GDN_ERR_INVALID_ARG;
    if (dt != GDN_BF16 && dt != GDN_FP32) return GDN_ERR_INVALID_ARG;
    if (dk != dv) return GDN_ERR_UNSUPPORTED;
    if (dt == GDN_BF16 && dk != 128) return GDN_ERR_UNSUPPORTED;
    if (dt == GDN_FP32 && !fp32_head_size_ok(dk)) return GDN_ERR_UNSUPPORTED;
    return GDN_OK;
}

gdn_status_t hip_status(hipError_t e) { return e == hipSuccess ? GDN_OK : GDN_ERR_HIP; }

constexpr uint32_t kKnownFlags = GDN_FLAG_QK_L2NORM;

}  // namespace

extern "C" {

size_t gdn_prefill_workspace_size(int64_t total_tokens, int32_t num_seqs, int32_t num_qk_heads,
                                  int32_t num_v_heads, int32_t d_k, int32_t d_v, gdn_dtype_t dtype) {
    if (total_tokens < 0 || num_seqs < 0) return 0;
    if (check_heads(num_qk_heads, num_v_heads, d_k, d_v, dtype) != GDN_OK) return 0;
    if (dtype == GDN_FP32) return 0;
    return gdn::prefill_bf16_workspace_bytes(total_tokens, num_seqs, num_qk_heads, num_v_heads);
}

int32_t gdn_prefill_segment_chunks(int64_t total_tokens, int32_t num_seqs, int32_t num_qk_heads,
                                   int32_t num_v_heads, int32_t d_k, int32_t d_v, gdn_dtype_t dtype) {
    if (total_tokens < 0 || num_seqs < 0) return 0;
    if (check_heads(num_qk_heads, num_v_heads, d_k, d_v, dtype) != GDN_OK) return 0;
    if (dtype == GDN_FP32) return 0;
    return gdn::cp_segment_chunks(total_tokens, num_seqs, num_v_heads);
}

}  // extern "C"

namespace {

// Shared body of gdn_prefill and gdn_prefill_slots.
gdn_status_t prefill_impl(const void* q, const void* k, const void* v, const float* g, const float* beta,
                          const float* initial_state, const int32_t* cu_seqlens, int32_t num_seqs,
                          int64_t total_tokens, int32_t num_qk_heads, int32_t num_v_heads, int32_t d_k,
                          int32_t d_v, float scale, gdn_dtype_t dtype, void* out, float* final_state,
                          void* workspace, size_t workspace_bytes, void* stream,
                          const int32_t* state_indices, const int32_t* has_initial, int32_t num_slots,
                          uint32_t flags = 0) {
    gdn_status_t st = check_heads(num_qk_heads, num_v_heads, d_k, d_v, dtype);
    if (st != GDN_OK) return st;
    if (flags & ~kKnownFlags) return GDN_ERR_INVALID_ARG;
    if (total_tokens < 0 || num_seqs < 0) return GDN_ERR_INVALID_ARG;
    if (total_tokens > INT32_MAX) return GDN_ERR_UNSUPPORTED;   // cu_seqlens are int32
    if (cu_seqlens == nullptr && num_seqs != 1) return GDN_ERR_INVALID_ARG;
    if (total_tokens > 0 && (!q || !k || !v || !g || !beta || !out)) return GDN_ERR_INVALID_ARG;
    if (num_seqs == 0) return GDN_OK;
    const size_t need = gdn_prefill_workspace_size(total_tokens, num_seqs, num_qk_heads, num_v_heads,
                                                   d_k, d_v, dtype);
    if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return GDN_ERR_WORKSPACE;
    if (total_tokens == 0 && final_state == nullptr) return GDN_OK;

    gdn::PrefillArgs a;
    a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta;
    a.initial_state = initial_state; a.cu_seqlens = cu_seqlens; a.final_state = final_state;
    a.state_indices = state_indices; a.has_initial = has_initial; a.num_slots = num_slots;
    a.out = out; a.workspace = workspace; a.workspace_bytes = workspace_bytes;
    a.total_tokens = total_tokens; a.num_seqs = num_seqs; a.num_qk_heads = num_qk_heads;
    a.num_v_heads = num_v_heads; a.d = d_k; a.scale = scale; a.bf16 = (dtype == GDN_BF16);
    a.qk_norm = (flags & GDN_FLAG_QK_L2NORM) != 0;
    hipStream_t s = static_cast<hipStream_t>(stream);
    return hip_status(a.bf16 ? gdn::launch_prefill_bf16(a, s) : gdn::launch_prefill_f32(a, s));
}

// Shared body of gdn_decode_step, gdn_decode_step_slots and gdn_decode_multi.
gdn_status_t decode_impl(const void* q, const void* k, const void* v, const float* g, const float* beta,
                         float* state, int32_t num_seqs, int32_t num_qk_heads, int32_t num_v_heads,
                         int32_t d_k, int32_t d_v, float scale, gdn_dtype_t dtype, void* out, void* stream,
                         const int32_t* state_indices, int32_t num_slots, int32_t num_tokens = 1,
                         float* token_states = nullptr, bool multi = false, uint32_t flags = 0) {
    if (num_qk_heads <= 0 || num_v_heads <= 0 || d_k <= 0 || d_v <= 0 || num_seqs < 0)
        return GDN_ERR_INVALID_ARG;
    if (flags & ~kKnownFlags) return GDN_ERR_INVALID_ARG;
    if (num_v_heads % num_qk_heads != 0) return GDN_ERR_INVALID_ARG;
    if (dtype != GDN_BF16 && dtype != GDN_FP32) return GDN_ERR_INVALID_ARG;
    if (d_k != d_v || !fp32_head_size_ok(d_k)) return GDN_ERR_UNSUPPORTED;
    if (num_seqs == 0) return GDN_OK;
    if (!q || !k || !v || !g || !beta || !out) return GDN_ERR_INVALID_ARG;
    if (!state && !(state_indices && num_slots == 0)) return GDN_ERR_INVALID_ARG;
    if ((int64_t)num_seqs * num_v_heads > INT32_MAX) return GDN_ERR_UNSUPPORTED;
    if ((int64_t)num_seqs * num_tokens * num_v_heads > INT32_MAX) return GDN_ERR_UNSUPPORTED;
    gdn::DecodeArgs a;
    a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta; a.state = state; a.out = out;
    a.state_indices = state_indices; a.num_slots = num_slots;
    a.num_seqs = num_seqs; a.num_qk_heads = num_qk_heads; a.num_v_heads = num_v_heads; a.d = d_k;
    a.scale = scale; a.bf16 = (dtype == GDN_BF16);
    a.num_tokens = num_tokens; a.token_states = token_states;
    a.qk_norm = (flags & GDN_FLAG_QK_L2NORM) != 0;
    hipStream_t s = static_cast<hipStream_t>(stream);
    return hip_status(multi ? gdn::launch_decode_multi(a, s) : gdn::launch_decode(a, s));
}

// Shared body of gdn_decode_ex and gdn_decode_multi: token count, state and pool checks, then the
// multi-token kernel (multi) or the single-step one.
gdn_status_t decode_ex_impl(const void* q, const void* k, const void* v, const float* g, const float* beta,
                            float* state, const int32_t* state_indices, int32_t num_slots, int32_t num_seqs,
                            int32_t num_tokens, int32_t num_qk_heads, int32_t num_v_heads, int32_t d_k, int32_t d_v,
                            float scale, gdn_dtype_t dtype, uint32_t flags, void* out, float* token_states,
                            void* stream, bool multi) {
    if (num_tokens < 1) return GDN_ERR_INVALID_ARG;
    if (num_tokens > 64) return GDN_ERR_UNSUPPORTED;
    if (state_indices) {
        if (num_slots < 0) return GDN_ERR_INVALID_ARG;
        if (num_slots > 0 && state == nullptr) return GDN_ERR_INVALID_ARG;
    } else {
        if (num_seqs > 0 && state == nullptr) return GDN_ERR_INVALID_ARG;
        num_slots = 0;
    }
    return decode_impl(q, k, v, g, beta, state, num_seqs, num_qk_heads, num_v_heads, d_k, d_v, scale, dtype, out,
                       stream, state_indices, num_slots, num_tokens, token_states, multi, flags);
}

}  // namespace

extern "C" {

gdn_status_t gdn_prefill(const void* q, const void* k, const void* v, const float* g, const float* beta,
                         const float* initial_state, const int32_t* cu_seqlens, int32_t num_seqs,
                         int64_t total_tokens, int32_t num_qk_heads, int32_t num_v_heads, int32_t d_k,
                         int32_t d_v, float scale, gdn_dtype_t dtype, void* out, float* final_state,
                         void* workspace, size_t workspace_bytes, void* stream) {
    return prefill_impl(q, k, v, g, beta, initial_state, cu_seqlens, num_seqs, total_tokens, num_qk_heads,
                        num_v_heads, d_k, d_v, scale, dtype, out, final_state, workspace, workspace_bytes, stream,
                        nullptr, nullptr, 0);
}

gdn_status_t gdn_prefill_slots(const void* q, const void* k, const void* v, const float* g, const float* beta,
                               float* state_pool, const int32_t* state_indices, const int32_t* has_initial_state,
                               int32_t num_slots, const int32_t* cu_seqlens, int32_t num_seqs,
                               int64_t total_tokens, int32_t num_qk_heads, int32_t num_v_heads, int32_t d_k,
                               int32_t d_v, float scale, gdn_dtype_t dtype, void* out, void* workspace,
                               size_t workspace_bytes, void* stream) {
    if (num_slots < 0) return GDN_ERR_INVALID_ARG;
    if (num_seqs > 0 && state_indices == nullptr) return GDN_ERR_INVALID_ARG;
    if (num_slots > 0 && state_pool == nullptr) return GDN_ERR_INVALID_ARG;
    return prefill_impl(q, k, v, g, beta, state_pool, cu_seqlens, num_seqs, total_tokens, num_qk_heads,
                        num_v_heads, d_k, d_v, scale, dtype, out, state_pool, workspace, workspace_bytes, stream,
                        state_indices, has_initial_state, num_slots);
}

gdn_status_t gdn_decode_step(const void* q, const void* k, const void* v, const float* g, const float* beta,
                             float* state, int32_t num_seqs, int32_t num_qk_heads, int32_t num_v_heads,
                             int32_t d_k, int32_t d_v, float scale, gdn_dtype_t dtype, void* out,
                             void* stream) {
    if (num_seqs > 0 && state == nullptr) return GDN_ERR_INVALID_ARG;
    return decode_impl(q, k, v, g, beta, state, num_seqs, num_qk_heads, num_v_heads, d_k, d_v, scale, dtype, out,
                       stream, nullptr, 0);
}

gdn_status_t gdn_decode_ex(const void* q, const void* k, const void* v, const float* g, const float* beta,
                           float* state, const int32_t* state_indices, int32_t num_slots, int32_t num_seqs,
                           int32_t num_tokens, int32_t num_qk_heads, int32_t num_v_heads, int32_t d_k, int32_t d_v,
                           float scale, gdn_dtype_t dtype, uint32_t flags, void* out, float* token_states,
                           void* stream) {
    return decode_ex_impl(q, k, v, g, beta, state, state_indices, num_slots, num_seqs, num_tokens, num_qk_heads,
                          num_v_heads, d_k, d_v, scale, dtype, flags, out, token_states, stream,
                          num_tokens > 1 || token_states != nullptr);
}

gdn_status_t gdn_decode_multi(const void* q, const void* k, const void* v, const float* g, const float* beta,
                              float* state, const int32_t* state_indices, int32_t num_slots, int32_t num_seqs,
                              int32_t num_tokens, int32_t num_qk_heads, int32_t num_v_heads, int32_t d_k, int32_t d_v,
                              float scale, gdn_dtype_t dtype, void* out, float* token_states, void* stream) {
    return decode_ex_impl(q, k, v, g, beta, state, state_indices, num_slots, num_seqs, num_tokens, num_qk_heads,
                          num_v_heads, d_k, d_v, scale, dtype, 0, out, token_states, stream, true);
}

gdn_status_t gdn_prefill_ex(const void* q, const void* k, const void* v, const float* g, const float* beta,
                            const float* initial_state, float* final_state, const int32_t* state_indices,
                            const int32_t* has_initial_state, int32_t num_slots, const int32_t* cu_seqlens,
                            int32_t num_seqs, int64_t total_tokens, int32_t num_qk_heads, int32_t num_v_heads,
                            int32_t d_k, int32_t d_v, float scale, gdn_dtype_t dtype, uint32_t flags, void* out,
                            void* workspace, size_t workspace_bytes, void* stream) {
    if (state_indices) {
        if (num_slots < 0) return GDN_ERR_INVALID_ARG;
    } else {
        has_initial_state = nullptr;   // plain arrays: every sequence reads initial_state (if given)
        num_slots = 0;
    }
    return prefill_impl(q, k, v, g, beta, initial_state, cu_seqlens, num_seqs, total_tokens, num_qk_heads,
                        num_v_heads, d_k, d_v, scale, dtype, out, final_state, workspace, workspace_bytes, stream,
                        state_indices, has_initial_state, num_slots, flags);
}

gdn_status_t gdn_decode_step_slots(const void* q, const void* k, const void* v, const float* g, const float* beta,
                                   float* state_pool, const int32_t* state_indices, int32_t num_slots,
                                   int32_t num_seqs, int32_t num_qk_heads, int32_t num_v_heads, int32_t d_k,
                                   int32_t d_v, float scale, gdn_dtype_t dtype, void* out, void* stream) {
    if (num_slots < 0) return GDN_ERR_INVALID_ARG;
    if (num_seqs > 0 && state_indices == nullptr) return GDN_ERR_INVALID_ARG;
    if (num_slots > 0 && state_pool == nullptr) return GDN_ERR_INVALID_ARG;
    return decode_impl(q, k, v, g, beta, state_pool, num_seqs, num_qk_heads, num_v_heads, d_k, d_v, scale, dtype,
                       out, stream, state_indices, num_slots);
}

size_t gdn_backward_workspace_size(int64_t total_tokens, int32_t num_seqs, int32_t num_qk_heads,
                                   int32_t num_v_heads, int32_t d_k, int32_t d_v, gdn_dtype_t dtype) {
    if (total_tokens < 0 || num_seqs < 0) return 0;
    if (num_qk_heads <= 0 || num_v_heads <= 0 || num_v_heads % num_qk_heads != 0) return 0;
    if ((dtype != GDN_BF16 && dtype != GDN_FP32) || d_k != d_v || !fp32_head_size_ok(d_k)) return 0;
    return gdn::backward_workspace_bytes(total_tokens, num_seqs, num_v_heads, d_k);
}

gdn_status_t gdn_backward(const void* q, const void* k, const void* v, const float* g, const float* beta,
                          const float* initial_state, const int32_t* cu_seqlens, int32_t num_seqs,
                          int64_t total_tokens, int32_t num_qk_heads, int32_t num_v_heads, int32_t d_k, int32_t d_v,
                          float scale, gdn_dtype_t dtype, const void* d_out, const float* d_final_state, float* dq,
                          float* dk, float* dv, float* dg, float* dbeta, float* d_initial_state, void* workspace,
                          size_t workspace_bytes, void* stream) {
    if (num_qk_heads <= 0 || num_v_heads <= 0 || d_k <= 0 || d_v <= 0) return GDN_ERR_INVALID_ARG;
    if (num_v_heads % num_qk_heads != 0) return GDN_ERR_INVALID_ARG;
    if (dtype != GDN_BF16 && dtype != GDN_FP32) return GDN_ERR_INVALID_ARG;
    if (d_k != d_v || !fp32_head_size_ok(d_k)) return GDN_ERR_UNSUPPORTED;
    if (total_tokens < 0 || num_seqs < 0) return GDN_ERR_INVALID_ARG;
    if (total_tokens > INT32_MAX) return GDN_ERR_UNSUPPORTED;
    if (cu_seqlens == nullptr && num_seqs != 1) return GDN_ERR_INVALID_ARG;
    if (total_tokens > 0 && (!q || !k || !v || !g || !beta || !d_out || !dq || !dk || !dv || !dg || !dbeta))
        return GDN_ERR_INVALID_ARG;
    if (num_seqs == 0) return GDN_OK;
    const size_t need = gdn_backward_workspace_size(total_tokens, num_seqs, num_qk_heads, num_v_heads, d_k, d_v,
                                                    dtype);
    if (workspace == nullptr || workspace_bytes < need) return GDN_ERR_WORKSPACE;
    gdn::BackwardArgs a;
    a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta; a.initial_state = initial_state; a.cu_seqlens = cu_seqlens;
    a.d_out = d_out; a.d_final_state = d_final_state; a.dq = dq; a.dk = dk; a.dv = dv; a.dg = dg; a.dbeta = dbeta;
    a.d_initial_state = d_initial_state; a.workspace = workspace; a.total_tokens = total_tokens;
    a.num_seqs = num_seqs; a.num_qk_heads = num_qk_heads; a.num_v_heads = num_v_heads; a.d = d_k; a.scale = scale;
    a.bf16 = (dtype == GDN_BF16);
    return hip_status(gdn::launch_backward(a, static_cast<hipStream_t>(stream)));
}

gdn_status_t gdn_conv_prologue(const void* x, const float* weight, const void* conv_state_in,
                               const int32_t* cu_seqlens, int32_t num_seqs, int64_t total_tokens,
                               int32_t num_qk_heads, int32_t num_v_heads, int32_t d_k, int32_t d_v,
                               int32_t kernel_size, gdn_dtype_t dtype, uint32_t flags,
                               void* q, void* k, void* v, void* conv_state_out, void* stream) {
    if (num_qk_heads <= 0 || num_v_heads <= 0 || d_k <= 0 || d_v <= 0) return GDN_ERR_INVALID_ARG;
    if (dtype != GDN_BF16 && dtype != GDN_FP32) return GDN_ERR_INVALID_ARG;
    if (flags & ~(GDN_FLAG_QK_L2NORM | GDN_FLAG_CONV_SILU)) return GDN_ERR_INVALID_ARG;
    if (d_k != d_v || !fp32_head_size_ok(d_k)) return GDN_ERR_UNSUPPORTED;
    if (kernel_size < 1) return GDN_ERR_INVALID_ARG;
    if (kernel_size > 4) return GDN_ERR_UNSUPPORTED;
    if (total_tokens < 0 || num_seqs < 0) return GDN_ERR_INVALID_ARG;
    if (total_tokens > INT32_MAX) return GDN_ERR_UNSUPPORTED;
    if (num_seqs == 0) return total_tokens == 0 ? GDN_OK : GDN_ERR_INVALID_ARG;
    if (cu_seqlens == nullptr && total_tokens % num_seqs != 0) return GDN_ERR_INVALID_ARG;
    if (total_tokens > 0 && (!x || !weight || !q || !k || !v)) return GDN_ERR_INVALID_ARG;
    gdn::ConvPrologueArgs a;
    a.x = x; a.weight = weight; a.conv_state_in = conv_state_in; a.conv_state_out = conv_state_out;
    a.cu_seqlens = cu_seqlens; a.q = q; a.k = k; a.v = v; a.total_tokens = total_tokens; a.num_seqs = num_seqs;
    a.num_qk_heads = num_qk_heads; a.num_v_heads = num_v_heads; a.d = d_k; a.kernel_size = kernel_size;
    a.silu = (flags & GDN_FLAG_CONV_SILU) != 0; a.qk_norm = (flags & GDN_FLAG_QK_L2NORM) != 0;
    a.bf16 = (dtype == GDN_BF16);
    return hip_status(gdn::launch_conv_prologue(a, static_cast<hipStream_t>(stream)));
}

gdn_status_t gdn_decode_conv(const void* x, const float* weight, const void* conv_state_in, void* conv_state_out,
                             const float* g, const float* beta, float* state, int32_t num_seqs,
                             int32_t num_qk_heads, int32_t num_v_heads, int32_t d_k, int32_t d_v,
                             int32_t kernel_size, float scale, gdn_dtype_t dtype, uint32_t flags, void* out,
                             void* stream) {
    if (num_qk_heads <= 0 || num_v_heads <= 0 || d_k <= 0 || d_v <= 0 || num_seqs < 0)
        return GDN_ERR_INVALID_ARG;
    if (num_v_heads % num_qk_heads != 0) return GDN_ERR_INVALID_ARG;
    if (dtype != GDN_BF16 && dtype != GDN_FP32) return GDN_ERR_INVALID_ARG;
    if (flags & ~(GDN_FLAG_QK_L2NORM | GDN_FLAG_CONV_SILU)) return GDN_ERR_INVALID_ARG;
    if (d_k != d_v || !fp32_head_size_ok(d_k)) return GDN_ERR_UNSUPPORTED;
    if (kernel_size < 1) return GDN_ERR_INVALID_ARG;
    if (kernel_size > 4) return GDN_ERR_UNSUPPORTED;
    if (num_seqs == 0) return GDN_OK;
    if (!x || !weight || !g || !beta || !state || !out) return GDN_ERR_INVALID_ARG;
    if ((int64_t)num_seqs * num_v_heads > INT32_MAX) return GDN_ERR_UNSUPPORTED;
    // The two histories must not overlap: other workgroups still read rows of conv_state_in
    // after one has written its new rows.
    const int64_t C = (int64_t)(2 * num_qk_heads + num_v_heads) * d_k;
    const int64_t hist_bytes = (int64_t)num_seqs * (kernel_size - 1) * C * (dtype == GDN_BF16 ? 2 : 4);
    if (conv_state_in && conv_state_out && hist_bytes > 0) {
        const uintptr_t a0 = reinterpret_cast<uintptr_t>(conv_state_in), b0 = reinterpret_cast<uintptr_t>(conv_state_out);
        if (a0 < b0 + (uintptr_t)hist_bytes && b0 < a0 + (uintptr_t)hist_bytes) return GDN_ERR_INVALID_ARG;
    }
    gdn::DecodeArgs a;
    a.q = a.k = a.v = nullptr;
    a.g = g; a.beta = beta; a.state = state; a.out = out;
    a.state_indices = nullptr; a.num_slots = 0;
    a.num_seqs = num_seqs; a.num_qk_heads = num_qk_heads; a.num_v_heads = num_v_heads; a.d = d_k;
    a.scale = scale; a.bf16 = (dtype == GDN_BF16);
    a.qk_norm = (flags & GDN_FLAG_QK_L2NORM) != 0;
    a.conv_x = x; a.conv_w = weight; a.conv_in = conv_state_in; a.conv_out = conv_state_out;
    a.conv_K = kernel_size; a.conv_silu = (flags & GDN_FLAG_CONV_SILU) != 0;
    return hip_status(gdn::launch_decode(a, static_cast<hipStream_t>(stream)));
}

const char* gdn_status_string(gdn_status_t s) {
    switch (s) {
        case GDN_OK: return "GDN_OK";
        case GDN_ERR_INVALID_ARG: return "GDN_ERR_INVALID_ARG: invalid argument";
        case GDN_ERR_UNSUPPORTED: return "GDN_ERR_UNSUPPORTED: dtype or head size not supported";
        case GDN_ERR_WORKSPACE: return "GDN_ERR_WORKSPACE: workspace missing or too small";
        case GDN_ERR_HIP: return "GDN_ERR_HIP: HIP kernel launch failed";
        case GDN_ERR_SCRATCH_LIMIT:
            return "GDN_ERR_SCRATCH_LIMIT: the call needs more workspace than gdn_prefill_noalloc's static array";
        default: return "GDN: unknown status";
    }
}

const char* gdn_build_info(void) { return "libgdn 0.1 gfx950 (MI355X)"; }

}  // extern "C"
