// Internal launch interface between the C ABI (gdn_api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gdn {

constexpr int kChunk = 64;   // prefill chunk length (tokens)
// In-kernel q/k normalisation: x / sqrt(sum(x^2) + kQkNormEps) per token and head.
constexpr float kQkNormEps = 1e-6f;

struct DecodeArgs {
    const void* q;
    const void* k;
    const void* v;
    const float* g;
    const float* beta;
    float* state;
    void* out;
    const int32_t* state_indices;   // null: sequence n uses state row n; else row state_indices[n]
    int32_t num_slots;              // rows in the state pool (with state_indices)
    int32_t num_tokens = 1;         // tokens per sequence (multi-token step)
    float* token_states = nullptr;  // multi-token step: state after every token, or null
    bool qk_norm = false;           // L2-normalise q and k in the kernel
    int32_t num_seqs, num_qk_heads, num_v_heads, d;
    float scale;
    bool bf16;
    // Fused input prologue (conv_K > 0): q, k, v come from the causal convolution of conv_x
    // (one token per sequence) instead of the q, k, v arrays.
    const void* conv_x = nullptr;   // [num_seqs, C]
    const float* conv_w = nullptr;  // [C, conv_K]
    const void* conv_in = nullptr;  // [num_seqs, conv_K - 1, C] or null (zeros)
    void* conv_out = nullptr;       // [num_seqs, conv_K - 1, C] or null; never overlaps conv_in
    int32_t conv_K = 0;
    bool conv_silu = false;
};

struct PrefillArgs {
    const void* q;
    const void* k;
    const void* v;
    const float* g;
    const float* beta;
    const float* initial_state;   // may be null (zeros)
    const int32_t* cu_seqlens;    // may be null (one sequence of total_tokens)
    float* final_state;           // may be null
    const int32_t* state_indices; // null: sequence n uses state row n; else row state_indices[n]
    const int32_t* has_initial;   // null: every sequence reads its initial state row (if any)
    int32_t num_slots;            // rows in the state pool (with state_indices)
    bool qk_norm = false;         // L2-normalise q and k in the kernel
    void* out;
    void* workspace;
    size_t workspace_bytes;
    int64_t total_tokens;
    int32_t num_seqs, num_qk_heads, num_v_heads, d;
    float scale;
    bool bf16;
};

// Row of the state array that sequence n reads and writes: n itself, or its
// slot in a state pool. A slot outside [0, num_slots) marks a padding entry
// (-1): no state is read or written for it.
__device__ __forceinline__ int64_t state_row(const int32_t* state_indices, int32_t num_slots, int n) {
    if (state_indices == nullptr) return n;
    const int32_t s = state_indices[n];
    return (s >= 0 && s < num_slots) ? s : -1;
}

struct BackwardArgs {
    const void* q;
    const void* k;
    const void* v;
    const float* g;
    const float* beta;
    const float* initial_state;   // may be null (zeros)
    const int32_t* cu_seqlens;    // may be null (one sequence)
    const void* d_out;            // [T, Hv, d], the dtype of q
    const float* d_final_state;   // may be null (zeros)
    float* dq;                    // [T, Hqk, d]
    float* dk;                    // [T, Hqk, d]
    float* dv;                    // [T, Hv, d]
    float* dg;                    // [T, Hv]
    float* dbeta;                 // [T, Hv]
    float* d_initial_state;       // may be null
    void* workspace;
    int64_t total_tokens;
    int32_t num_seqs, num_qk_heads, num_v_heads, d;
    float scale;
    bool bf16;
};

struct ConvPrologueArgs {
    const void* x;                // [T, C] inputs, C = 2 Hqk d + Hv d (q, k, v channels)
    const float* weight;          // [C, K]
    const void* conv_state_in;    // [N, K - 1, C] history or null (zeros)
    void* conv_state_out;         // [N, K - 1, C] or null; may alias conv_state_in
    const int32_t* cu_seqlens;    // null: num_seqs sequences of total_tokens / num_seqs tokens
    void* q;
    void* k;
    void* v;
    int64_t total_tokens;
    int32_t num_seqs, num_qk_heads, num_v_heads, d, kernel_size;
    bool silu, qk_norm, bf16;
};

namespace prof {
// Event pair around one kernel launch when instrumentation is on (no-op otherwise).
void begin(hipStream_t s, const char* name);
void end(hipStream_t s);
}  // namespace prof

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream);
hipError_t launch_conv_prologue(const ConvPrologueArgs& a, hipStream_t stream);
hipError_t launch_backward(const BackwardArgs& a, hipStream_t stream);
size_t backward_workspace_bytes(int64_t total_tokens, int32_t num_seqs, int32_t num_v_heads, int32_t d);
hipError_t launch_decode_multi(const DecodeArgs& a, hipStream_t stream);
hipError_t launch_prefill_f32(const PrefillArgs& a, hipStream_t stream);
hipError_t launch_prefill_bf16(const PrefillArgs& a, hipStream_t stream);
int cp_segment_chunks(int64_t total_tokens, int32_t num_seqs, int32_t num_v_heads);
size_t prefill_bf16_workspace_bytes(int64_t total_tokens, int32_t num_seqs, int32_t num_qk_heads,
                                    int32_t num_v_heads);

}  // namespace gdn
