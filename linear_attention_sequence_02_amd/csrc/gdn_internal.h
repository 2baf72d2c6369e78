// Internal launch interface between the C ABI (gdn_api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gdn {

constexpr int kChunk = 64;   // prefill chunk length (tokens)

struct DecodeArgs {
    const void* q;
    const void* k;
    const void* v;
    const float* g;
    const float* beta;
    float* state;
    void* out;
    int32_t num_seqs, num_qk_heads, num_v_heads, d;
    float scale;
    bool bf16;
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
    void* out;
    void* workspace;
    size_t workspace_bytes;
    int64_t total_tokens;
    int32_t num_seqs, num_qk_heads, num_v_heads, d;
    float scale;
    bool bf16;
};

namespace prof {
// Event pair around one kernel launch when instrumentation is on (no-op otherwise).
void begin(hipStream_t s, const char* name);
void end(hipStream_t s);
}  // namespace prof

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream);
hipError_t launch_prefill_f32(const PrefillArgs& a, hipStream_t stream);
hipError_t launch_prefill_bf16(const PrefillArgs& a, hipStream_t stream);
int cp_segment_chunks(int64_t total_tokens, int32_t num_seqs, int32_t num_v_heads);
size_t prefill_bf16_workspace_bytes(int64_t total_tokens, int32_t num_seqs, int32_t num_qk_heads,
                                    int32_t num_v_heads);

}  // namespace gdn
