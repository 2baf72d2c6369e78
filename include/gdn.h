/*
 * gdn.h - C ABI of libgdn, a Gated DeltaNet token mixer for AMD Instinct
 * MI355X (gfx950).
 *
 * The layer (page "Qwen3-Next-80B-A3B-Instruct" model card, section "Model
 * Overview": Gated DeltaNet, 32 V heads and 16 QK heads, head dimension 128;
 * page "Qwen3-Next and vLLM", section "Hybrid Attention": Gated DeltaNet is the
 * linear-attention half of the hybrid layout) keeps, per sequence and V head,
 * a d_v x d_k fp32 state S. For every token, in order:
 *
 *     alpha = exp(g)
 *     S     = alpha * S                              decay
 *     S     = S + beta * (v - S k) k^T               delta-rule write along the unit key k
 *     out   = scale * S q                            read-out after the write
 *
 * V head h reads QK head h / (num_v_heads / num_qk_heads), so consecutive V
 * heads share a QK head (the pages give only the head counts; this grouping is
 * the library's reading).
 *
 * Conventions for every entry point
 *   - All tensor pointers are DEVICE pointers to contiguous row-major arrays
 *     owned by the caller. The library never allocates, frees or keeps them.
 *   - `stream` is a hipStream_t (NULL = the null stream). Work is enqueued
 *     asynchronously on it; no entry point synchronises with the host, so the
 *     calls can be captured in a HIP graph. Results are ready when the stream
 *     has reached the call.
 *   - q and k must already be L2-normalised per token and head; g <= 0 and
 *     finite; beta in [0, 1]. These preconditions are not checked.
 *   - State element S[i][j]: i is the value index (0..d_v-1), j the key index.
 *   - Argument errors are detected on the host before anything is enqueued
 *     and return a non-zero status; nothing is launched then. No C++
 *     exception crosses this interface.
 *
 * Supported shapes: GDN_BF16 requires d_k = d_v = 128; GDN_FP32 requires
 * d_k = d_v in {16, 32, 64, 128}. num_v_heads must be a multiple of
 * num_qk_heads.
 */
#ifndef GDN_H_
#define GDN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    GDN_OK = 0,
    GDN_ERR_INVALID_ARG = 1,   /* null required pointer, bad count or size */
    GDN_ERR_UNSUPPORTED = 2,   /* valid but not implemented (dtype / head size) */
    GDN_ERR_WORKSPACE = 3,     /* workspace missing or smaller than required */
    GDN_ERR_HIP = 4,           /* a HIP launch failed (the status string has no detail) */
    GDN_ERR_SCRATCH_LIMIT = 5  /* gdn_prefill_noalloc: the call needs more workspace than its static array */
} gdn_status_t;

typedef enum {
    GDN_BF16 = 0,   /* q, k, v and out are bfloat16 */
    GDN_FP32 = 1    /* q, k, v and out are float */
} gdn_dtype_t;
/* g, beta and all states are float in both modes. */

/*
 * Bytes of device workspace gdn_prefill needs for these sizes (may be 0).
 * Returns 0 as well for arguments gdn_prefill would reject.
 */
size_t gdn_prefill_workspace_size(int64_t total_tokens, int32_t num_seqs,
                                  int32_t num_qk_heads, int32_t num_v_heads,
                                  int32_t d_k, int32_t d_v, gdn_dtype_t dtype);

/*
 * Planning query: chunks (of 64 tokens) per segment in the bf16 prefill's
 * segment-parallel schedule for these sizes, as gdn_prefill will use them on
 * the current device. Every sequence is split into segments of this many
 * chunks (the last one shorter); the first launch produces the outputs of
 * each sequence's first segment and the maps of the others, the last launch
 * the outputs of segments 1 onward. For accounting and tests; the result
 * does not need to be passed to gdn_prefill. Returns 0 for fp32 (one chain
 * per sequence and head, no segments) and for arguments gdn_prefill would
 * reject.
 */
int32_t gdn_prefill_segment_chunks(int64_t total_tokens, int32_t num_seqs,
                                   int32_t num_qk_heads, int32_t num_v_heads,
                                   int32_t d_k, int32_t d_v, gdn_dtype_t dtype);

/*
 * Chunked prefill over packed variable-length sequences (chunk size 64: the
 * intra-chunk decay masks, the UT/WY transform of the beta-weighted
 * (I - beta k k^T) factors by a triangular solve, and the inter-chunk state
 * propagation the layer's description names).
 *
 *   q, k           [total_tokens, num_qk_heads, d_k]   dtype
 *   v              [total_tokens, num_v_heads, d_v]    dtype
 *   g, beta        [total_tokens, num_v_heads]         float (g = log alpha)
 *   initial_state  [num_seqs, num_v_heads, d_v, d_k]   float, or NULL for zeros
 *   cu_seqlens     [num_seqs + 1] int32 token offsets, device memory, starting
 *                  at 0, non-decreasing, ending at total_tokens; or NULL for one
 *                  sequence of total_tokens tokens (num_seqs must be 1).
 *                  Sequences may be empty (their final state is their initial
 *                  state). Offsets are read on the device and are a
 *                  precondition, not checked.
 *   out            [total_tokens, num_v_heads, d_v]    dtype, written
 *   final_state    [num_seqs, num_v_heads, d_v, d_k]   float, written; or NULL.
 *                  May be the same pointer as initial_state (each state slice
 *                  is read before it is overwritten); any other overlap with
 *                  an input is undefined.
 *   workspace      device buffer of at least gdn_prefill_workspace_size(...)
 *                  bytes (NULL allowed when that size is 0). Its contents
 *                  need no initialisation; concurrent calls need separate
 *                  workspaces.
 * total_tokens = 0 is allowed (only the states are copied).
 */
gdn_status_t gdn_prefill(const void* q, const void* k, const void* v,
                         const float* g, const float* beta,
                         const float* initial_state,
                         const int32_t* cu_seqlens, int32_t num_seqs,
                         int64_t total_tokens, int32_t num_qk_heads, int32_t num_v_heads,
                         int32_t d_k, int32_t d_v, float scale, gdn_dtype_t dtype,
                         void* out, float* final_state,
                         void* workspace, size_t workspace_bytes, void* stream);

/*
 * One decode step for num_seqs independent sequences, one token each; the
 * state is read and updated in place (the per-sequence recurrent state a
 * serving engine's hybrid cache keeps for a linear-attention layer).
 *
 *   q, k     [num_seqs, num_qk_heads, d_k]   dtype
 *   v        [num_seqs, num_v_heads, d_v]    dtype
 *   g, beta  [num_seqs, num_v_heads]         float
 *   state    [num_seqs, num_v_heads, d_v, d_k] float, updated in place
 *   out      [num_seqs, num_v_heads, d_v]    dtype, written
 * num_seqs = 0 is allowed (nothing is launched).
 */
gdn_status_t gdn_decode_step(const void* q, const void* k, const void* v,
                             const float* g, const float* beta, float* state,
                             int32_t num_seqs, int32_t num_qk_heads, int32_t num_v_heads,
                             int32_t d_k, int32_t d_v, float scale, gdn_dtype_t dtype,
                             void* out, void* stream);

/*
 * State-pool variants (page "Qwen3-Next and vLLM: Advancing Efficient
 * Long-Context AI with Hybrid Architecture": section "Hybrid Attention: The
 * Best of Both Worlds" names the hybrid cache manager that keeps each
 * request's linear-attention state, section "Performance Optimized for Real
 * Applications" the full graph mode of decode). The states live in a pool
 * indexed by slot instead of one row per sequence of the batch:
 *
 *   state_pool     [num_slots, num_v_heads, d_v, d_k] float, device
 *   state_indices  [num_seqs] int32, device: sequence n reads and writes pool
 *                  row state_indices[n]. An index outside [0, num_slots) marks
 *                  a padding entry: no pool row is read or written for it (the
 *                  kernels check the range; it is not an error). Non-padding
 *                  indices must be distinct; sharing a row is undefined.
 * Rows not named by an index are never touched. Everything else is as in
 * gdn_decode_step / gdn_prefill, including the argument checks and the
 * statuses; num_slots < 0 or a NULL state_indices (with num_seqs > 0), or a
 * NULL state_pool with num_slots > 0, is GDN_ERR_INVALID_ARG.
 */

/*
 * Decode step on a state pool. A padding entry's outputs are written as zeros.
 * The order of the rows in the pool does not change any result bit; a batch of
 * at most min(d * d / 16, 512) sequences (512 at d = 128) is worked through in
 * pool-row order, which streams the rows fastest.
 */
gdn_status_t gdn_decode_step_slots(const void* q, const void* k, const void* v,
                                   const float* g, const float* beta,
                                   float* state_pool, const int32_t* state_indices, int32_t num_slots,
                                   int32_t num_seqs, int32_t num_qk_heads, int32_t num_v_heads,
                                   int32_t d_k, int32_t d_v, float scale, gdn_dtype_t dtype,
                                   void* out, void* stream);

/*
 * Prefill on a state pool: sequence n starts from pool row state_indices[n]
 * when has_initial_state is NULL or has_initial_state[n] != 0 (device int32
 * [num_seqs]), from zeros otherwise, and its final state is written back to
 * the same row. A padding entry starts from zeros, its outputs are computed,
 * and no row is written. Workspace as for gdn_prefill with the same sizes.
 */
gdn_status_t gdn_prefill_slots(const void* q, const void* k, const void* v,
                               const float* g, const float* beta,
                               float* state_pool, const int32_t* state_indices,
                               const int32_t* has_initial_state, int32_t num_slots,
                               const int32_t* cu_seqlens, int32_t num_seqs,
                               int64_t total_tokens, int32_t num_qk_heads, int32_t num_v_heads,
                               int32_t d_k, int32_t d_v, float scale, gdn_dtype_t dtype,
                               void* out, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Multi-token decode step: num_tokens consecutive tokens per sequence from its
 * state in one call, as when a model's multi-token-prediction drafts are
 * verified (page "Qwen3-Next and vLLM: Advancing Efficient Long-Context AI with
 * Hybrid Architecture", section "Multi-Token Prediction for Acceleration").
 * Same recurrence as gdn_decode_step applied num_tokens times; the state is
 * read once and written once.
 *
 *   q, k          [num_seqs * num_tokens, num_qk_heads, d_k]   dtype; token t of
 *                 sequence n is row n * num_tokens + t
 *   v             [num_seqs * num_tokens, num_v_heads, d_v]    dtype
 *   g, beta       [num_seqs * num_tokens, num_v_heads]         float
 *   state         [num_seqs, num_v_heads, d_v, d_k] float, updated in place to
 *                 the state after the last token; with state_indices != NULL a
 *                 state pool [num_slots, ...] as for gdn_decode_step_slots
 *                 (padding entries: zero outputs, no state access)
 *   out           [num_seqs * num_tokens, num_v_heads, d_v]    dtype, written
 *   token_states  [num_seqs * num_tokens, num_v_heads, d_v, d_k] float: the state
 *                 after each token (so that a caller can resume from the last
 *                 accepted draft token), or NULL
 * 1 <= num_tokens <= 64 (GDN_ERR_INVALID_ARG below 1, GDN_ERR_UNSUPPORTED above
 * 64: use gdn_prefill). Other checks and statuses as for gdn_decode_step.
 */
gdn_status_t gdn_decode_multi(const void* q, const void* k, const void* v,
                              const float* g, const float* beta,
                              float* state, const int32_t* state_indices, int32_t num_slots,
                              int32_t num_seqs, int32_t num_tokens,
                              int32_t num_qk_heads, int32_t num_v_heads,
                              int32_t d_k, int32_t d_v, float scale, gdn_dtype_t dtype,
                              void* out, float* token_states, void* stream);

/*
 * General forms with option flags. Every entry point above is one of these
 * with flags = 0.
 *
 * Flags (bitwise OR):
 *   GDN_FLAG_QK_L2NORM  the kernels L2-normalise each token's q and k per QK
 *                       head before using them, x / sqrt(sum(x^2) + 1e-6) in
 *                       fp32 (bf16 inputs: the staged keys and queries are the
 *                       normalised values rounded to bf16). It lifts the
 *                       unit-length precondition on q and k: the input
 *                       prologue that page "Qwen3-Next-80B-A3B-Instruct",
 *                       section "Quickstart", leaves to the flash-linear-
 *                       attention kernels. (The epsilon is this library's
 *                       choice; the pages give none.)
 * Unknown flag bits are GDN_ERR_INVALID_ARG.
 */
#define GDN_FLAG_QK_L2NORM 1u

/*
 * gdn_prefill_ex: with state_indices == NULL, initial_state and final_state
 * are [num_seqs, ...] arrays as in gdn_prefill (has_initial_state and
 * num_slots are ignored); otherwise both are pools of num_slots rows
 * addressed as in gdn_prefill_slots (they may be the same pool), where a NULL
 * initial_state means zeros and a NULL final_state writes nothing.
 */
gdn_status_t gdn_prefill_ex(const void* q, const void* k, const void* v,
                            const float* g, const float* beta,
                            const float* initial_state, float* final_state,
                            const int32_t* state_indices, const int32_t* has_initial_state,
                            int32_t num_slots,
                            const int32_t* cu_seqlens, int32_t num_seqs,
                            int64_t total_tokens, int32_t num_qk_heads, int32_t num_v_heads,
                            int32_t d_k, int32_t d_v, float scale, gdn_dtype_t dtype, uint32_t flags,
                            void* out, void* workspace, size_t workspace_bytes, void* stream);

/*
 * gdn_decode_ex: gdn_decode_multi with flags (num_tokens = 1 and
 * token_states = NULL is gdn_decode_step, or gdn_decode_step_slots with
 * state_indices).
 */
gdn_status_t gdn_decode_ex(const void* q, const void* k, const void* v,
                           const float* g, const float* beta,
                           float* state, const int32_t* state_indices, int32_t num_slots,
                           int32_t num_seqs, int32_t num_tokens,
                           int32_t num_qk_heads, int32_t num_v_heads,
                           int32_t d_k, int32_t d_v, float scale, gdn_dtype_t dtype, uint32_t flags,
                           void* out, float* token_states, void* stream);

/*
 * Backward of the prefill (for training; page "Qwen3-Next-80B-A3B-Instruct",
 * section "Highlights", on the hybrid layout's training efficiency): the
 * gradients of the recurrence with respect to q, k, v, g, beta and the initial
 * states, given the gradient of the outputs and, optionally, of the final
 * states. Inputs and shapes as for gdn_prefill (flags 0: q and k unit-length);
 *   d_out           [total_tokens, num_v_heads, d_v]    dtype of q
 *   d_final_state   [num_seqs, num_v_heads, d_v, d_k]   float, or NULL (zeros)
 * Outputs, all float, written:
 *   dq, dk          [total_tokens, num_qk_heads, d_k]   (summed over the V heads of a QK head)
 *   dv              [total_tokens, num_v_heads, d_v]
 *   dg, dbeta       [total_tokens, num_v_heads]         (dg: with respect to g = log alpha)
 *   d_initial_state [num_seqs, num_v_heads, d_v, d_k], or NULL
 * The computation is in fp32 by chunks of 16 tokens, each chunk's token rule
 * unrolled into closed form (triangular solve and matrix products on fp32
 * MFMA): a pass builds every chunk's factors, two scans (forward and reverse,
 * 16 state rows per workgroup) store the state before and the state gradient
 * after every chunk in the workspace, every chunk's gradients then follow in
 * parallel from those two. dq and dk of a QK head are formed from its V heads'
 * shares deterministically: one V head stores its share, two add theirs into
 * the output zeroed beforehand (0 + a + b and 0 + b + a are the same float),
 * three or more are summed by a last pass in a fixed order.
 * workspace: gdn_backward_workspace_size(...) bytes, for d = d_k = d_v:
 * 8 d^2 Hv (T / 16 + N) + 8 d Hv T + 3328 Hv (T / 16 + N).
 */
size_t gdn_backward_workspace_size(int64_t total_tokens, int32_t num_seqs,
                                   int32_t num_qk_heads, int32_t num_v_heads,
                                   int32_t d_k, int32_t d_v, gdn_dtype_t dtype);
gdn_status_t gdn_backward(const void* q, const void* k, const void* v,
                          const float* g, const float* beta,
                          const float* initial_state,
                          const int32_t* cu_seqlens, int32_t num_seqs,
                          int64_t total_tokens, int32_t num_qk_heads, int32_t num_v_heads,
                          int32_t d_k, int32_t d_v, float scale, gdn_dtype_t dtype,
                          const void* d_out, const float* d_final_state,
                          float* dq, float* dk, float* dv, float* dg, float* dbeta,
                          float* d_initial_state,
                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * gdn_prefill for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Arguments, results and errors are gdn_prefill's, without the workspace: the
 * bf16 path's segment workspace is a static device array of
 * GDN_PREFILL_NOALLOC_SCRATCH_BYTES held by every GPU the library is loaded on
 * until the process ends. A call whose gdn_prefill_workspace_size exceeds it
 * returns GDN_ERR_SCRATCH_LIMIT before anything is enqueued (with 32 V heads it
 * covers one sequence of any length, and up to about 10 long sequences per
 * call). The entry point allocates nothing. All calls on one GPU share its
 * array: calls that may overlap on one GPU (other streams, other threads
 * without ordering) race and must be serialised by the caller.
 */
#define GDN_PREFILL_NOALLOC_SCRATCH_BYTES (192ull << 20)
gdn_status_t gdn_prefill_noalloc(const void* q, const void* k, const void* v,
                                 const float* g, const float* beta,
                                 const float* initial_state,
                                 const int32_t* cu_seqlens, int32_t num_seqs,
                                 int64_t total_tokens, int32_t num_qk_heads, int32_t num_v_heads,
                                 int32_t d_k, int32_t d_v, float scale, gdn_dtype_t dtype,
                                 void* out, float* final_state, void* stream);

/*
 * Input prologue: the short causal convolution in front of the mixer. The
 * model card (page "Qwen3-Next-80B-A3B-Instruct", section "Quickstart")
 * points to the causal-conv1d kernels beside flash-linear-attention without
 * saying what they convolve; the library's reading is a depthwise causal 1-D
 * convolution over the mixer's input channels, with each channel's own K taps:
 *
 *     y_t[c] = sum_{i=0}^{K-1} weight[c][i] * x_{t-K+1+i}[c]
 *
 * (tap K-1 multiplies the current token), optionally followed by SiLU
 * y * sigmoid(y), then split into the q, k and v arrays the mixer reads and,
 * with GDN_FLAG_QK_L2NORM, the L2 normalisation of each q and k head, so the
 * outputs feed gdn_prefill / gdn_decode_step directly.
 *   x               [total_tokens, C] dtype, C = 2 Hqk d + Hv d: channel c is
 *                   q (c < Hqk d, head c / d), then k, then v
 *   weight          [C, K] float, 1 <= K <= 4
 *   conv_state_in   [num_seqs, K - 1, C] dtype: each sequence's history, the
 *                   K - 1 inputs before its first token, oldest first; NULL
 *                   means zeros (a sequence's start)
 *   cu_seqlens      [num_seqs + 1] device int32 offsets, or NULL: num_seqs
 *                   sequences of total_tokens / num_seqs tokens each (one
 *                   token per sequence is a decode step)
 *   q, k, v         outputs [T, Hqk, d], [T, Hqk, d], [T, Hv, d], dtype
 *   conv_state_out  [num_seqs, K - 1, C] dtype, or NULL: each sequence's last
 *                   K - 1 inputs (reaching into conv_state_in when it is
 *                   shorter than K - 1). May alias conv_state_in: outputs are
 *                   computed first, the new history written by a second launch.
 * Flags: GDN_FLAG_CONV_SILU, GDN_FLAG_QK_L2NORM (1e-6 inside the square root).
 * d = d_k = d_v in {16, 32, 64, 128}. Errors: GDN_ERR_INVALID_ARG for null
 * pointers, K outside [1, 4] with K > 4 reported as GDN_ERR_UNSUPPORTED,
 * total_tokens not a multiple of num_seqs without cu_seqlens, or unknown flags.
 */
#define GDN_FLAG_CONV_SILU 2u
gdn_status_t gdn_conv_prologue(const void* x, const float* weight, const void* conv_state_in,
                               const int32_t* cu_seqlens, int32_t num_seqs, int64_t total_tokens,
                               int32_t num_qk_heads, int32_t num_v_heads, int32_t d_k, int32_t d_v,
                               int32_t kernel_size, gdn_dtype_t dtype, uint32_t flags,
                               void* q, void* k, void* v, void* conv_state_out, void* stream);

/*
 * Decode step with the input prologue fused in: gdn_conv_prologue on one token
 * per sequence followed by gdn_decode_step, in one launch (the reading of the
 * prologue is gdn_conv_prologue's, page "Qwen3-Next-80B-A3B-Instruct", section
 * "Quickstart"). The workgroup of (sequence n, V head h) convolves only the
 * channels it reads (its QK head's q and k, its V head's v), applies SiLU with
 * GDN_FLAG_CONV_SILU and the q/k L2 normalisation with GDN_FLAG_QK_L2NORM, and
 * runs the decode step on them; q, k and v never go through HBM and stay fp32
 * (the unfused pair rounds them to dtype in between).
 *   x               [num_seqs, C] dtype, C = 2 Hqk d + Hv d, channel order as
 *                   for gdn_conv_prologue (one token per sequence)
 *   weight          [C, K] float, 1 <= K <= 4
 *   conv_state_in   [num_seqs, K - 1, C] dtype, or NULL (zeros)
 *   conv_state_out  [num_seqs, K - 1, C] dtype, or NULL: the new history (the
 *                   last K - 1 inputs, the input's bits). It must not overlap
 *                   conv_state_in, since the workgroups of the V heads that
 *                   share a QK head read the same q/k history rows; callers
 *                   alternate two arrays between steps.
 *   g, beta, state, out, scale   as for gdn_decode_step (state updated in place)
 * d = d_k = d_v in {16, 32, 64, 128}. Errors:
 * GDN_ERR_INVALID_ARG for null pointers, Hv not a multiple of Hqk, K < 1,
 * unknown flags or overlapping histories; GDN_ERR_UNSUPPORTED for K > 4 or
 * another head size. num_seqs = 0 enqueues nothing.
 */
gdn_status_t gdn_decode_conv(const void* x, const float* weight, const void* conv_state_in,
                             void* conv_state_out, const float* g, const float* beta, float* state,
                             int32_t num_seqs, int32_t num_qk_heads, int32_t num_v_heads,
                             int32_t d_k, int32_t d_v, int32_t kernel_size, float scale,
                             gdn_dtype_t dtype, uint32_t flags, void* out, void* stream);

/*
 * Instrumentation (for benchmarks and profiling; process-global, not
 * thread-safe, not for graph capture). After gdn_profile_start(), every kernel
 * the library launches is bracketed by a pair of HIP events recorded on the
 * stream it is launched on. gdn_profile_stop() turns this off, waits for the
 * recorded events and aggregates them per kernel: names receives up to
 * max_kernels NUL-terminated names of at most 63 characters in slots of 64
 * bytes, counts the launches and total_ms the summed durations. Returns the
 * number of distinct kernels, or -1 if a HIP event call failed.
 */
gdn_status_t gdn_profile_start(void);
int32_t gdn_profile_stop(int32_t max_kernels, char* names, int32_t* counts, double* total_ms);

/* Static, NUL-terminated description of a status code. */
const char* gdn_status_string(gdn_status_t status);

/* Static, NUL-terminated build description (library version and GPU target). */
const char* gdn_build_info(void);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H_ */
