// Chunked Gated DeltaNet prefill, fp32 inputs and fp32 arithmetic (plain FMA).
//
// This is the library's fp32-input mode: the same chunk algorithm as the bf16
// MFMA kernel, without any reduced-precision operand, for head sizes 16..128.
//
// Chunk algebra (chunk of n <= 64 tokens, state S0 = d_v x d_k on entry;
// gamma = in-chunk cumulative sum of g, Gamma = exp(gamma)):
//   A[r][c] = beta_r exp(gamma_r - gamma_c) (k_r . k_c)   for c < r
//   Tm      = (I + A)^-1                                   (UT transform, triangular solve)
//   U       = Tm diag(beta) (V - diag(Gamma) K S0^T)       the chunk's delta writes
//   O       = scale (diag(Gamma) Q S0^T + (Dm * Q K^T) U), Dm[r][c] = exp(gamma_r - gamma_c), c <= r
//   S_end   = Gamma_last S0 + U^T diag(exp(gamma_last - gamma)) K
// U follows from unrolling the per-token rule inside the chunk: the write u_r
// sees the state decayed to token r plus the earlier writes of the chunk, which
// gives the unit lower-triangular system (I + A) U = diag(beta)(V - diag(Gamma) K S0^T).
//
// Work split: one workgroup per (sequence, V head), 2*d threads. Thread t owns
// state row i = t / 2 and key columns [(t % 2) * d/2, (t % 2 + 1) * d/2) in
// registers; the two halves of a row sit in adjacent lanes and combine their
// partial dot products with one DPP exchange. Chunk tiles (K, Q, V and the
// 64 x 64 matrices) live in LDS; padded rows of a partial last chunk are zero
// with g = beta = 0, which leaves the state and the real rows unchanged.
#include "gdn_common.h"
#include "gdn_internal.h"

namespace gdn {

template <int D>
struct F32Smem {
    float K[kChunk][D + 1];
    float Q[kChunk][D + 1];
    float V[kChunk][D + 1];   // V, then beta * R, then U
    float A[kChunk][kChunk + 1];
    float T[kChunk][kChunk + 1];
    float P[kChunk][kChunk + 1];
    float graw[kChunk], gam[kChunk], Gam[kChunk], dec[kChunk], bet[kChunk];
};

template <int D>
__global__ __launch_bounds__(2 * D) void prefill_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    const float* __restrict__ g, const float* __restrict__ beta,
    const float* initial_state, const int32_t* __restrict__ cu_seqlens, float* final_state,
    float* __restrict__ out, int64_t total_tokens, int32_t num_qk_heads, int32_t num_v_heads,
    float scale, const int32_t* __restrict__ state_indices, const int32_t* __restrict__ has_initial,
    int32_t num_slots, int32_t qk_norm) {
    constexpr int NT = 2 * D;
    constexpr int H = D / 2;   // key columns per thread
    __shared__ F32Smem<D> sm;

    const int tid = threadIdx.x;
    const int i = tid >> 1;          // state row (value index)
    const int hf = tid & 1;          // key-column half
    const int jb = hf * H;
    const int n = blockIdx.x / num_v_heads;
    const int h = blockIdx.x % num_v_heads;
    const int hq = h / (num_v_heads / num_qk_heads);
    const int64_t bos = cu_seqlens ? (int64_t)cu_seqlens[n] : 0;
    const int64_t eos = cu_seqlens ? (int64_t)cu_seqlens[n + 1] : total_tokens;

    // State row of this sequence (a pool slot, or -1 for a padding entry: zero
    // entry state, nothing written back).
    const int64_t srow = state_row(state_indices, num_slots, n);
    const bool read_init = initial_state && srow >= 0 && (has_initial == nullptr || has_initial[n] != 0);
    float s[H];
    const int64_t sbase = ((srow * num_v_heads + h) * D + i) * D + jb;
#pragma unroll
    for (int jj = 0; jj < H; ++jj) s[jj] = read_init ? initial_state[sbase + jj] : 0.f;

    for (int64_t c0 = bos; c0 < eos; c0 += kChunk) {
        const int nc = (int)((eos - c0) < kChunk ? (eos - c0) : kChunk);
        // Phase 0: chunk tiles into LDS (zero rows past the end).
        for (int e = tid; e < kChunk * D; e += NT) {
            const int r = e / D, j = e % D;
            const bool in = r < nc;
            const int64_t t = c0 + r;
            sm.K[r][j] = in ? k[(t * num_qk_heads + hq) * D + j] : 0.f;
            sm.Q[r][j] = in ? q[(t * num_qk_heads + hq) * D + j] : 0.f;
            sm.V[r][j] = in ? v[(t * num_v_heads + h) * D + j] : 0.f;
        }
        for (int r = tid; r < kChunk; r += NT) {
            const bool in = r < nc;
            sm.graw[r] = in ? g[(c0 + r) * num_v_heads + h] : 0.f;
            sm.bet[r] = in ? beta[(c0 + r) * num_v_heads + h] : 0.f;
        }
        __syncthreads();
        if (qk_norm) {
            // In-kernel L2 normalisation of every k and q row (rows past the end stay zero).
            for (int r = tid; r < 2 * kChunk; r += NT) {
                float* row = (r < kChunk) ? sm.K[r] : sm.Q[r - kChunk];
                float ss = 0.f;
                for (int j = 0; j < D; ++j) ss = fmaf(row[j], row[j], ss);
                const float f = rsqrtf(ss + kQkNormEps);
                for (int j = 0; j < D; ++j) row[j] *= f;
            }
            __syncthreads();
        }
        // Phase 1: in-chunk cumulative decay.
        for (int r = tid; r < kChunk; r += NT) {
            float acc = 0.f;
            for (int c = 0; c <= r; ++c) acc += sm.graw[c];
            sm.gam[r] = acc;
        }
        __syncthreads();
        for (int r = tid; r < kChunk; r += NT) {
            sm.Gam[r] = exp_nonpos(sm.gam[r]);
            sm.dec[r] = exp_nonpos(sm.gam[kChunk - 1] - sm.gam[r]);
        }
        // Phase 2: A (strictly lower), P = Dm * Q K^T (lower incl. diagonal), Tm := I.
        for (int e = tid; e < kChunk * kChunk; e += NT) {
            const int r = e / kChunk, c = e % kChunk;
            float a = 0.f, p = 0.f;
            if (c <= r) {
                float dk = 0.f, dq = 0.f;
                for (int j = 0; j < D; ++j) {
                    dk = fmaf(sm.K[r][j], sm.K[c][j], dk);
                    dq = fmaf(sm.Q[r][j], sm.K[c][j], dq);
                }
                const float decay = exp_nonpos(sm.gam[r] - sm.gam[c]);
                p = decay * dq;
                if (c < r) a = sm.bet[r] * decay * dk;
            }
            sm.A[r][c] = a;
            sm.P[r][c] = p;
            sm.T[r][c] = (r == c) ? 1.f : 0.f;
        }
        __syncthreads();
        // Phase 3: Tm = (I + A)^-1 by forward substitution, one column per lane:
        // Tm[r][c] = -sum_{c <= j < r} A[r][j] Tm[j][c]; entries above the diagonal stay 0.
        for (int c = tid; c < kChunk; c += NT) {
            for (int r = 1; r < kChunk; ++r) {
                float acc = 0.f;
                for (int j = 0; j < r; ++j) acc = fmaf(sm.A[r][j], sm.T[j][c], acc);
                if (r > c) sm.T[r][c] = -acc;
            }
        }
        __syncthreads();
        // Phase 4: V <- beta * (V - Gamma * (K S0^T)), row r owned by lane half r / 32.
        for (int r = 0; r < kChunk; ++r) {
            float z = 0.f;
#pragma unroll
            for (int jj = 0; jj < H; ++jj) z = fmaf(sm.K[r][jb + jj], s[jj], z);
            z += dpp_quad_xor1(z);
            if ((r >> 5) == hf) sm.V[r][i] = sm.bet[r] * (sm.V[r][i] - sm.Gam[r] * z);
        }
        __syncthreads();
        // Phase 5: U = Tm (beta R), rows [32 hf, 32 hf + 32) of column i.
        float u[32];
#pragma unroll
        for (int rr = 0; rr < 32; ++rr) {
            const int r = hf * 32 + rr;
            float acc = 0.f;
            for (int c = 0; c <= r; ++c) acc = fmaf(sm.T[r][c], sm.V[c][i], acc);
            u[rr] = acc;
        }
        __syncthreads();
#pragma unroll
        for (int rr = 0; rr < 32; ++rr) sm.V[hf * 32 + rr][i] = u[rr];
        __syncthreads();
        // Phase 6: O = scale (Gamma * (Q S0^T) + P U), the two lanes of a row
        // split both sums and exchange once.
        for (int r = 0; r < nc; ++r) {
            float y = 0.f;
#pragma unroll
            for (int jj = 0; jj < H; ++jj) y = fmaf(sm.Q[r][jb + jj], s[jj], y);
            float pu = 0.f;
            const int cend = (hf * 32 + 32 <= r + 1) ? hf * 32 + 32 : r + 1;
            for (int c = hf * 32; c < cend; ++c) pu = fmaf(sm.P[r][c], sm.V[c][i], pu);
            float tot = sm.Gam[r] * y + pu;
            tot += dpp_quad_xor1(tot);
            if (hf == 0) out[((c0 + r) * num_v_heads + h) * D + i] = scale * tot;
        }
        // Phase 7: S = Gamma_last S0 + U^T diag(dec) K (this lane's row and key half).
        const float glast = sm.Gam[kChunk - 1];
#pragma unroll
        for (int jj = 0; jj < H; ++jj) s[jj] *= glast;
        for (int r = 0; r < kChunk; ++r) {
            const float ur = sm.dec[r] * sm.V[r][i];
#pragma unroll
            for (int jj = 0; jj < H; ++jj) s[jj] = fmaf(ur, sm.K[r][jb + jj], s[jj]);
        }
        __syncthreads();
    }
    if (final_state && srow >= 0) {
#pragma unroll
        for (int jj = 0; jj < H; ++jj) final_state[sbase + jj] = s[jj];
    }
}

template <int D>
static hipError_t launch_f32_t(const PrefillArgs& a, hipStream_t stream) {
    const int64_t blocks = (int64_t)a.num_seqs * a.num_v_heads;
    prof::begin(stream, "gdn_prefill_f32");
    hipLaunchKernelGGL((prefill_f32_kernel<D>), dim3((unsigned)blocks), dim3(2 * D), 0, stream,
                       (const float*)a.q, (const float*)a.k, (const float*)a.v, a.g, a.beta,
                       a.initial_state, a.cu_seqlens, a.final_state, (float*)a.out, a.total_tokens,
                       a.num_qk_heads, a.num_v_heads, a.scale, a.state_indices, a.has_initial, a.num_slots,
                       a.qk_norm ? 1 : 0);
    prof::end(stream);
    return hipGetLastError();
}

hipError_t launch_prefill_f32(const PrefillArgs& a, hipStream_t stream) {
    switch (a.d) {
        case 16: return launch_f32_t<16>(a, stream);
        case 32: return launch_f32_t<32>(a, stream);
        case 64: return launch_f32_t<64>(a, stream);
        case 128: return launch_f32_t<128>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace gdn
