// Gradients of the Gated DeltaNet recurrence, token by token in fp32.
//
// Forward rule per (sequence, V head), token t (alpha = exp(g), w = S k):
//     u   = beta (v - alpha w)            S_t = alpha S + u k^T          o = scale S_t q
// Reverse, with dS the gradient of S_t (it already holds every later token's
// contribution) and S the state before token t:
//     dS  += scale do q^T                 (the read-out)
//     du   = dS k,   dv = beta du,   dbeta = du . (v - alpha w)
//     dalpha = <dS, S> - beta du . w,    dg = alpha dalpha
//     dk   = dS^T u - alpha beta S^T du,  dq = scale (alpha S^T do + k (u . do))
//     dS  <- alpha dS - alpha beta du k^T (the gradient of the state before t)
// (dq and dk are per V head here and summed over the V heads that share a QK
// head by a second kernel, in a fixed order.)
//
// One workgroup per (sequence, V head); each thread holds R rows x 16 key
// columns of S and dS in registers, as in the decode step. The states before
// every token are not stored: a first pass runs the forward rule over the
// sequence and keeps the state at the start of every interval of 16 tokens;
// the reverse pass walks the intervals backwards, keeps the interval's
// checkpoint in registers and, for each token, rebuilds the state before it
// from there. Each interval's inputs (k, q, v, dO, g, beta) are staged in LDS
// once, so the recomputation reads no global memory. Row sums stay inside a
// row's lane group (DPP); the column sums of dq and dk go across lanes by
// shuffles and across waves through LDS, one barrier per token.
#include "gdn_common.h"
#include "gdn_internal.h"

#include <type_traits>

namespace gdn {

typedef float f32x4 __attribute__((ext_vector_type(4)));
constexpr int kCkpt = 16;   // tokens per checkpoint interval

template <int D>
struct BwdShape {
    static constexpr int L = D / 16;                          // lanes per state row
    static constexpr int NT = (D * L < 512) ? D * L : 512;    // threads
    static constexpr int RPP = NT / L;                        // rows per pass
    static constexpr int R = D / RPP;                         // rows per thread
    static constexpr int WL = NT < 64 ? NT : 64;              // lanes per wave in use
    static constexpr int NW = (NT + 63) / 64;                 // waves
};

// Slot of interval j of sequence n in the checkpoint array: cu[n] / 16 + n + j.
// The ranges of different sequences are disjoint and below T / 16 + N.
__device__ __forceinline__ int64_t ckpt_base(const int32_t* cu, int n) {
    return cu ? (int64_t)(cu[n] / kCkpt) + n : 0;
}

template <int D, bool BF16>
__global__ __launch_bounds__(BwdShape<D>::NT) void backward_kernel(
    const void* __restrict__ q_, const void* __restrict__ k_, const void* __restrict__ v_,
    const float* __restrict__ g, const float* __restrict__ beta, const float* __restrict__ initial_state,
    const int32_t* __restrict__ cu, int64_t total_tokens, int32_t num_qk_heads, int32_t num_v_heads, float scale,
    const void* __restrict__ dout_, const float* __restrict__ dfinal, float* __restrict__ dq_v,
    float* __restrict__ dk_v, float* __restrict__ dv, float* __restrict__ dg, float* __restrict__ dbeta,
    float* __restrict__ dinit, float* __restrict__ ckpt) {
    using Sh = BwdShape<D>;
    constexpr int L = Sh::L, NT = Sh::NT, RPP = Sh::RPP, R = Sh::R, WL = Sh::WL, NW = Sh::NW;
    static_assert(R * RPP == D, "rows must tile");
    __shared__ float red[2][NW][2][D];
    __shared__ float reds[2][NW][4];
    __shared__ float kI[kCkpt][D], qI[kCkpt][D], vI[kCkpt][D], doI[kCkpt][D];   // one interval's inputs
    __shared__ float gI[kCkpt], bI[kCkpt];

    const int tid = threadIdx.x;
    const int c = tid % L, r0 = tid / L, wv = tid / 64, ln = tid % 64;
    const int n = blockIdx.x / num_v_heads, h = blockIdx.x % num_v_heads;
    const int hq = h / (num_v_heads / num_qk_heads);
    const int64_t bos = cu ? (int64_t)cu[n] : 0, eos = cu ? (int64_t)cu[n + 1] : total_tokens;
    const int64_t sbase = ((int64_t)n * num_v_heads + h) * D * D;
    const int64_t cbase = ckpt_base(cu, n);
    auto col = [&](int i, int e) { return 4 * (c + L * i) + e; };
    auto row = [&](int m) { return r0 + m * RPP; };
    auto ld = [&](const void* p, int64_t idx) -> float {
        if constexpr (BF16) return bf16_bits_to_float(reinterpret_cast<const uint16_t*>(p)[idx]);
        else return reinterpret_cast<const float*>(p)[idx];
    };
    auto ck_ptr = [&](int64_t j) { return ckpt + ((cbase + j) * num_v_heads + h) * (int64_t)D * D; };

    // Tokens t0 .. t1 - 1 (at most 16) into kI, qI, vI, doI, gI, bI (fp32); every
    // thread has finished with the previous interval before it is overwritten.
    auto stage = [&](int64_t t0, int64_t t1, bool with_grad_inputs) {
        __syncthreads();
        const int cnt = (int)(t1 - t0);
        for (int e = tid; e < cnt * D; e += NT) {
            const int tt = e / D, jj = e % D;
            const int64_t t = t0 + tt;
            kI[tt][jj] = ld(k_, (t * num_qk_heads + hq) * D + jj);
            vI[tt][jj] = ld(v_, (t * num_v_heads + h) * D + jj);
            if (with_grad_inputs) {
                qI[tt][jj] = ld(q_, (t * num_qk_heads + hq) * D + jj);
                doI[tt][jj] = ld(dout_, (t * num_v_heads + h) * D + jj);
            }
        }
        for (int e = tid; e < cnt; e += NT) {
            gI[e] = g[(t0 + e) * num_v_heads + h];
            bI[e] = beta[(t0 + e) * num_v_heads + h];
        }
        __syncthreads();
    };
    auto lds_row = [&](const float (*X)[D], int tt, float (&x)[4][4]) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const f32x4 y = *reinterpret_cast<const f32x4*>(&X[tt][col(i, 0)]);
#pragma unroll
            for (int e = 0; e < 4; ++e) x[i][e] = y[e];
        }
    };

    float S[R][4][4];
    // One forward step on S (registers) for the staged token tt.
    auto step = [&](int tt) {
        float kk[4][4];
        lds_row(kI, tt, kk);
        const float alpha = exp_nonpos(gI[tt]), b = bI[tt];
#pragma unroll
        for (int m = 0; m < R; ++m) {
            float w = 0.f;
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int e = 0; e < 4; ++e) w = fmaf(S[m][i][e], kk[i][e], w);
            w = group_sum<L>(w);
            const float u = b * (vI[tt][row(m)] - alpha * w);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int e = 0; e < 4; ++e) S[m][i][e] = fmaf(alpha, S[m][i][e], u * kk[i][e]);
        }
    };
    auto store_S = [&](float* dst) {
#pragma unroll
        for (int m = 0; m < R; ++m)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                *reinterpret_cast<f32x4*>(dst + row(m) * D + col(i, 0)) = f32x4{S[m][i][0], S[m][i][1], S[m][i][2], S[m][i][3]};
    };
    auto load_S = [&](const float* src) {
#pragma unroll
        for (int m = 0; m < R; ++m)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const f32x4 x = src ? *reinterpret_cast<const f32x4*>(src + row(m) * D + col(i, 0)) : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int e = 0; e < 4; ++e) S[m][i][e] = x[e];
            }
    };

    // Forward pass: the state at the start of every interval of 16 tokens.
    load_S(initial_state ? initial_state + sbase : nullptr);
    const int64_t ntok = eos - bos;
    const int64_t nint = (ntok + kCkpt - 1) / kCkpt;
    for (int64_t j = 0; j < nint; ++j) {
        store_S(ck_ptr(j));
        const int64_t t0 = bos + j * kCkpt;
        const int64_t t1 = (t0 + kCkpt < eos) ? t0 + kCkpt : eos;
        stage(t0, t1, false);
        for (int tt = 0; tt < (int)(t1 - t0); ++tt) step(tt);
    }

    // Reverse pass.
    float dS[R][4][4];
#pragma unroll
    for (int m = 0; m < R; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const f32x4 x = dfinal ? *reinterpret_cast<const f32x4*>(dfinal + sbase + row(m) * D + col(i, 0)) : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int e = 0; e < 4; ++e) dS[m][i][e] = x[e];
        }
    int par = 0;
    float Sck[R][4][4];
    for (int64_t j = nint - 1; j >= 0; --j) {
        const int64_t t0 = bos + j * kCkpt;
        const int64_t t1 = (t0 + kCkpt < eos) ? t0 + kCkpt : eos;
        // The interval's checkpoint (the thread reads back exactly the elements it
        // wrote) and inputs.
        load_S(ck_ptr(j));
#pragma unroll
        for (int m = 0; m < R; ++m)
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int e = 0; e < 4; ++e) Sck[m][i][e] = S[m][i][e];
        stage(t0, t1, true);
        for (int64_t t = t1 - 1; t >= t0; --t) {
            const int tt = (int)(t - t0);
            // The state before token t, rebuilt from the checkpoint.
#pragma unroll
            for (int m = 0; m < R; ++m)
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int e = 0; e < 4; ++e) S[m][i][e] = Sck[m][i][e];
            for (int tau = 0; tau < tt; ++tau) step(tau);

            float kk[4][4], qq[4][4];
            lds_row(kI, tt, kk);
            lds_row(qI, tt, qq);
            const int64_t gb = t * num_v_heads + h;
            const float alpha = exp_nonpos(gI[tt]), b = bI[tt];
            float colA[4][4], colB[4][4];
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int e = 0; e < 4; ++e) colA[i][e] = colB[i][e] = 0.f;
            float s_beta = 0.f, s_dw = 0.f, s_udo = 0.f, s_dss = 0.f;
#pragma unroll
            for (int m = 0; m < R; ++m) {
                float w = 0.f;
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int e = 0; e < 4; ++e) w = fmaf(S[m][i][e], kk[i][e], w);
                w = group_sum<L>(w);
                const float vm = vI[tt][row(m)];
                const float u = b * (vm - alpha * w);
                const float dom = doI[tt][row(m)];
                float du = 0.f;
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        dS[m][i][e] = fmaf(scale * dom, qq[i][e], dS[m][i][e]);
                        du = fmaf(dS[m][i][e], kk[i][e], du);
                    }
                du = group_sum<L>(du);
                if (c == 0) {
                    dv[gb * D + row(m)] = b * du;
                    s_beta = fmaf(du, vm - alpha * w, s_beta);
                    s_dw = fmaf(du, w, s_dw);
                    s_udo = fmaf(u, dom, s_udo);
                }
                const float ab = alpha * b;
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        colA[i][e] = fmaf(S[m][i][e], dom, colA[i][e]);
                        colB[i][e] = fmaf(dS[m][i][e], u, colB[i][e]) - ab * S[m][i][e] * du;
                        s_dss = fmaf(dS[m][i][e], S[m][i][e], s_dss);
                        dS[m][i][e] = alpha * dS[m][i][e] - ab * du * kk[i][e];
                    }
            }
            // Column sums over the row groups of the wave, then over the waves.
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int e = 0; e < 4; ++e)
#pragma unroll
                    for (int mask = L; mask < WL; mask *= 2) {
                        colA[i][e] += __shfl_xor(colA[i][e], mask);
                        colB[i][e] += __shfl_xor(colB[i][e], mask);
                    }
#pragma unroll
            for (int mask = 1; mask < WL; mask *= 2) {
                s_beta += __shfl_xor(s_beta, mask);
                s_dw += __shfl_xor(s_dw, mask);
                s_udo += __shfl_xor(s_udo, mask);
                s_dss += __shfl_xor(s_dss, mask);
            }
            if (ln < L) {
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        red[par][wv][0][col(i, e)] = colA[i][e];
                        red[par][wv][1][col(i, e)] = colB[i][e];
                    }
            }
            if (ln == 0) {
                reds[par][wv][0] = s_beta;
                reds[par][wv][1] = s_dw;
                reds[par][wv][2] = s_udo;
                reds[par][wv][3] = s_dss;
            }
            __syncthreads();
            float sb = 0.f, sdw = 0.f, sudo = 0.f, sdss = 0.f;
#pragma unroll
            for (int x = 0; x < NW; ++x) {
                sb += reds[par][x][0];
                sdw += reds[par][x][1];
                sudo += reds[par][x][2];
                sdss += reds[par][x][3];
            }
            for (int jj = tid; jj < D; jj += NT) {
                float a = 0.f, bb = 0.f;
#pragma unroll
                for (int x = 0; x < NW; ++x) {
                    a += red[par][x][0][jj];
                    bb += red[par][x][1][jj];
                }
                const float kj = kI[tt][jj];
                dq_v[gb * D + jj] = scale * fmaf(alpha, a, kj * sudo);
                dk_v[gb * D + jj] = bb;
            }
            if (tid == 0) {
                dg[gb] = alpha * (sdss - b * sdw);
                dbeta[gb] = sb;
            }
            par ^= 1;   // the other buffer is free: every thread has passed this token's barrier
        }
    }
    if (dinit) {
#pragma unroll
        for (int m = 0; m < R; ++m)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                *reinterpret_cast<f32x4*>(dinit + sbase + row(m) * D + col(i, 0)) = f32x4{dS[m][i][0], dS[m][i][1], dS[m][i][2], dS[m][i][3]};
    }
}

// dq, dk of a QK head: the sum of its V heads' parts, in V-head order.
__global__ void backward_group_sum_kernel(const float* __restrict__ part, float* __restrict__ dst, int64_t rows,
                                          int32_t num_qk_heads, int32_t group, int32_t d) {
    const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;   // over rows * num_qk_heads * d
    if (e >= rows * num_qk_heads * d) return;
    const int64_t t = e / ((int64_t)num_qk_heads * d);
    const int64_t r = e % ((int64_t)num_qk_heads * d);
    const int hq = (int)(r / d), j = (int)(r % d);
    const float* p = part + ((t * num_qk_heads + hq) * group) * (int64_t)d + j;
    float s = 0.f;
    for (int x = 0; x < group; ++x) s += p[(int64_t)x * d];
    dst[e] = s;
}

size_t backward_workspace_bytes(int64_t total_tokens, int32_t num_seqs, int32_t num_v_heads, int32_t d) {
    const int64_t slots = total_tokens / kCkpt + num_seqs;
    const size_t ck = (size_t)slots * num_v_heads * d * d * sizeof(float);
    const size_t part = (size_t)total_tokens * num_v_heads * d * sizeof(float);
    return ck + 2 * part;
}

template <int D, bool BF16>
static hipError_t launch_bwd_t(const BackwardArgs& a, hipStream_t stream) {
    float* ws = static_cast<float*>(a.workspace);
    const int64_t slots = a.total_tokens / kCkpt + a.num_seqs;
    float* ckpt = ws;
    float* dq_v = ckpt + (size_t)slots * a.num_v_heads * D * D;
    float* dk_v = dq_v + (size_t)a.total_tokens * a.num_v_heads * D;
    prof::begin(stream, "gdn_backward");
    hipLaunchKernelGGL((backward_kernel<D, BF16>), dim3((unsigned)((int64_t)a.num_seqs * a.num_v_heads)),
                       dim3(BwdShape<D>::NT), 0, stream, a.q, a.k, a.v, a.g, a.beta, a.initial_state, a.cu_seqlens,
                       a.total_tokens, a.num_qk_heads, a.num_v_heads, a.scale, a.d_out, a.d_final_state, dq_v, dk_v,
                       a.dv, a.dg, a.dbeta, a.d_initial_state, ckpt);
    prof::end(stream);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.total_tokens == 0) return e;
    const int64_t n = a.total_tokens * a.num_qk_heads * D;
    const int group = a.num_v_heads / a.num_qk_heads;
    prof::begin(stream, "gdn_backward_group_sum");
    hipLaunchKernelGGL(backward_group_sum_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, dq_v,
                       a.dq, a.total_tokens, a.num_qk_heads, group, D);
    hipLaunchKernelGGL(backward_group_sum_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, dk_v,
                       a.dk, a.total_tokens, a.num_qk_heads, group, D);
    prof::end(stream);
    return hipGetLastError();
}

hipError_t launch_backward(const BackwardArgs& a, hipStream_t stream) {
    const bool bf = a.bf16;
    switch (a.d) {
        case 16: return bf ? launch_bwd_t<16, true>(a, stream) : launch_bwd_t<16, false>(a, stream);
        case 32: return bf ? launch_bwd_t<32, true>(a, stream) : launch_bwd_t<32, false>(a, stream);
        case 64: return bf ? launch_bwd_t<64, true>(a, stream) : launch_bwd_t<64, false>(a, stream);
        case 128: return bf ? launch_bwd_t<128, true>(a, stream) : launch_bwd_t<128, false>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace gdn
