// Single-token decode step of the Gated DeltaNet recurrence, state updated in
// place in HBM.
//
// Per (sequence, V head) with state S (d x d fp32), unit key k, query q:
//     a = S k,  b = S q                      (both from ONE read of the old S)
//     u = beta * (v - alpha * a)             delta-rule write
//     S <- alpha * S + u k^T                 (ONE write of the new S)
//     o = scale * (alpha * b + u * (k . q))  = scale * S_new q
// The last line uses S_new q = alpha S q + u (k^T q), so the output needs no
// second pass over the state. Rows of S are independent: every row i needs
// only its own dot products a_i, b_i.
//
// With a state pool, sequence n's state is row state_indices[n] of the pool;
// an index outside the pool marks a padding entry (state untouched, zero
// outputs).
//
// Memory pattern: the state is >99% of the bytes (64 KiB per head at d = 128).
// Each thread owns R rows x 16 columns as four dwordx4 loads per row; the L
// lanes that share a row are adjacent, so one load instruction of a wave
// covers 64/L rows with fully used 128-byte segments. All loads of a thread
// are issued before any arithmetic. At d = 128 a workgroup is 512 threads
// with two rows each: on gfx950 that streams the in-place read + write about
// 4% faster than 256 threads with four rows (same bytes per workgroup, half
// the registers per thread, twice the waves). Several heads per workgroup,
// one after another, were slower: each head's load, compute and store then
// run back to back. Loads and stores are non-temporal: the
// state of a large batch is touched once per step and exceeds the last-level
// cache.
#include "gdn_common.h"
#include "gdn_internal.h"

#include <type_traits>

namespace gdn {

typedef float f32x4 __attribute__((ext_vector_type(4)));

template <int D, bool BF16, bool QKN>
__global__ __launch_bounds__(512) void decode_step_kernel(
    const void* __restrict__ q_, const void* __restrict__ k_, const void* __restrict__ v_,
    const float* __restrict__ g, const float* __restrict__ beta, float* __restrict__ state,
    int32_t num_qk_heads, int32_t num_v_heads, float scale, void* __restrict__ out_,
    const int32_t* __restrict__ state_indices, int32_t num_slots) {
    constexpr int L = D / 16;                    // lanes per state row (16 floats each)
    constexpr int NT = (D * L < 512) ? D * L : 512;
    constexpr int ROWS_PER_PASS = NT / L;
    constexpr int R = D / ROWS_PER_PASS;         // rows per thread
    static_assert(R * ROWS_PER_PASS == D, "rows must tile");

    const int tid = threadIdx.x;
    const int c = tid % L;                       // lane within the row group
    const int r0 = tid / L;
    const int64_t sh = blockIdx.x;               // sequence * num_v_heads + head
    const int n = static_cast<int>(sh / num_v_heads);
    const int h = static_cast<int>(sh % num_v_heads);
    const int hq = h / (num_v_heads / num_qk_heads);
    const int64_t vo_base = sh * D;

    // Padding entry of a slot-indexed batch: no state access, zero outputs.
    const int64_t srow = state_row(state_indices, num_slots, n);
    if (srow < 0) {
        if (c == 0) {
#pragma unroll
            for (int m = 0; m < R; ++m) {
                const int row = r0 + m * ROWS_PER_PASS;
                if constexpr (BF16) reinterpret_cast<uint16_t*>(out_)[vo_base + row] = 0;
                else reinterpret_cast<float*>(out_)[vo_base + row] = 0.f;
            }
        }
        return;
    }
    f32x4* S = reinterpret_cast<f32x4*>(state + (srow * num_v_heads + h) * (int64_t)D * D);

    // Issue the state loads first: R rows x 4 float4 per thread.
    f32x4 s[R][4];
#pragma unroll
    for (int m = 0; m < R; ++m) {
        const int row = r0 + m * ROWS_PER_PASS;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            s[m][i] = __builtin_nontemporal_load(&S[row * (D / 4) + c + L * i]);
    }

    // Key / query slices owned by this lane: columns 4 * (c + L * i) .. +3.
    float kr[4][4], qr[4][4];
    const int64_t qk_base = ((int64_t)n * num_qk_heads + hq) * D;
    if constexpr (BF16) {
        const uint2* k2 = reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(k_) + qk_base);
        const uint2* q2 = reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(q_) + qk_base);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint2 kk = k2[c + L * i], qq = q2[c + L * i];
            kr[i][0] = __uint_as_float(kk.x << 16); kr[i][1] = __uint_as_float(kk.x & 0xFFFF0000u);
            kr[i][2] = __uint_as_float(kk.y << 16); kr[i][3] = __uint_as_float(kk.y & 0xFFFF0000u);
            qr[i][0] = __uint_as_float(qq.x << 16); qr[i][1] = __uint_as_float(qq.x & 0xFFFF0000u);
            qr[i][2] = __uint_as_float(qq.y << 16); qr[i][3] = __uint_as_float(qq.y & 0xFFFF0000u);
        }
    } else {
        const float4* k4 = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(k_) + qk_base);
        const float4* q4 = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(q_) + qk_base);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float4 kk = k4[c + L * i], qq = q4[c + L * i];
            kr[i][0] = kk.x; kr[i][1] = kk.y; kr[i][2] = kk.z; kr[i][3] = kk.w;
            qr[i][0] = qq.x; qr[i][1] = qq.y; qr[i][2] = qq.z; qr[i][3] = qq.w;
        }
    }
    const float alpha = exp_nonpos(g[sh]);
    const float b = beta[sh];

    // In-kernel L2 normalisation: k and q enter through the factors rk, rq
    // (1 when off: every product below is then exactly the plain one).
    float rk = 1.f, rq = 1.f;
    if constexpr (QKN) {
        float nk = 0.f, nq = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                nk = fmaf(kr[i][e], kr[i][e], nk);
                nq = fmaf(qr[i][e], qr[i][e], nq);
            }
        rk = rsqrtf(group_sum<L>(nk) + kQkNormEps);
        rq = rsqrtf(group_sum<L>(nq) + kQkNormEps);
    }
    float kq = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) kq = fmaf(kr[i][e], qr[i][e], kq);
    kq = group_sum<L>(kq) * (rk * rq);

#pragma unroll
    for (int m = 0; m < R; ++m) {
        const int row = r0 + m * ROWS_PER_PASS;
        float a = 0.f, bq = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                a = fmaf(s[m][i][e], kr[i][e], a);
                bq = fmaf(s[m][i][e], qr[i][e], bq);
            }
        }
        a = group_sum<L>(a) * rk;
        bq = group_sum<L>(bq) * rq;
        float vi;
        if constexpr (BF16) vi = bf16_bits_to_float(reinterpret_cast<const uint16_t*>(v_)[vo_base + row]);
        else vi = reinterpret_cast<const float*>(v_)[vo_base + row];
        const float u = b * (vi - alpha * a);
        const float uk = u * rk;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f32x4 t;
#pragma unroll
            for (int e = 0; e < 4; ++e) t[e] = fmaf(alpha, s[m][i][e], uk * kr[i][e]);
            __builtin_nontemporal_store(t, &S[row * (D / 4) + c + L * i]);
        }
        if (c == 0) {
            const float o = scale * fmaf(alpha, bq, u * kq);
            if constexpr (BF16) reinterpret_cast<uint16_t*>(out_)[vo_base + row] = float_to_bf16_bits(o);
            else reinterpret_cast<float*>(out_)[vo_base + row] = o;
        }
    }
}

// Several tokens per sequence from one state (draft tokens of multi-token
// prediction, verified in one call): the state is read once, advanced token by
// token in registers with the same per-token update as above, and written
// once; optionally the state after every token is stored as well, so that a
// caller can resume from the last accepted token. Inputs are token-major per
// sequence: token t of sequence n is row n * num_tokens + t.
template <int D, bool BF16, bool QKN>
__global__ __launch_bounds__(512) void decode_multi_kernel(
    const void* __restrict__ q_, const void* __restrict__ k_, const void* __restrict__ v_,
    const float* __restrict__ g, const float* __restrict__ beta, float* __restrict__ state, int32_t num_tokens,
    int32_t num_qk_heads, int32_t num_v_heads, float scale, void* __restrict__ out_,
    float* __restrict__ token_states, const int32_t* __restrict__ state_indices, int32_t num_slots) {
    constexpr int L = D / 16;
    constexpr int NT = (D * L < 512) ? D * L : 512;
    constexpr int ROWS_PER_PASS = NT / L;
    constexpr int R = D / ROWS_PER_PASS;
    static_assert(R * ROWS_PER_PASS == D, "rows must tile");

    const int tid = threadIdx.x;
    const int c = tid % L;
    const int r0 = tid / L;
    const int64_t sh = blockIdx.x;               // sequence * num_v_heads + head
    const int n = static_cast<int>(sh / num_v_heads);
    const int h = static_cast<int>(sh % num_v_heads);
    const int hq = h / (num_v_heads / num_qk_heads);

    const int64_t srow = state_row(state_indices, num_slots, n);
    if (srow < 0) {   // padding entry: zero outputs, no state access
        if (c == 0) {
            for (int t = 0; t < num_tokens; ++t) {
                const int64_t ob = (((int64_t)n * num_tokens + t) * num_v_heads + h) * D;
#pragma unroll
                for (int m = 0; m < R; ++m) {
                    const int row = r0 + m * ROWS_PER_PASS;
                    if constexpr (BF16) reinterpret_cast<uint16_t*>(out_)[ob + row] = 0;
                    else reinterpret_cast<float*>(out_)[ob + row] = 0.f;
                }
            }
        }
        return;
    }
    // One token's inputs for this lane: k and q slices, the value of each owned
    // row, g and beta. Token t + 1's are requested before token t is computed.
    using raw_t = typename std::conditional<BF16, uint2, float4>::type;
    struct TokIn {
        raw_t kraw[4], qraw[4];
        float vi[R];
        float g, b;
    };
    auto load_tok = [&](int t, TokIn& in) {
        const int64_t tok = (int64_t)n * num_tokens + t;
        const int64_t qk_base = (tok * num_qk_heads + hq) * D;
        const raw_t* k2 = reinterpret_cast<const raw_t*>(reinterpret_cast<const char*>(k_) + qk_base * (BF16 ? 2 : 4));
        const raw_t* q2 = reinterpret_cast<const raw_t*>(reinterpret_cast<const char*>(q_) + qk_base * (BF16 ? 2 : 4));
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            in.kraw[i] = k2[c + L * i];
            in.qraw[i] = q2[c + L * i];
        }
        const int64_t gb = tok * num_v_heads + h;
#pragma unroll
        for (int m = 0; m < R; ++m) {
            const int row = r0 + m * ROWS_PER_PASS;
            if constexpr (BF16) in.vi[m] = bf16_bits_to_float(reinterpret_cast<const uint16_t*>(v_)[gb * D + row]);
            else in.vi[m] = reinterpret_cast<const float*>(v_)[gb * D + row];
        }
        in.g = g[gb];
        in.b = beta[gb];
    };

    f32x4* S = reinterpret_cast<f32x4*>(state + (srow * num_v_heads + h) * (int64_t)D * D);
    f32x4 s[R][4];
#pragma unroll
    for (int m = 0; m < R; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            s[m][i] = __builtin_nontemporal_load(&S[(r0 + m * ROWS_PER_PASS) * (D / 4) + c + L * i]);
    TokIn cur, nxt;
    load_tok(0, cur);

    for (int t = 0; t < num_tokens; ++t) {
        if (t + 1 < num_tokens) load_tok(t + 1, nxt);
        const int64_t gb = ((int64_t)n * num_tokens + t) * num_v_heads + h;
        // Key / query element e of this lane's slice i (bf16: from the packed bits).
        auto kf = [&](int i, int e) {
            if constexpr (BF16) {
                const uint32_t w = (e < 2) ? cur.kraw[i].x : cur.kraw[i].y;
                return __uint_as_float((e & 1) ? (w & 0xFFFF0000u) : (w << 16));
            } else {
                return e == 0 ? cur.kraw[i].x : e == 1 ? cur.kraw[i].y : e == 2 ? cur.kraw[i].z : cur.kraw[i].w;
            }
        };
        auto qf = [&](int i, int e) {
            if constexpr (BF16) {
                const uint32_t w = (e < 2) ? cur.qraw[i].x : cur.qraw[i].y;
                return __uint_as_float((e & 1) ? (w & 0xFFFF0000u) : (w << 16));
            } else {
                return e == 0 ? cur.qraw[i].x : e == 1 ? cur.qraw[i].y : e == 2 ? cur.qraw[i].z : cur.qraw[i].w;
            }
        };
        const float alpha = exp_nonpos(cur.g);
        float rk = 1.f, rq = 1.f;   // in-kernel L2 normalisation factors (1 when off)
        if constexpr (QKN) {
            float nk = 0.f, nq = 0.f;
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    nk = fmaf(kf(i, e), kf(i, e), nk);
                    nq = fmaf(qf(i, e), qf(i, e), nq);
                }
            rk = rsqrtf(group_sum<L>(nk) + kQkNormEps);
            rq = rsqrtf(group_sum<L>(nq) + kQkNormEps);
        }
        float kq = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int e = 0; e < 4; ++e) kq = fmaf(kf(i, e), qf(i, e), kq);
        kq = group_sum<L>(kq) * (rk * rq);
        const int64_t vo_base = gb * D;
#pragma unroll
        for (int m = 0; m < R; ++m) {
            const int row = r0 + m * ROWS_PER_PASS;
            float a = 0.f, bq = 0.f;
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    a = fmaf(s[m][i][e], kf(i, e), a);
                    bq = fmaf(s[m][i][e], qf(i, e), bq);
                }
            a = group_sum<L>(a) * rk;
            bq = group_sum<L>(bq) * rq;
            const float u = cur.b * (cur.vi[m] - alpha * a);
            const float uk = u * rk;
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int e = 0; e < 4; ++e) s[m][i][e] = fmaf(alpha, s[m][i][e], uk * kf(i, e));
            if (c == 0) {
                const float o = scale * fmaf(alpha, bq, u * kq);
                if constexpr (BF16) reinterpret_cast<uint16_t*>(out_)[vo_base + row] = float_to_bf16_bits(o);
                else reinterpret_cast<float*>(out_)[vo_base + row] = o;
            }
        }
        if (token_states) {
            f32x4* TS = reinterpret_cast<f32x4*>(token_states + gb * (int64_t)D * D);
#pragma unroll
            for (int m = 0; m < R; ++m)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    __builtin_nontemporal_store(s[m][i], &TS[(r0 + m * ROWS_PER_PASS) * (D / 4) + c + L * i]);
        }
        cur = nxt;
    }
#pragma unroll
    for (int m = 0; m < R; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            __builtin_nontemporal_store(s[m][i], &S[(r0 + m * ROWS_PER_PASS) * (D / 4) + c + L * i]);
}

template <int D, bool BF16, bool QKN>
static hipError_t launch_decode_multi_t(const DecodeArgs& a, hipStream_t stream) {
    constexpr int L = D / 16;
    constexpr int NT = (D * L < 512) ? D * L : 512;
    const int64_t blocks = (int64_t)a.num_seqs * a.num_v_heads;
    prof::begin(stream, "gdn_decode_multi");
    hipLaunchKernelGGL((decode_multi_kernel<D, BF16, QKN>), dim3((unsigned)blocks), dim3(NT), 0, stream,
                       a.q, a.k, a.v, a.g, a.beta, a.state, a.num_tokens, a.num_qk_heads, a.num_v_heads, a.scale,
                       a.out, a.token_states, a.state_indices, a.num_slots);
    prof::end(stream);
    return hipGetLastError();
}

template <int D, bool BF16>
static hipError_t launch_decode_multi_n(const DecodeArgs& a, hipStream_t stream) {
    return a.qk_norm ? launch_decode_multi_t<D, BF16, true>(a, stream) : launch_decode_multi_t<D, BF16, false>(a, stream);
}

hipError_t launch_decode_multi(const DecodeArgs& a, hipStream_t stream) {
    const bool bf = a.bf16;
    switch (a.d) {
        case 16: return bf ? launch_decode_multi_n<16, true>(a, stream) : launch_decode_multi_n<16, false>(a, stream);
        case 32: return bf ? launch_decode_multi_n<32, true>(a, stream) : launch_decode_multi_n<32, false>(a, stream);
        case 64: return bf ? launch_decode_multi_n<64, true>(a, stream) : launch_decode_multi_n<64, false>(a, stream);
        case 128: return bf ? launch_decode_multi_n<128, true>(a, stream) : launch_decode_multi_n<128, false>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

template <int D, bool BF16, bool QKN>
static hipError_t launch_decode_t(const DecodeArgs& a, hipStream_t stream) {
    constexpr int L = D / 16;
    constexpr int NT = (D * L < 512) ? D * L : 512;
    const int64_t blocks = (int64_t)a.num_seqs * a.num_v_heads;
    prof::begin(stream, "gdn_decode_step");
    hipLaunchKernelGGL((decode_step_kernel<D, BF16, QKN>), dim3((unsigned)blocks), dim3(NT), 0, stream,
                       a.q, a.k, a.v, a.g, a.beta, a.state, a.num_qk_heads, a.num_v_heads, a.scale, a.out,
                       a.state_indices, a.num_slots);
    prof::end(stream);
    return hipGetLastError();
}

template <int D, bool BF16>
static hipError_t launch_decode_n(const DecodeArgs& a, hipStream_t stream) {
    return a.qk_norm ? launch_decode_t<D, BF16, true>(a, stream) : launch_decode_t<D, BF16, false>(a, stream);
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream) {
    const bool bf = a.bf16;
    switch (a.d) {
        case 16: return bf ? launch_decode_n<16, true>(a, stream) : launch_decode_n<16, false>(a, stream);
        case 32: return bf ? launch_decode_n<32, true>(a, stream) : launch_decode_n<32, false>(a, stream);
        case 64: return bf ? launch_decode_n<64, true>(a, stream) : launch_decode_n<64, false>(a, stream);
        case 128: return bf ? launch_decode_n<128, true>(a, stream) : launch_decode_n<128, false>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace gdn
