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

constexpr int kTokBatch = 16;   // multi-token decode: tokens staged in LDS at a time

// Fused input prologue of the decode step (one token per sequence).
struct DecodeConv {
    const void* x;     // [N, C] raw q | k | v channels, C = (2 Hqk + Hv) D
    const float* w;    // [C, K]
    const void* hin;   // [N, K - 1, C] history (oldest first), or null (zeros)
    void* hout;        // [N, K - 1, C] new history, or null; never overlaps hin
    bool silu;
};

// The fused prologue of one workgroup: channel t < 3 D of its inputs (its QK
// head's q, then k, then its V head's v channels), CPT channels per thread.
// Its loads are issued before the state's (global loads complete in order, so
// loads issued after the state's would wait for all of it).
template <int D, bool BF16, int K, int NT>
struct ConvPhase {
    static constexpr int CPT = (3 * D + NT - 1) / NT;
    static constexpr int KH = K > 1 ? K - 1 : 1;
    uint32_t h[CPT][KH];   // history rows (input bits), oldest first
    uint32_t x[CPT];       // the token
    float w[CPT][K];       // taps
    int64_t ch[CPT];       // channel index in the token row

    __device__ __forceinline__ static uint32_t ld(const void* p, int64_t i) {
        if constexpr (BF16) return reinterpret_cast<const uint16_t*>(p)[i];
        else return __float_as_uint(reinterpret_cast<const float*>(p)[i]);
    }
    __device__ __forceinline__ static float widen(uint32_t r) {
        if constexpr (BF16) return __uint_as_float(r << 16);
        else return __uint_as_float(r);
    }

    __device__ __forceinline__ void load(const DecodeConv& cv, int n, int h_, int hq, int hqk, int hv, int tid) {
        const int64_t C = (int64_t)(2 * hqk + hv) * D;
        // Sequence n's history rows through a buffer resource: with no history its range is
        // empty and every read returns 0, so the loads need no branch (a branch here made the
        // wave wait for the first of them before issuing the rest).
        constexpr int ES = BF16 ? 2 : 4;
        const char* hbase = cv.hin ? reinterpret_cast<const char*>(cv.hin) + (int64_t)n * (K - 1) * C * ES
                                   : reinterpret_cast<const char*>(cv.x);
        const __amdgpu_buffer_rsrc_t hist = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<char*>(hbase), (short)0, cv.hin ? (int)((K - 1) * C * ES) : 0, 0x00020000);
#pragma unroll
        for (int r = 0; r < CPT; ++r) {
            const int t = tid + r * NT;
            const int tt = t < 3 * D ? t : 0;   // threads past the last channel load channel 0, store nothing
            const int part = tt / D, j = tt % D;
            ch[r] = part == 0 ? (int64_t)hq * D + j
                    : part == 1 ? (int64_t)(hqk + hq) * D + j
                                : (int64_t)2 * hqk * D + (int64_t)h_ * D + j;
#pragma unroll
            for (int i = 0; i < K - 1; ++i) {
                const uint32_t off = (uint32_t)(((int64_t)i * C + ch[r]) * (BF16 ? 2 : 4));
                if constexpr (BF16) h[r][i] = __builtin_amdgcn_raw_buffer_load_b16(hist, (int)off, 0, 0);
                else h[r][i] = __builtin_amdgcn_raw_buffer_load_b32(hist, (int)off, 0, 0);
            }
            x[r] = ld(cv.x, (int64_t)n * C + ch[r]);
#pragma unroll
            for (int i = 0; i < K; ++i) w[r][i] = cv.w[ch[r] * K + i];
        }
    }

    // y = sum_{i < K - 1} w[i] hist[i] + w[K - 1] x, optionally y * sigmoid(y), into s[t]; the
    // channels' new history (old rows 1 .. K - 2, then the token) to hout, the q and k channels only
    // by the first V head of their QK head, the one workgroup that owns them.
    __device__ __forceinline__ void finish(const DecodeConv& cv, int n, int h_, int hqk, int hv, int tid,
                                           float* __restrict__ s) const {
        const int64_t C = (int64_t)(2 * hqk + hv) * D;
        const bool owns_qk = (h_ % (hv / hqk)) == 0;
#pragma unroll
        for (int r = 0; r < CPT; ++r) {
            const int t = tid + r * NT;
            if (t >= 3 * D) break;
            float y = 0.f;
#pragma unroll
            for (int i = 0; i < K - 1; ++i) y = fmaf(w[r][i], widen(h[r][i]), y);
            y = fmaf(w[r][K - 1], widen(x[r]), y);
            if (cv.silu) y = y * __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(y * -1.4426950408889634f));
            s[t] = y;
            if (cv.hout && (t >= 2 * D || owns_qk)) {
#pragma unroll
                for (int i = 0; i < K - 1; ++i) {
                    // new row i: old row i + 1, the last one the token ((i + 1) % KH only keeps the
                    // unused branch's index in range)
                    const uint32_t b = (i == K - 2) ? x[r] : h[r][(i + 1) % KH];
                    const int64_t o = ((int64_t)n * (K - 1) + i) * C + ch[r];
                    if constexpr (BF16) reinterpret_cast<uint16_t*>(cv.hout)[o] = (uint16_t)b;
                    else reinterpret_cast<float*>(cv.hout)[o] = __uint_as_float(b);
                }
            }
        }
    }
};

// Sequences of a slot-indexed batch in the order of their pool rows: the
// sequence whose key (pool row, then batch position) ranks r-th among the
// batch's keys. Keys are distinct, so the ranks are a permutation of the
// batch and every sequence is taken by exactly one rank. Padding entries sort
// after every pool row. Workgroups that run at the same time then stream
// state rows that lie close together in the pool; on MI355X that reads and
// writes the 2 MiB rows of a 384-row pool in random order as fast as in
// ascending order. Needs num_seqs <= NT (one key per thread) and
// num_slots < kOrdPadRow.
constexpr uint32_t kOrdPadRow = (1u << 22) - 1;

template <int NT>
__device__ __forceinline__ int sequence_of_rank(const int32_t* __restrict__ state_indices,
                                                int32_t num_slots, int num_seqs, int r, int tid) {
    __shared__ uint4 s_key4[NT / 4];
    __shared__ int s_seq;
    uint32_t* s_key = reinterpret_cast<uint32_t*>(s_key4);
    uint32_t key = 0xFFFFFFFFu;
    if (tid < num_seqs) {
        const int32_t s = state_indices[tid];
        const uint32_t row = (s >= 0 && s < num_slots) ? static_cast<uint32_t>(s) : kOrdPadRow;
        key = (row << 9) | static_cast<uint32_t>(tid);
    }
    s_key[tid] = key;   // entries past the batch hold the largest key
    __syncthreads();
    if (tid < num_seqs) {
        int rank = 0;
        for (int j = 0; j < (num_seqs + 3) / 4; ++j) {
            const uint4 kk = s_key4[j];
            rank += (kk.x < key) + (kk.y < key) + (kk.z < key) + (kk.w < key);
        }
        if (rank == r) s_seq = tid;
    }
    __syncthreads();
    return s_seq;
}

// CK > 0: q, k and v come from the fused input prologue with K = CK taps (the
// q, k, v pointers are unused); CK = 0: from the q, k, v arrays. ORD: a
// slot-indexed batch taken in pool-row order (sequence_of_rank).
template <int D, bool BF16, bool QKN, int CK = 0, bool ORD = false>
__global__ __launch_bounds__(512) void decode_step_kernel(
    const void* __restrict__ q_, const void* __restrict__ k_, const void* __restrict__ v_,
    const float* __restrict__ g, const float* __restrict__ beta, float* __restrict__ state,
    int32_t num_qk_heads, int32_t num_v_heads, float scale, void* __restrict__ out_,
    const int32_t* __restrict__ state_indices, int32_t num_slots, DecodeConv cv) {
    constexpr int L = D / 16;                    // lanes per state row (16 floats each)
    constexpr int NT = (D * L < 512) ? D * L : 512;
    constexpr int ROWS_PER_PASS = NT / L;
    constexpr int R = D / ROWS_PER_PASS;         // rows per thread
    static_assert(R * ROWS_PER_PASS == D, "rows must tile");

    const int tid = threadIdx.x;
    const int c = tid % L;                       // lane within the row group
    const int r0 = tid / L;
    const int h = static_cast<int>(blockIdx.x % num_v_heads);
    int n = static_cast<int>(blockIdx.x / num_v_heads);
    if constexpr (ORD)
        n = sequence_of_rank<NT>(state_indices, num_slots, static_cast<int>(gridDim.x / num_v_heads), n, tid);
    const int64_t sh = (int64_t)n * num_v_heads + h;   // sequence * num_v_heads + head
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

    // Fused prologue: its few loads go out ahead of the state's.
    ConvPhase<D, BF16, (CK > 0 ? CK : 1), NT> cp;
    if constexpr (CK > 0) {
        cp.load(cv, n, h, hq, num_qk_heads, num_v_heads, tid);
        __builtin_amdgcn_sched_barrier(0);
    }

    // The state loads (first of all without the prologue): R rows x 4 float4 per thread.
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
    __shared__ float s_qkv[CK > 0 ? 3 * D : 1];   // fused prologue: q, k, v of this workgroup
    if constexpr (CK > 0) {
        cp.finish(cv, n, h, num_qk_heads, num_v_heads, tid, s_qkv);
        __syncthreads();
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                qr[i][e] = s_qkv[4 * (c + L * i) + e];
                kr[i][e] = s_qkv[D + 4 * (c + L * i) + e];
            }
    } else if constexpr (BF16) {
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
        if constexpr (CK > 0) vi = s_qkv[2 * D + row];
        else if constexpr (BF16) vi = bf16_bits_to_float(reinterpret_cast<const uint16_t*>(v_)[vo_base + row]);
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
    // The tokens' inputs (k and q of the QK head, v of the V head, g, beta) are
    // staged in LDS by the whole workgroup, kTokBatch tokens at a time, right
    // after the state loads are issued. Rows of the state are independent, so
    // each thread runs all staged tokens on its first row, stores it, then on
    // its second row: the first row's work and store overlap the second row's
    // load, which would otherwise all wait for the slowest of them.
    using word_t = typename std::conditional<BF16, uint2, float4>::type;   // 4 elements of k or q
    constexpr int KQW = D / 4;                                              // words per k (or q) row
    __shared__ word_t s_k[kTokBatch][KQW], s_q[kTokBatch][KQW];
    __shared__ float s_v[kTokBatch][D];
    __shared__ float s_g[kTokBatch], s_b[kTokBatch];

    f32x4* S = reinterpret_cast<f32x4*>(state + (srow * num_v_heads + h) * (int64_t)D * D);
    f32x4 s[R][4];
#pragma unroll
    for (int m = 0; m < R; ++m)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            s[m][i] = __builtin_nontemporal_load(&S[(r0 + m * ROWS_PER_PASS) * (D / 4) + c + L * i]);

    for (int t0 = 0; t0 < num_tokens; t0 += kTokBatch) {
        const int nb = (num_tokens - t0 < kTokBatch) ? num_tokens - t0 : kTokBatch;
        if (t0 > 0) __syncthreads();   // the previous batch's LDS reads are done
        for (int w = tid; w < nb * KQW; w += NT) {
            const int tt = w / KQW, j = w % KQW;
            const int64_t tok = (int64_t)n * num_tokens + t0 + tt;
            const int64_t qk_base = (tok * num_qk_heads + hq) * D;
            s_k[tt][j] = reinterpret_cast<const word_t*>(reinterpret_cast<const char*>(k_) + qk_base * (BF16 ? 2 : 4))[j];
            s_q[tt][j] = reinterpret_cast<const word_t*>(reinterpret_cast<const char*>(q_) + qk_base * (BF16 ? 2 : 4))[j];
        }
        for (int w = tid; w < nb * D; w += NT) {
            const int tt = w / D, j = w % D;
            const int64_t gb = ((int64_t)n * num_tokens + t0 + tt) * num_v_heads + h;
            if constexpr (BF16) s_v[tt][j] = bf16_bits_to_float(reinterpret_cast<const uint16_t*>(v_)[gb * D + j]);
            else s_v[tt][j] = reinterpret_cast<const float*>(v_)[gb * D + j];
        }
        if (tid < nb) {
            const int64_t gb = ((int64_t)n * num_tokens + t0 + tid) * num_v_heads + h;
            s_g[tid] = g[gb];
            s_b[tid] = beta[gb];
        }
        __syncthreads();

#pragma unroll
        for (int m = 0; m < R; ++m) {
            const int row = r0 + m * ROWS_PER_PASS;
#pragma unroll 1
            for (int tt = 0; tt < nb; ++tt) {
                const int64_t gb = ((int64_t)n * num_tokens + t0 + tt) * num_v_heads + h;
                word_t kraw[4], qraw[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    kraw[i] = s_k[tt][c + L * i];
                    qraw[i] = s_q[tt][c + L * i];
                }
                // Key / query element e of this lane's slice i (bf16: from the packed bits).
                auto kf = [&](int i, int e) {
                    if constexpr (BF16) {
                        const uint32_t w = (e < 2) ? kraw[i].x : kraw[i].y;
                        return __uint_as_float((e & 1) ? (w & 0xFFFF0000u) : (w << 16));
                    } else {
                        return e == 0 ? kraw[i].x : e == 1 ? kraw[i].y : e == 2 ? kraw[i].z : kraw[i].w;
                    }
                };
                auto qf = [&](int i, int e) {
                    if constexpr (BF16) {
                        const uint32_t w = (e < 2) ? qraw[i].x : qraw[i].y;
                        return __uint_as_float((e & 1) ? (w & 0xFFFF0000u) : (w << 16));
                    } else {
                        return e == 0 ? qraw[i].x : e == 1 ? qraw[i].y : e == 2 ? qraw[i].z : qraw[i].w;
                    }
                };
                const float alpha = exp_nonpos(s_g[tt]);
                const float bt = s_b[tt];
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
                float kq = 0.f, a = 0.f, bq = 0.f;
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        kq = fmaf(kf(i, e), qf(i, e), kq);
                        a = fmaf(s[m][i][e], kf(i, e), a);
                        bq = fmaf(s[m][i][e], qf(i, e), bq);
                    }
                kq = group_sum<L>(kq) * (rk * rq);
                a = group_sum<L>(a) * rk;
                bq = group_sum<L>(bq) * rq;
                const float u = bt * (s_v[tt][row] - alpha * a);
                const float uk = u * rk;
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int e = 0; e < 4; ++e) s[m][i][e] = fmaf(alpha, s[m][i][e], uk * kf(i, e));
                if (c == 0) {
                    const float o = scale * fmaf(alpha, bq, u * kq);
                    if constexpr (BF16) reinterpret_cast<uint16_t*>(out_)[gb * D + row] = float_to_bf16_bits(o);
                    else reinterpret_cast<float*>(out_)[gb * D + row] = o;
                }
                if (token_states) {
                    f32x4* TS = reinterpret_cast<f32x4*>(token_states + gb * (int64_t)D * D);
#pragma unroll
                    for (int i = 0; i < 4; ++i) __builtin_nontemporal_store(s[m][i], &TS[row * (D / 4) + c + L * i]);
                }
            }
            if (t0 + nb >= num_tokens) {
#pragma unroll
                for (int i = 0; i < 4; ++i) __builtin_nontemporal_store(s[m][i], &S[row * (D / 4) + c + L * i]);
            }
        }
    }
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

template <int D, bool BF16, bool QKN, int CK>
static hipError_t launch_decode_t(const DecodeArgs& a, hipStream_t stream) {
    constexpr int L = D / 16;
    constexpr int NT = (D * L < 512) ? D * L : 512;
    const int64_t blocks = (int64_t)a.num_seqs * a.num_v_heads;
    const DecodeConv cv{a.conv_x, a.conv_w, a.conv_in, a.conv_out, a.conv_silu};
    prof::begin(stream, CK > 0 ? "gdn_decode_conv" : "gdn_decode_step");
    bool ordered = false;
    if constexpr (CK == 0)
        ordered = a.state_indices != nullptr && a.num_seqs <= NT && (uint32_t)a.num_slots < kOrdPadRow;
    if (ordered)
        hipLaunchKernelGGL((decode_step_kernel<D, BF16, QKN, CK, true>), dim3((unsigned)blocks), dim3(NT), 0,
                           stream, a.q, a.k, a.v, a.g, a.beta, a.state, a.num_qk_heads, a.num_v_heads, a.scale,
                           a.out, a.state_indices, a.num_slots, cv);
    else
        hipLaunchKernelGGL((decode_step_kernel<D, BF16, QKN, CK>), dim3((unsigned)blocks), dim3(NT), 0, stream,
                           a.q, a.k, a.v, a.g, a.beta, a.state, a.num_qk_heads, a.num_v_heads, a.scale, a.out,
                           a.state_indices, a.num_slots, cv);
    prof::end(stream);
    return hipGetLastError();
}

template <int D, bool BF16, int CK>
static hipError_t launch_decode_c(const DecodeArgs& a, hipStream_t stream) {
    return a.qk_norm ? launch_decode_t<D, BF16, true, CK>(a, stream) : launch_decode_t<D, BF16, false, CK>(a, stream);
}

template <int D, bool BF16>
static hipError_t launch_decode_n(const DecodeArgs& a, hipStream_t stream) {
    switch (a.conv_K) {
        case 0: return launch_decode_c<D, BF16, 0>(a, stream);
        case 1: return launch_decode_c<D, BF16, 1>(a, stream);
        case 2: return launch_decode_c<D, BF16, 2>(a, stream);
        case 3: return launch_decode_c<D, BF16, 3>(a, stream);
        case 4: return launch_decode_c<D, BF16, 4>(a, stream);
        default: return hipErrorInvalidValue;
    }
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
