// Chunked bf16 prefill, segment-parallel: the whole prefill in three launches.
//
// Chunk algebra (chunk of n <= 64 tokens, entry state S (d_v x d_k), gamma =
// in-chunk cumulative sum of g, Gamma = exp(gamma)):
//   A[r][c] = beta_r exp(gamma_r - gamma_c) (k_r . k_c)   c < r   decay-masked Gram
//   Tm      = (I + A)^-1                                          UT transform
//   U       = Tm (beta * (V - Gamma * (K S^T)))                   the chunk's delta writes
//   O       = scale (Gamma * (Q S^T) + P U),  P[r][c] = exp(gamma_r - gamma_c) (q_r . k_c), c <= r
//   S_end   = Gamma_last S + U^T diag(exp(gamma_last - gamma)) K
// (unrolling the per-token rule inside the chunk: the write of token r sees
// the decayed entry state plus the chunk's earlier writes, which is the unit
// lower-triangular system (I + A) U = beta * (V - Gamma * K S^T)).
//
// Segments. S_end is affine in the entry state: over a segment of L chunks,
// S_end = S_in M_seg + H_seg, where H_seg is the segment run from S_in = 0 and
// M_seg (d_k x d_k) the run from S_in = I with V = 0. The launches:
//   pass A   every segment but a sequence's last: H (segment 0 starts from
//            the sequence's initial state, so its H is its end state) and,
//            for segments >= 1, M; one 8-wave workgroup computes both.
//   combine  S_in(1) = H_0, S_in(j+1) = S_in(j) M_j + H_j, in fp32.
//   pass C   every segment from its true entry state: outputs and, for the
//            last segment, the final state.
// Each chunk's factors (Gram products, masks, Tm, P) are computed inside the
// workgroup that uses them, so nothing but the states leaves the chip.
//
// Work split. A workgroup is one (segment, V head). Every wave of a chain
// owns 32 value columns of the 128 x 128 state (two 16-column MFMA tiles,
// fp32 accumulators held transposed: tile t, lane (g, m), element e is
// S[col][key 16 t + 4 g + e]) and needs nothing from the other waves; the
// factors of the chunk are built by all waves together in LDS. The state
// update's K^T operand is read from the token-major K tile with the LDS
// transpose read, so K is staged once.
#include "gdn_mfma.h"

namespace gdn {

using namespace mf;

namespace {

enum { kModeOut = 0, kModeHM = 1 };
constexpr size_t kSegMat = (size_t)D * D;   // floats in one 128 x 128 matrix
constexpr int kSegMats = 3;                 // H, M, S_in per (segment, V head)

// Segments: sequence n owns [f(n), f(n) + nseg_n) with f(n) = cu[n] / (64 L) + n;
// the ranges are disjoint and below total_tokens / (64 L) + num_seqs, so the
// workspace is sized on the host without reading the offsets.
__device__ __forceinline__ int64_t seg_base(const int32_t* cu, int n, int L) {
    return cu ? (int64_t)(cu[n] / (kChunk * L)) + n : 0;
}

__device__ __forceinline__ int find_seq_for_seg(const int32_t* cu, int N, int64_t s, int L) {
    if (!cu) return 0;
    int lo = 0, hi = N - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (seg_base(cu, mid, L) <= s) lo = mid;
        else hi = mid - 1;
    }
    return lo;
}

struct __attribute__((aligned(16))) SegSmem {
    uint16_t K[kChunk][RP];          // keys, token-major
    uint16_t Q[kChunk][RP];          // queries (output pass)
    uint16_t V[kChunk][RP];          // values
    uint16_t T[kChunk][CP];          // Tm, bf16
    uint16_t P[kChunk][CP];          // P, bf16 (output pass)
    float A[kChunk][kChunk + 1];     // A, fp32 (strictly lower part used)
    float Tf[kChunk][kChunk + 1];    // Tm, fp32, during the solve
    float gam[kChunk], Gam[kChunk], Dec[kChunk], bet[kChunk];
};

template <int NT>
struct SegPrefetch {
    static constexpr int NP = kChunk * (D / 8) / NT;   // 16-byte pieces per thread per 64 x 128 tile
    u32x4 k[NP], q[NP], v[NP];
    float s;                                           // g (wave 0) or beta (wave 1)
};

// Loads for one chunk of nc tokens. Rows past the end re-read row nc - 1 (they
// are zeroed when stored), so no load leaves the sequence and none is branched.
template <int MODE, int NT>
__device__ __forceinline__ void seg_fetch(SegPrefetch<NT>& pf, const uint16_t* kc, const uint16_t* qc,
                                          const uint16_t* vc, const float* gc, const float* bc, int nc, int ldk,
                                          int ldv, int num_v_heads, int tid) {
    constexpr int NP = SegPrefetch<NT>::NP;
#pragma unroll
    for (int i = 0; i < NP; ++i) {
        const int p = tid + NT * i;
        const int row = p >> 4, c8 = p & 15;                 // row-major 16-byte pieces
        const int rr = row < nc ? row : nc - 1;
        if (MODE == kModeOut) pf.q[i] = *reinterpret_cast<const u32x4*>(qc + rr * ldk + c8 * 8);
        pf.v[i] = *reinterpret_cast<const u32x4*>(vc + rr * ldv + c8 * 8);
        pf.k[i] = *reinterpret_cast<const u32x4*>(kc + rr * ldk + c8 * 8);
    }
    const int r = tid & 63;
    const float* sp = (tid < 64) ? gc : bc;
    pf.s = sp[(r < nc ? r : nc - 1) * num_v_heads];
}

template <int MODE, int NT>
__device__ __forceinline__ void seg_stage(SegSmem& sm, SegPrefetch<NT>& pf, int nc, int tid, int w) {
    constexpr int NP = SegPrefetch<NT>::NP;
    const u32x4 z = {0u, 0u, 0u, 0u};
    if (nc < kChunk) {   // partial last chunk: rows past the end are zero (uniform branch)
#pragma unroll
        for (int i = 0; i < NP; ++i) {
            const int p = tid + NT * i;
            pf.k[i] = (p >> 4) < nc ? pf.k[i] : z;
            pf.q[i] = (p >> 4) < nc ? pf.q[i] : z;
            pf.v[i] = (p >> 4) < nc ? pf.v[i] : z;
        }
        pf.s = (tid & 63) < nc ? pf.s : 0.f;
    }
#pragma unroll
    for (int i = 0; i < NP; ++i) {
        const int p = tid + NT * i;
        const int row = p >> 4, c8 = p & 15;
        *reinterpret_cast<u32x4*>(&sm.K[row][c8 * 8]) = pf.k[i];
        if (MODE == kModeOut) *reinterpret_cast<u32x4*>(&sm.Q[row][c8 * 8]) = pf.q[i];
        *reinterpret_cast<u32x4*>(&sm.V[row][c8 * 8]) = pf.v[i];
    }
    const int lane = tid & 63;
    if (w == 0) {
        // gamma = in-chunk inclusive prefix sum of g (padded rows add 0)
        float x = pf.s;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const float y = __shfl_up(x, d, 64);
            if (lane >= d) x += y;
        }
        const float glast = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 63));
        sm.gam[lane] = x;
        sm.Gam[lane] = fast_exp(x);
        sm.Dec[lane] = fast_exp(glast - x);
    } else if (w == 1) {
        sm.bet[lane] = pf.s;
    }
}

// fp32 MFMA 16x16x4: lane (g, m) supplies A[m][g] and B[g][m]; D[4 g + e][m] in element e.
__device__ __forceinline__ f32x4 mfma_f32(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Off-diagonal 16 x 16 blocks of Tm at distance L from the diagonal, one block
// per wave: Tm[bi][bj] = -Tm[bi][bi] X with X = A[bi rows][16 bj : 16 bi]
// Tm[16 bj : 16 bi][bj cols], both products in fp32 MFMA. X stays in the
// accumulators: the second product takes it as its B operand by visiting the
// reduction index 4 g + kk in step kk (the A operand follows the same order).
template <int L>
__device__ __forceinline__ void tsolve_level(SegSmem& sm, int w, int g, int m) {
    if (w < 4 - L) {
        const int bj = w, bi = w + L;
        f32x4 X = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < 4 * L; ++kk)
            X = mfma_f32(sm.A[16 * bi + m][16 * bj + 4 * kk + g], sm.Tf[16 * bj + 4 * kk + g][16 * bj + m], X);
        f32x4 Y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) Y = mfma_f32(sm.Tf[16 * bi + m][16 * bi + 4 * g + kk], X[kk], Y);
#pragma unroll
        for (int e = 0; e < 4; ++e) sm.Tf[16 * bi + 4 * g + e][16 * bj + m] = -Y[e];
    }
    __syncthreads();
}

// The chunk's factors in LDS: A and P (masked Gram products by MFMA), then
// Tm = (I + A)^-1 by forward substitution on the 16 x 16 diagonal blocks
// (wave 0, lane = 16 b + column) and three levels of fp32 block products.
template <int MODE, int NT>
__device__ __forceinline__ void seg_prep(SegSmem& sm, int tid, int w, int lg, int lm) {
    constexpr int NWAVE = NT / 64;
    constexpr int NJOBS = (MODE == kModeOut) ? 20 : 10;
    for (int job = w; job < NJOBS; job += NWAVE) {
        const int which = job / 10, ti = job % 10;        // 0: K K^T -> A, 1: Q K^T -> P
        const int mt = (ti >= 6) ? 3 : (ti >= 3) ? 2 : (ti >= 1) ? 1 : 0;
        const int nt = ti - mt * (mt + 1) / 2;
        const uint16_t* Asrc = which ? &sm.Q[0][0] : &sm.K[0][0];
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
            acc = mfma16(lds_row8(Asrc, RP, 16 * mt + lm, kk, lg), lds_row8(&sm.K[0][0], RP, 16 * nt + lm, kk, lg), acc);
        const int cc = 16 * nt + lm;
        const float gc = sm.gam[cc];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int r = 16 * mt + 4 * lg + e;
            const float dec = (cc <= r) ? fast_exp(sm.gam[r] - gc) : 0.f;
            if (which) sm.P[r][cc] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(dec * acc[e]));
            else sm.A[r][cc] = (cc < r) ? sm.bet[r] * dec * acc[e] : 0.f;
        }
    }
    __syncthreads();
    if (w == 0) {
        const int b = lg, col = lm;
        float t[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const float* arow = &sm.A[16 * b + r][16 * b];
            float p0 = 0.f, p1 = 0.f, p2 = 0.f, p3 = 0.f;
#pragma unroll
            for (int jj = 0; jj < r; ++jj) {
                const float term = arow[jj] * t[jj];
                if ((jj & 3) == 0) p0 += term;
                else if ((jj & 3) == 1) p1 += term;
                else if ((jj & 3) == 2) p2 += term;
                else p3 += term;
            }
            t[r] = (r == col ? 1.f : 0.f) - ((p0 + p1) + (p2 + p3));
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) sm.Tf[16 * b + r][16 * b + col] = t[r];
    }
    __syncthreads();
    tsolve_level<1>(sm, w, lg, lm);
    tsolve_level<2>(sm, w, lg, lm);
    tsolve_level<3>(sm, w, lg, lm);
    // Tm (lower block triangle) to bf16; its upper blocks were zeroed once.
    for (int e = tid; e < 10 * 128; e += NT) {
        const int ti = e >> 7, ii = (e >> 3) & 15, c2 = e & 7;
        const int mt = (ti >= 6) ? 3 : (ti >= 3) ? 2 : (ti >= 1) ? 1 : 0;
        const int nt = ti - mt * (mt + 1) / 2;
        const int r = 16 * mt + ii, c = 16 * nt + 2 * c2;
        *reinterpret_cast<uint32_t*>(&sm.T[r][c]) = pack_bf16(sm.Tf[r][c], sm.Tf[r][c + 1]);
    }
    __syncthreads();
}

// One chunk of one chain for this wave's 32 value columns (cw .. cw + 31).
// ST: S^T accumulator tiles. WITH_V: values present (false for the M map).
template <bool WITH_V, bool WITH_OUT>
__device__ __forceinline__ void seg_chain(SegSmem& sm, f32x4 (&ST)[8][2], int cw, int g, int m, uint16_t* orow0,
                                          int ldv, int nc, float scale) {
    bf16x8 Sb[4][2];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) Sb[kk][nt] = pack_acc_pair(ST[2 * kk][nt], ST[2 * kk + 1][nt]);
    // beta R = beta (V - Gamma K S^T)
    f32x4 BR[4][2];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
        f32x4 z0 = {0.f, 0.f, 0.f, 0.f}, z1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            const bf16x8 a = lds_a_perm(&sm.K[0][0], RP, 16 * mt + m, kk, g);
            z0 = mfma16(a, Sb[kk][0], z0);
            z1 = mfma16(a, Sb[kk][1], z1);
        }
        const int r0 = 16 * mt + 4 * g;
        const f32x4 Gr = *reinterpret_cast<const f32x4*>(&sm.Gam[r0]);
        const f32x4 Br = *reinterpret_cast<const f32x4*>(&sm.bet[r0]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            float v0 = 0.f, v1 = 0.f;
            if (WITH_V) {
                v0 = bf16_bits_to_float(sm.V[r0 + e][cw + m]);
                v1 = bf16_bits_to_float(sm.V[r0 + e][cw + 16 + m]);
            }
            BR[mt][0][e] = Br[e] * (v0 - Gr[e] * z0[e]);
            BR[mt][1][e] = Br[e] * (v1 - Gr[e] * z1[e]);
        }
    }
    bf16x8 Bb[2][2];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) Bb[kk][nt] = pack_acc_pair(BR[2 * kk][nt], BR[2 * kk + 1][nt]);
    // U = Tm (beta R); Tm is lower triangular, so token tiles 0 and 1 need reduction step 0 only.
    f32x4 U[4][2];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
        const bf16x8 a0 = lds_a_perm(&sm.T[0][0], CP, 16 * mt + m, 0, g);
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) U[mt][nt] = mfma16(a0, Bb[0][nt], f32x4{0.f, 0.f, 0.f, 0.f});
        if (mt >= 2) {
            const bf16x8 a1 = lds_a_perm(&sm.T[0][0], CP, 16 * mt + m, 1, g);
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) U[mt][nt] = mfma16(a1, Bb[1][nt], U[mt][nt]);
        }
    }
    if (WITH_OUT) {
        // O = scale (Gamma (Q S^T) + P U), written for the rows of this chunk.
        bf16x8 Ub[2][2];
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) Ub[kk][nt] = pack_acc_pair(U[2 * kk][nt], U[2 * kk + 1][nt]);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
            f32x4 y0 = {0.f, 0.f, 0.f, 0.f}, y1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                const bf16x8 a = lds_a_perm(&sm.Q[0][0], RP, 16 * mt + m, kk, g);
                y0 = mfma16(a, Sb[kk][0], y0);
                y1 = mfma16(a, Sb[kk][1], y1);
            }
            const int r0 = 16 * mt + 4 * g;
            const f32x4 Gr = *reinterpret_cast<const f32x4*>(&sm.Gam[r0]);
            y0 = Gr * y0;
            y1 = Gr * y1;
#pragma unroll
            for (int kk = 0; kk <= (mt >> 1); ++kk) {
                const bf16x8 a = lds_a_perm(&sm.P[0][0], CP, 16 * mt + m, kk, g);
                y0 = mfma16(a, Ub[kk][0], y0);
                y1 = mfma16(a, Ub[kk][1], y1);
            }
            uint16_t* orow = orow0 + (int64_t)r0 * ldv;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                if (nc == kChunk || r0 + e < nc) {
                    orow[e * ldv] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(scale * y0[e]));
                    orow[e * ldv + 16] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(scale * y1[e]));
                }
            }
        }
    }
    // S^T = Gamma_last S^T + K^T (exp(gamma_last - gamma) U)
    bf16x8 Wb[2][2];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
        const f32x4 d0 = *reinterpret_cast<const f32x4*>(&sm.Dec[32 * kk + 4 * g]);
        const f32x4 d1 = *reinterpret_cast<const f32x4*>(&sm.Dec[32 * kk + 16 + 4 * g]);
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) Wb[kk][nt] = pack_acc_pair(d0 * U[2 * kk][nt], d1 * U[2 * kk + 1][nt]);
    }
    const float Glast = sm.Gam[kChunk - 1];
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        const bf16x8 a0 = lds_kt_tr(&sm.K[0][0], RP, t, 0, g, m);
        const bf16x8 a1 = lds_kt_tr(&sm.K[0][0], RP, t, 1, g, m);
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
            f32x4 acc = ST[t][nt] * Glast;
            acc = mfma16(a0, Wb[0][nt], acc);
            ST[t][nt] = mfma16(a1, Wb[1][nt], acc);
        }
    }
}

template <int MODE>
__global__ __launch_bounds__(MODE == kModeOut ? 256 : 512) void segment_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const float* __restrict__ g, const float* __restrict__ beta, const float* initial_state,
    const int32_t* __restrict__ cu, float* final_state, uint16_t* __restrict__ out, float* __restrict__ segws,
    int64_t total_tokens, int32_t num_seqs, int32_t num_qk_heads, int32_t num_v_heads, int32_t L, int64_t num_segs,
    float scale) {
    constexpr int NT = (MODE == kModeOut) ? 256 : 512;
    __shared__ SegSmem sm;
    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, lg = lane >> 4, lm = lane & 15;

    // XCD-aware placement: workgroups are dealt round-robin to the 8 XCDs
    // (bid % 8). The V heads of one (segment, QK head) - which read the same K
    // and Q - get consecutive slots on the XCD (segment * Hqk + QK head) % 8.
    const int group = num_v_heads / num_qk_heads;
    const int xcd = blockIdx.x & 7;
    const int64_t kx = blockIdx.x >> 3;
    const int vh = (int)(kx % group);
    const int64_t u = 8 * (kx / group) + xcd;            // (segment, QK head) unit
    if (u >= num_segs * num_qk_heads) return;
    const int64_t sg = u / num_qk_heads;
    const int hq = (int)(u % num_qk_heads);
    const int h = hq * group + vh;

    const int n = find_seq_for_seg(cu, num_seqs, sg, L);
    const SeqRange sr = seq_range(cu, n, total_tokens);
    const int64_t j = sg - seg_base(cu, n, L);
    const int64_t nch = (sr.eos - sr.bos + kChunk - 1) / kChunk;
    const int64_t nseg = nch > 0 ? (nch + L - 1) / L : 1;   // an empty sequence still copies its state
    if (j < 0 || j >= nseg) return;                          // unused segment index
    if (MODE == kModeHM && j == nseg - 1) return;            // the last segment needs no map
    const int64_t c_begin = j * L;
    const int64_t c_end = (c_begin + L < nch) ? c_begin + L : nch;
    float* segmat = segws + ((size_t)sg * num_v_heads + h) * kSegMats * kSegMat;

    // Chain of this wave: OUT: the state from its true entry value; HM: waves
    // 0-3 the H map (from the initial state in segment 0, else from 0), waves
    // 4-7 the M map (from I, without values; not needed in segment 0).
    const bool mchain = (MODE == kModeHM) && w >= 4;
    const int cw = 32 * (w & 3);
    f32x4 ST[8][2];
    const float* src = nullptr;
    if (MODE == kModeOut)
        src = (j == 0) ? (initial_state ? initial_state + ((int64_t)n * num_v_heads + h) * kSegMat : nullptr)
                       : segmat + 2 * kSegMat;
    if (MODE == kModeHM && !mchain && j == 0 && initial_state)
        src = initial_state + ((int64_t)n * num_v_heads + h) * kSegMat;
#pragma unroll
    for (int t = 0; t < 8; ++t)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
            const int col = cw + 16 * nt + lm;
            f32x4 s = {0.f, 0.f, 0.f, 0.f};
            if (mchain) {
#pragma unroll
                for (int e = 0; e < 4; ++e) s[e] = (16 * t + 4 * lg + e == col) ? 1.f : 0.f;
            } else if (src) {
                s = *reinterpret_cast<const f32x4*>(src + (int64_t)col * D + 16 * t + 4 * lg);
            }
            ST[t][nt] = s;
        }

    // Upper block triangles of Tm and P stay zero for every chunk.
    for (int e = tid; e < kChunk * kChunk; e += NT) {
        const int r = e >> 6, c = e & 63;
        if ((c >> 4) > (r >> 4)) {
            sm.T[r][c] = 0;
            sm.P[r][c] = 0;
        }
    }

    const int ldk = num_qk_heads * D, ldv = num_v_heads * D;
    SegPrefetch<NT> pf;
    auto fetch = [&](int64_t c) {
        const int64_t t0 = sr.bos + c * kChunk;
        const int nc = (int)((sr.eos - t0) < kChunk ? (sr.eos - t0) : kChunk);
        seg_fetch<MODE, NT>(pf, k + t0 * ldk + hq * D, q + t0 * ldk + hq * D, v + t0 * ldv + h * D,
                            g + t0 * num_v_heads + h, beta + t0 * num_v_heads + h, nc, ldk, ldv, num_v_heads, tid);
        return nc;
    };
    if (c_begin < c_end) {
        const int nc0 = fetch(c_begin);
        seg_stage<MODE, NT>(sm, pf, nc0, tid, w);
    }
    __syncthreads();

    for (int64_t c = c_begin; c < c_end; ++c) {
        const int64_t t0 = sr.bos + c * kChunk;
        const int nc = (int)((sr.eos - t0) < kChunk ? (sr.eos - t0) : kChunk);
        // Next chunk's operands (the last chunk re-reads itself: no branch around loads).
        const int ncn = fetch((c + 1 < c_end) ? c + 1 : c);

        seg_prep<MODE, NT>(sm, tid, w, lg, lm);
        if (MODE == kModeOut) {
            seg_chain<true, true>(sm, ST, cw, lg, lm, out + t0 * ldv + h * D + cw + lm, ldv, nc, scale);
        } else if (mchain) {
            if (j > 0) seg_chain<false, false>(sm, ST, cw, lg, lm, nullptr, ldv, nc, scale);
        } else {
            seg_chain<true, false>(sm, ST, cw, lg, lm, nullptr, ldv, nc, scale);
        }
        __syncthreads();                       // every wave is done with this chunk's operands
        seg_stage<MODE, NT>(sm, pf, ncn, tid, w);
        __syncthreads();
    }

    float* dst = nullptr;
    if (MODE == kModeOut)
        dst = (j == nseg - 1 && final_state) ? final_state + ((int64_t)n * num_v_heads + h) * kSegMat : nullptr;
    if (MODE == kModeHM) dst = mchain ? (j > 0 ? segmat + kSegMat : nullptr) : segmat;
    if (dst) {
#pragma unroll
        for (int t = 0; t < 8; ++t)
#pragma unroll
            for (int nt = 0; nt < 2; ++nt)
                *reinterpret_cast<f32x4*>(dst + (int64_t)(cw + 16 * nt + lm) * D + 16 * t + 4 * lg) = ST[t][nt];
    }
}

// Combine, fp32: for each (sequence, V head, block of 16 state rows), walk the
// sequence's segments: S_in(1) = H_0, S_in(j+1) = S_in(j) M_j + H_j; S_in(j) is
// stored for pass C. Thread t: row 16 rb + t / 16, columns 8 (t % 16) .. +7.
__global__ __launch_bounds__(256) void combine_kernel(const int32_t* __restrict__ cu, float* __restrict__ segws,
                                                      int64_t total_tokens, int32_t num_seqs, int32_t num_v_heads,
                                                      int32_t L) {
    __shared__ float Srow[16][D + 4];
    const int tid = threadIdx.x;
    const int rb = blockIdx.x & 7;
    const int h = (blockIdx.x >> 3) % num_v_heads;
    const int n = (blockIdx.x >> 3) / num_v_heads;
    const SeqRange sr = seq_range(cu, n, total_tokens);
    const int64_t nch = (sr.eos - sr.bos + kChunk - 1) / kChunk;
    const int64_t nseg = (nch + L - 1) / L;
    if (nseg < 2) return;
    const int64_t s0 = seg_base(cu, n, L);
    const int i = tid >> 4, c0 = 8 * (tid & 15);
    const int row = 16 * rb + i;
    auto mat = [&](int64_t jseg, int which) {
        return segws + (((size_t)(s0 + jseg) * num_v_heads + h) * kSegMats + which) * kSegMat;
    };
    float acc[8];
    {
        const float* H0 = mat(0, 0) + (size_t)row * D + c0;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = H0[e];
    }
    for (int64_t jj = 1; jj < nseg; ++jj) {
        float* Sin = mat(jj, 2) + (size_t)row * D + c0;
#pragma unroll
        for (int e = 0; e < 8; ++e) Sin[e] = acc[e];
        if (jj == nseg - 1) break;
        __syncthreads();
#pragma unroll
        for (int e = 0; e < 8; ++e) Srow[i][c0 + e] = acc[e];
        __syncthreads();
        const float* M = mat(jj, 1);
        const float* H = mat(jj, 0) + (size_t)row * D + c0;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = H[e];
        for (int kk = 0; kk < D; ++kk) {
            const float sv = Srow[i][kk];
            const float4 m0 = *reinterpret_cast<const float4*>(M + (size_t)kk * D + c0);
            const float4 m1 = *reinterpret_cast<const float4*>(M + (size_t)kk * D + c0 + 4);
            acc[0] = fmaf(sv, m0.x, acc[0]); acc[1] = fmaf(sv, m0.y, acc[1]);
            acc[2] = fmaf(sv, m0.z, acc[2]); acc[3] = fmaf(sv, m0.w, acc[3]);
            acc[4] = fmaf(sv, m1.x, acc[4]); acc[5] = fmaf(sv, m1.y, acc[5]);
            acc[6] = fmaf(sv, m1.z, acc[6]); acc[7] = fmaf(sv, m1.w, acc[7]);
        }
    }
}

int64_t num_segments(int64_t total_tokens, int32_t num_seqs, int L) {
    return total_tokens / ((int64_t)kChunk * L) + num_seqs;
}

}  // namespace

// Chunks per segment: enough segments for about 512 (segment, V head) workgroups.
int cp_segment_chunks(int64_t total_tokens, int32_t num_seqs, int32_t num_v_heads) {
    const int64_t chunks = total_tokens / kChunk + num_seqs;
    const int64_t want = (chunks * num_v_heads + 511) / 512;
    int L = 8;
    while (L < want && L < (1 << 24)) L <<= 1;
    return L;
}

size_t cp_segment_workspace_bytes(int64_t total_tokens, int32_t num_seqs, int32_t num_v_heads) {
    const int L = cp_segment_chunks(total_tokens, num_seqs, num_v_heads);
    return (size_t)num_segments(total_tokens, num_seqs, L) * num_v_heads * kSegMats * kSegMat * sizeof(float);
}

hipError_t launch_prefill_bf16(const PrefillArgs& a, hipStream_t stream) {
    float* seg_ws = static_cast<float*>(a.workspace);
    const int L = cp_segment_chunks(a.total_tokens, a.num_seqs, a.num_v_heads);
    const int64_t segs = num_segments(a.total_tokens, a.num_seqs, L);
    const int64_t units = segs * a.num_qk_heads;
    const int group = a.num_v_heads / a.num_qk_heads;
    const dim3 grid((unsigned)(((units + 7) / 8) * 8 * group));
    const uint16_t* q = (const uint16_t*)a.q;
    const uint16_t* k = (const uint16_t*)a.k;
    const uint16_t* v = (const uint16_t*)a.v;
    // Pass A and the combine are needed only when some sequence spans more than one segment.
    if (a.num_seqs > 1 || a.total_tokens > (int64_t)kChunk * L) {
        prof::begin(stream, "gdn_segment_maps");
        hipLaunchKernelGGL((segment_kernel<kModeHM>), grid, dim3(512), 0, stream, q, k, v, a.g, a.beta,
                           a.initial_state, a.cu_seqlens, a.final_state, (uint16_t*)a.out, seg_ws, a.total_tokens,
                           a.num_seqs, a.num_qk_heads, a.num_v_heads, L, segs, a.scale);
        prof::end(stream);
        prof::begin(stream, "gdn_segment_combine");
        hipLaunchKernelGGL(combine_kernel, dim3((unsigned)((int64_t)a.num_seqs * a.num_v_heads * 8)), dim3(256), 0,
                           stream, a.cu_seqlens, seg_ws, a.total_tokens, a.num_seqs, a.num_v_heads, L);
        prof::end(stream);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    prof::begin(stream, "gdn_segment_out");
    hipLaunchKernelGGL((segment_kernel<kModeOut>), grid, dim3(256), 0, stream, q, k, v, a.g, a.beta,
                       a.initial_state, a.cu_seqlens, a.final_state, (uint16_t*)a.out, seg_ws, a.total_tokens,
                       a.num_seqs, a.num_qk_heads, a.num_v_heads, L, segs, a.scale);
    prof::end(stream);
    return hipGetLastError();
}

size_t prefill_bf16_workspace_bytes(int64_t total_tokens, int32_t num_seqs, int32_t num_qk_heads,
                                    int32_t num_v_heads) {
    (void)num_qk_heads;
    return cp_segment_workspace_bytes(total_tokens, num_seqs, num_v_heads);
}

}  // namespace gdn
