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
// Two facts shape the kernels. The update of dS does not involve S, so the
// gradients at the interval boundaries follow from a reverse scan of their own.
// And every row i of S and dS (value index i) evolves on its own: rows meet only
// in the sums over i of dq, dk, dbeta and dalpha, which are linear in per-row
// parts. The passes:
//   1. scans, one workgroup per (sequence, V head, block of rows) and direction:
//      forward, the state at the start of every interval of 16 tokens; reverse,
//      the gradient of the state at the end of every interval (and of the
//      initial state);
//   2. one workgroup per (interval, V head, block of rows), all in parallel: the
//      interval is cut into four sub-blocks of 4 tokens; a forward sweep keeps
//      the state at each sub-block's start in registers, and each sub-block's
//      states are rebuilt from there, again in registers, before its tokens are
//      differentiated in reverse. The rows' parts of dq, dk, dg and dbeta go to
//      the workspace, dv in full;
//   3. the parts are added over row blocks (and, for dq and dk, over the V heads
//      that share a QK head) in a fixed order, so results are deterministic.
// Each row is held by d / 8 lanes, 8 key columns each, in registers; row sums
// stay in the lane group (DPP), column sums go across row groups by shuffles
// and across waves through LDS. An interval's inputs are staged in LDS once,
// with the decays exp(g) taken there.
#include "gdn_common.h"
#include "gdn_internal.h"

namespace gdn {

typedef float f32x4 __attribute__((ext_vector_type(4)));
constexpr int kCkpt = 16;   // tokens per checkpoint interval
constexpr int kSub = 4;     // tokens per sub-block of an interval

template <int D>
struct BwdShape {
    static constexpr int L = D / 8;                  // lanes per state row (8 columns each)
    static constexpr int ROWS = D < 32 ? D : 32;     // state rows per workgroup
    static constexpr int SPLIT = D / ROWS;           // row blocks per (sequence, V head)
    static constexpr int NT = ROWS * L;              // threads: one row per lane group
    static constexpr int WL = NT < 64 ? NT : 64;     // lanes per wave in use
    static constexpr int NW = (NT + 63) / 64;        // waves
    static constexpr int KPT = kCkpt * D / NT;       // staged k (or q) elements per thread
    static constexpr int VPT = (kCkpt * ROWS + NT - 1) / NT;   // staged v (or do) elements per thread
};

// Slot of interval j of sequence n among the checkpoints: cu[n] / 16 + n + j.
// The ranges of different sequences are disjoint and below T / 16 + N.
__device__ __forceinline__ int64_t ckpt_base(const int32_t* cu, int n) {
    return cu ? (int64_t)(cu[n] / kCkpt) + n : 0;
}

struct BwdIn {
    const void *q, *k, *v, *dout;
    const float *g, *beta;
    const int32_t* cu;
    int64_t total_tokens;
    int32_t num_seqs, num_qk_heads, num_v_heads;
    float scale;
};

typedef float Row[2][4];   // a lane's 8 columns of one state row

// x[lane] + x[lane ^ 16] and x[lane] + x[lane ^ 32]: each swap instruction
// exchanges half of one register with half of the other, so with both operands
// holding x the two results are the lane's own value and its partner's.
__device__ __forceinline__ float swap16_sum(float x) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float swap32_sum(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// Sum over the lanes of a wave's first WL lanes that share lane % L.
template <int L, int WL>
__device__ __forceinline__ float rows_sum(float x) {
#pragma unroll
    for (int mask = L; mask < WL; mask *= 2) {
        if (mask == 16) x = swap16_sum(x);
        else if (mask == 32) x = swap32_sum(x);
        else x += __shfl_xor(x, mask);
    }
    return x;
}

// Per-workgroup view: a row block of one (sequence, V head), its interval staging
// in LDS and the per-row arithmetic shared by the passes.
template <int D, bool BF16>
struct RowBlock {
    using Sh = BwdShape<D>;
    static constexpr int L = Sh::L, ROWS = Sh::ROWS, NT = Sh::NT, KPT = Sh::KPT, VPT = Sh::VPT;
    struct alignas(16) Lds {
        float k[kCkpt][D], q[kCkpt][D];
        float v[kCkpt][ROWS], dout[kCkpt][ROWS];   // this block's rows only
        float a[kCkpt], b[kCkpt];                  // exp(g), beta
    };
    // One interval's inputs on their way from HBM to LDS.
    struct Fetch {
        float k[KPT], q[KPT], v[VPT], dout[VPT], g, b;
    };
    const BwdIn& in;
    Lds& s;
    int tid, c, rl, row, h, hq, split;

    __device__ RowBlock(const BwdIn& in_, Lds& s_, int h_, int split_) : in(in_), s(s_), h(h_), split(split_) {
        tid = threadIdx.x;
        c = tid % L;
        rl = tid / L;
        row = split * ROWS + rl;
        hq = h / (in.num_v_heads / in.num_qk_heads);
    }
    __device__ __forceinline__ int col(int i, int e) const { return 4 * (c + L * i) + e; }
    __device__ __forceinline__ float ld(const void* p, int64_t idx) const {
        if constexpr (BF16) return bf16_bits_to_float(reinterpret_cast<const uint16_t*>(p)[idx]);
        else return reinterpret_cast<const float*>(p)[idx];
    }
    // Global loads of tokens t0 .. t1 - 1 (1 to 16 of them) into registers. Slots
    // past t1 load token t1 - 1 again (no branch around the loads); they are
    // never read.
    __device__ __forceinline__ void fetch(Fetch& f, int64_t t0, int64_t t1, bool want_q, bool want_v,
                                          bool want_do) const {
        const int last = (int)(t1 - t0) - 1;
        const int hqk = in.num_qk_heads, hv = in.num_v_heads;
#pragma unroll
        for (int r = 0; r < KPT; ++r) {
            const int e = tid + r * NT, tt = min(e / D, last), jj = e % D;
            const int64_t idx = ((t0 + tt) * hqk + hq) * D + jj;
            f.k[r] = ld(in.k, idx);
            if (want_q) f.q[r] = ld(in.q, idx);
        }
#pragma unroll
        for (int r = 0; r < VPT; ++r) {
            const int e = min(tid + r * NT, kCkpt * ROWS - 1), tt = min(e / ROWS, last), rr = e % ROWS;
            const int64_t idx = ((t0 + tt) * hv + h) * D + split * ROWS + rr;
            if (want_v) f.v[r] = ld(in.v, idx);
            if (want_do) f.dout[r] = ld(in.dout, idx);
        }
        const int64_t gi = (t0 + min(tid, last)) * hv + h;
        f.g = in.g[gi];
        f.b = in.beta[gi];
    }
    // Fetched registers into LDS, after every thread has finished with the
    // previous contents.
    __device__ __forceinline__ void commit(const Fetch& f, bool want_q, bool want_v, bool want_do) {
        __syncthreads();
#pragma unroll
        for (int r = 0; r < KPT; ++r) {
            const int e = tid + r * NT;
            s.k[e / D][e % D] = f.k[r];
            if (want_q) s.q[e / D][e % D] = f.q[r];
        }
#pragma unroll
        for (int r = 0; r < VPT; ++r) {
            const int e = tid + r * NT;
            if (e < kCkpt * ROWS) {
                if (want_v) s.v[e / ROWS][e % ROWS] = f.v[r];
                if (want_do) s.dout[e / ROWS][e % ROWS] = f.dout[r];
            }
        }
        if (tid < kCkpt) {
            s.a[tid] = exp_nonpos(f.g);
            s.b[tid] = f.b;
        }
        __syncthreads();
    }
    __device__ __forceinline__ void lds_row(const float (*X)[D], int tt, Row& x) const {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const f32x4 y = *reinterpret_cast<const f32x4*>(&X[tt][col(i, 0)]);
#pragma unroll
            for (int e = 0; e < 4; ++e) x[i][e] = y[e];
        }
    }
    __device__ __forceinline__ void load_row(const float* src, Row& x) const {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const f32x4 y = src ? *reinterpret_cast<const f32x4*>(src + row * D + col(i, 0)) : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int e = 0; e < 4; ++e) x[i][e] = y[e];
        }
    }
    __device__ __forceinline__ void store_row(float* dst, const Row& x) const {
#pragma unroll
        for (int i = 0; i < 2; ++i)
            *reinterpret_cast<f32x4*>(dst + row * D + col(i, 0)) = f32x4{x[i][0], x[i][1], x[i][2], x[i][3]};
    }
    __device__ __forceinline__ static void copy(Row& d, const Row& x) {
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int e = 0; e < 4; ++e) d[i][e] = x[i][e];
    }
    // One forward step of this row of S for staged token tt.
    __device__ __forceinline__ void step(Row& S, int tt) const {
        Row kk;
        lds_row(s.k, tt, kk);
        const float alpha = s.a[tt], b = s.b[tt];
        float w0 = 0.f, w1 = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            w0 = fmaf(S[0][e], kk[0][e], w0);
            w1 = fmaf(S[1][e], kk[1][e], w1);
        }
        const float w = group_sum<L>(w0 + w1);
        const float u = b * (s.v[tt][rl] - alpha * w);
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int e = 0; e < 4; ++e) S[i][e] = fmaf(alpha, S[i][e], u * kk[i][e]);
    }
    // One reverse step of this row of dS for staged token tt (read-out, then the
    // gradient of the state before the token).
    __device__ __forceinline__ void rstep(Row& dS, int tt) const {
        Row kk, qq;
        lds_row(s.k, tt, kk);
        lds_row(s.q, tt, qq);
        const float alpha = s.a[tt], b = s.b[tt];
        const float sd = in.scale * s.dout[tt][rl];
        float d0 = 0.f, d1 = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            dS[0][e] = fmaf(sd, qq[0][e], dS[0][e]);
            dS[1][e] = fmaf(sd, qq[1][e], dS[1][e]);
            d0 = fmaf(dS[0][e], kk[0][e], d0);
            d1 = fmaf(dS[1][e], kk[1][e], d1);
        }
        const float du = group_sum<L>(d0 + d1);
        const float ab = alpha * b;
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int e = 0; e < 4; ++e) dS[i][e] = alpha * dS[i][e] - ab * du * kk[i][e];
    }
};

// Pass 1: blocks [0, P) scan forward and store the state rows at the start of each
// interval; blocks [P, 2P) scan in reverse and store the gradient rows at the end
// of each interval, then the gradient of the initial state. P = N * Hv * SPLIT.
// The next interval's inputs are fetched while the current one is processed.
template <int D, bool BF16>
__global__ __launch_bounds__(BwdShape<D>::NT) void backward_scan_kernel(
    BwdIn in, const float* __restrict__ initial_state, const float* __restrict__ dfinal,
    float* __restrict__ dinit, float* __restrict__ ck_s, float* __restrict__ ck_ds) {
    using Sh = BwdShape<D>;
    using RB = RowBlock<D, BF16>;
    __shared__ typename RB::Lds lds;
    const int64_t P = (int64_t)in.num_seqs * in.num_v_heads * Sh::SPLIT;
    const bool rev = blockIdx.x >= P;
    const int64_t b = rev ? blockIdx.x - P : blockIdx.x;
    const int split = (int)(b % Sh::SPLIT);
    const int nh = (int)(b / Sh::SPLIT);
    const int n = nh / in.num_v_heads, h = nh % in.num_v_heads;
    RB rb(in, lds, h, split);
    const int64_t bos = in.cu ? (int64_t)in.cu[n] : 0, eos = in.cu ? (int64_t)in.cu[n + 1] : in.total_tokens;
    const int64_t sbase = ((int64_t)n * in.num_v_heads + h) * D * D;
    const int64_t cbase = ckpt_base(in.cu, n);
    const int64_t nint = (eos - bos + kCkpt - 1) / kCkpt;
    auto slot = [&](float* base, int64_t j) { return base + ((cbase + j) * in.num_v_heads + h) * (int64_t)D * D; };
    auto span = [&](int64_t j, int64_t& t0, int64_t& t1) {
        t0 = bos + j * kCkpt;
        t1 = (t0 + kCkpt < eos) ? t0 + kCkpt : eos;
    };
    Row X;
    typename RB::Fetch f;
    int64_t t0, t1;
    if (!rev) {
        rb.load_row(initial_state ? initial_state + sbase : nullptr, X);
        if (nint > 0) {
            span(0, t0, t1);
            rb.fetch(f, t0, t1, false, true, false);
        }
        for (int64_t j = 0; j < nint; ++j) {
            rb.store_row(slot(ck_s, j), X);
            span(j, t0, t1);
            rb.commit(f, false, true, false);
            if (j + 1 < nint) {
                int64_t u0, u1;
                span(j + 1, u0, u1);
                rb.fetch(f, u0, u1, false, true, false);
            }
            const int cnt = (int)(t1 - t0);
            if (cnt == kCkpt) {
#pragma unroll
                for (int tt = 0; tt < kCkpt; ++tt) rb.step(X, tt);
            } else {
                for (int tt = 0; tt < cnt; ++tt) rb.step(X, tt);
            }
        }
    } else {
        rb.load_row(dfinal ? dfinal + sbase : nullptr, X);
        if (nint > 0) {
            span(nint - 1, t0, t1);
            rb.fetch(f, t0, t1, true, false, true);
        }
        for (int64_t j = nint - 1; j >= 0; --j) {
            rb.store_row(slot(ck_ds, j), X);
            span(j, t0, t1);
            rb.commit(f, true, false, true);
            if (j > 0) {
                int64_t u0, u1;
                span(j - 1, u0, u1);
                rb.fetch(f, u0, u1, true, false, true);
            }
            const int cnt = (int)(t1 - t0);
            if (cnt == kCkpt) {
#pragma unroll
                for (int tt = kCkpt - 1; tt >= 0; --tt) rb.rstep(X, tt);
            } else {
                for (int tt = cnt - 1; tt >= 0; --tt) rb.rstep(X, tt);
            }
        }
        if (dinit) rb.store_row(dinit + sbase, X);
    }
}

// Pass 2, one workgroup (4 waves) per (interval, V head): the interval as a
// chunk of 16 tokens (padded with g = 0, beta = 0 and zero inputs, which are
// identity steps), entry state S0 and end gradient G from the scans. With
// gamma the in-chunk cumulative sum of g, Gam = exp(gamma), Gp = exp(gamma_last
// - gamma), dec[r][c] = exp(gamma_r - gamma_c), At = dec (K K^T) strictly below
// the diagonal, A = diag(beta) At, P = dec (Q K^T) on and below it and
// T = (I + A)^-1, the token rule unrolls to (rows are tokens):
//   U  = T diag(beta) (V - diag(Gam) K S0^T)       AW = diag(Gam) K S0^T + At U
//   dU = T^T (diag(Gp) K G^T + scale P^T dO)       (du_t = E_t k_t, E_t the state gradient)
//   dv = diag(beta) dU,   dbeta_t = du_t . (v_t - AW_t)
//   dQ = scale (diag(Gam) dO S0 + M4 K),           M4 = [tau <= t] dec (dO U^T)
//   dK = diag(Gp) U G - diag(beta Gam) dU S0 + scale M4^T Q - M5 K,
//        M5[t][s] = [s > t] dec[s][t] beta_s (dU U^T)[s][t] + [s < t] beta_t dec[t][s] (dU U^T)[t][s]
//   dg_t = exp(gamma_last) <G, S0> + sum_{tau < t} a_tau + sum_{s >= t} b_s - sum_{s > t} c_s
//          + sum_{s >= t, tau < t} scale P[s][tau] (dO U^T)[s][tau]
//          - sum_{s > t, tau < t} A[s][tau] (dU U^T)[s][tau] - beta_t du_t . AW_t,
//   a = Gp (U G . K), b = scale Gam (dO S0 . Q), c = Gam beta (dU S0 . K) (row dots).
// Products over the value index (U G, dO S0, dU S0, dO U^T, dU U^T, <G, S0>) run
// over blocks of 32 state rows staged in LDS and accumulate in registers. All
// products are fp32 MFMA 16x16x4 (lane (g, m): A[m][k], B[k][m], D[4 g + e][m];
// any fixed order of k serves, so long contractions take k = g (K / 4) + kk).
template <int D>
struct ChunkShape {
    static constexpr int R = D < 32 ? D : 32;   // state rows per block
    static constexpr int NB = D / R;            // blocks
    static constexpr int KP = D + 4;            // fp32 row pitch of d-wide rows
    static constexpr int BP = R + 4;            // fp32 row pitch of block-wide rows
    static constexpr int NTD = D / 16;          // 16-column tiles over d
    static constexpr int NTR = R / 16;          // 16-column tiles over a block
    static constexpr int TPW = (NTD + 3) / 4;   // d tiles per wave
};

__device__ __forceinline__ f32x4 mfma4(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

template <int D, bool BF16>
__global__ __launch_bounds__(256) void backward_grad_kernel(
    BwdIn in, const float* __restrict__ ck_s, const float* __restrict__ ck_ds, float* __restrict__ dq_h,
    float* __restrict__ dk_h, float* __restrict__ dg, float* __restrict__ dbeta, float* __restrict__ dv) {
    using CS = ChunkShape<D>;
    constexpr int C = kCkpt, R = CS::R, NB = CS::NB, KP = CS::KP, BP = CS::BP, NTD = CS::NTD, NTR = CS::NTR,
                  TPW = CS::TPW;
    constexpr int SP = C + 1;   // pitch of the 16 x 16 matrices
    static_assert(C == 16 && R % 16 == 0, "chunk of 16 tokens, blocks of whole tiles");
    __shared__ __align__(16) float Kf[C][KP], Qf[C][KP];
    __shared__ __align__(16) float Sb[R][KP], Gb[R][KP];
    __shared__ float Vb[C][BP], dOb[C][BP], KSs[C][BP], KGs[C][BP], Us[C][BP], dUs[C][BP], Rs[C][BP];
    __shared__ float At[C][SP], Pm[C][SP], Tm[C][SP], KK[C][SP], QK[C][SP], M4[C][SP], M5[C][SP], dOU[C][SP],
        DUm[C][SP];
    __shared__ float gin[C], gam[C], Gam[C], Gp[C], bet[C], part[4][3][C], red[4], dgs[C];

    const int h = blockIdx.x % in.num_v_heads;
    const int64_t sl = blockIdx.x / in.num_v_heads;
    int n = 0;
    if (in.cu) {
        int lo = 0, hi = in.num_seqs - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) / 2;
            if (ckpt_base(in.cu, mid) <= sl) lo = mid;
            else hi = mid - 1;
        }
        n = lo;
    }
    const int64_t bos = in.cu ? (int64_t)in.cu[n] : 0, eos = in.cu ? (int64_t)in.cu[n + 1] : in.total_tokens;
    const int64_t j = sl - ckpt_base(in.cu, n);
    if (j < 0 || j >= (eos - bos + C - 1) / C) return;   // a gap slot: uniform over the block
    const int64_t t0 = bos + j * C;
    const int cnt = (int)min((int64_t)C, eos - t0);
    const int tid = threadIdx.x, w = tid / 64, ln = tid % 64, g4 = ln / 16, m = ln % 16;
    const int hv = in.num_v_heads, hqk = in.num_qk_heads, hq = h / (hv / hqk);
    const float scale = in.scale;
    const int64_t off = (sl * hv + h) * (int64_t)D * D;
    auto ld = [&](const void* p, int64_t idx) -> float {
        if constexpr (BF16) return bf16_bits_to_float(reinterpret_cast<const uint16_t*>(p)[idx]);
        else return reinterpret_cast<const float*>(p)[idx];
    };
    const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};

    // Stage K, Q (rows past cnt are zero), g and beta.
    for (int e = tid; e < C * D; e += 256) {
        const int t = e / D, c = e % D;
        const int64_t idx = ((t0 + min(t, cnt - 1)) * hqk + hq) * D + c;
        const float keep = t < cnt ? 1.f : 0.f;
        Kf[t][c] = keep * ld(in.k, idx);
        Qf[t][c] = keep * ld(in.q, idx);
    }
    if (tid < C) {
        const int64_t gi = (t0 + min(tid, cnt - 1)) * hv + h;
        const float keep = tid < cnt ? 1.f : 0.f;
        gin[tid] = keep * in.g[gi];
        bet[tid] = keep * in.beta[gi];
    }
    __syncthreads();
    // Decays (wave 0) and the Gram matrices K K^T (wave 1), Q K^T (wave 2).
    if (w == 0) {
        if (ln < C) {
            float s = 0.f, tot = 0.f;
            for (int t = 0; t < C; ++t) {
                tot += gin[t];
                if (t == ln) s = tot;
            }
            gam[ln] = s;
            Gam[ln] = exp_nonpos(s);
            Gp[ln] = exp_nonpos(tot - s);
        }
    } else if (w <= 2) {
        const float (*X)[KP] = w == 1 ? Kf : Qf;
        f32x4 acc = zero4;
        for (int kk = 0; kk < D / 4; ++kk) {
            const int k = g4 * (D / 4) + kk;
            acc = mfma4(X[m][k], Kf[m][k], acc);
        }
        float (*dst)[SP] = w == 1 ? KK : QK;
#pragma unroll
        for (int e = 0; e < 4; ++e) dst[4 * g4 + e][m] = acc[e];
    }
    __syncthreads();
    // At, P and T = (I + diag(beta) At)^-1 (wave 0; lane c solves column c).
    if (w == 0 && ln < C) {
        const int c = ln;
        for (int r = 0; r < C; ++r) {
            const float dr = gam[r] - gam[c];
            At[r][c] = c < r ? exp_nonpos(dr) * KK[r][c] : 0.f;
            Pm[r][c] = c <= r ? exp_nonpos(dr) * QK[r][c] : 0.f;
        }
        float Tc[C];
#pragma unroll
        for (int r = 0; r < C; ++r) {
            float s = r == c ? 1.f : 0.f;
            const float br = bet[r];
#pragma unroll
            for (int p = 0; p < r; ++p) s = fmaf(-br * At[r][p], Tc[p], s);
            Tc[r] = s;
        }
#pragma unroll
        for (int r = 0; r < C; ++r) Tm[r][c] = Tc[r];
    }
    // Accumulators over the blocks: U G, dO S0, dU S0 for this wave's d tiles; dO U^T
    // (wave 2) and dU U^T (wave 3); row sums for dbeta and du . AW; <G, S0>.
    f32x4 accUG[TPW], accOS[TPW], accUS[TPW], accM = zero4;
#pragma unroll
    for (int i = 0; i < TPW; ++i) accUG[i] = accOS[i] = accUS[i] = zero4;
    float p_db = 0.f, p_dw = 0.f, p_gs = 0.f;
    const int vt = tid / 16, vp = tid % 16;   // token and column phase for the row sums

    for (int rb = 0; rb < NB; ++rb) {
        __syncthreads();   // the previous block's LDS reads are done (and T is written)
        // Stage this block's rows of S0 and G, and its columns of V and dO.
        {
            const float* s0 = ck_s + off + (int64_t)rb * R * D;
            const float* gg = ck_ds + off + (int64_t)rb * R * D;
            for (int e = 4 * tid; e < R * D; e += 4 * 256) {
                const int r = e / D, c = e % D;
                *reinterpret_cast<f32x4*>(&Sb[r][c]) = *reinterpret_cast<const f32x4*>(s0 + e);
                *reinterpret_cast<f32x4*>(&Gb[r][c]) = *reinterpret_cast<const f32x4*>(gg + e);
            }
            for (int e = tid; e < C * R; e += 256) {
                const int t = e / R, c = e % R;
                const int64_t idx = ((t0 + min(t, cnt - 1)) * hv + h) * D + rb * R + c;
                const float keep = t < cnt ? 1.f : 0.f;
                Vb[t][c] = keep * ld(in.v, idx);
                dOb[t][c] = keep * ld(in.dout, idx);
            }
        }
        __syncthreads();
        // K S0^T and K G^T for the block's columns: 2 NTR tiles.
        for (int tile = w; tile < 2 * NTR; tile += 4) {
            const float (*B)[KP] = tile < NTR ? Sb : Gb;
            const int nt = tile % NTR;
            f32x4 acc = zero4;
            for (int kk = 0; kk < D / 4; ++kk) {
                const int k = g4 * (D / 4) + kk;
                acc = mfma4(Kf[m][k], B[16 * nt + m][k], acc);
            }
            float (*dst)[BP] = tile < NTR ? KSs : KGs;
#pragma unroll
            for (int e = 0; e < 4; ++e) dst[4 * g4 + e][16 * nt + m] = acc[e];
        }
        __syncthreads();
        // U (waves 0 .. NTR - 1) and Z = P^T dO (waves 2 .. 2 + NTR - 1).
        if (w < NTR) {
            const int c = 16 * w + m;
            f32x4 acc = zero4;
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                const int k = 4 * kk + g4;
                acc = mfma4(Tm[m][k], bet[k] * (Vb[k][c] - Gam[k] * KSs[k][c]), acc);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) Us[4 * g4 + e][c] = acc[e];
        } else if (w >= 2 && w < 2 + NTR) {
            const int c = 16 * (w - 2) + m;
            f32x4 acc = zero4;
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                const int k = 4 * kk + g4;
                acc = mfma4(Pm[k][m], dOb[k][c], acc);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int t = 4 * g4 + e;
                KGs[t][c] = fmaf(Gp[t], KGs[t][c], scale * acc[e]);   // Y = Gp K G^T + scale P^T dO
            }
        }
        __syncthreads();
        // AW = Gam K S0^T + At U, R = V - AW (waves 0 ..); dU = T^T Y (waves 2 ..).
        if (w < NTR) {
            const int c = 16 * w + m;
            f32x4 acc = zero4;
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                const int k = 4 * kk + g4;
                acc = mfma4(At[m][k], Us[k][c], acc);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int t = 4 * g4 + e;
                Rs[t][c] = Vb[t][c] - fmaf(Gam[t], KSs[t][c], acc[e]);
            }
        } else if (w >= 2 && w < 2 + NTR) {
            const int c = 16 * (w - 2) + m;
            f32x4 acc = zero4;
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                const int k = 4 * kk + g4;
                acc = mfma4(Tm[k][m], KGs[k][c], acc);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) dUs[4 * g4 + e][c] = acc[e];
        }
        __syncthreads();
        // dv, the row sums and <G, S0> on the block.
        for (int c = vp; c < R; c += 16) {
            const float du = dUs[vt][c], r = Rs[vt][c];
            p_db = fmaf(du, r, p_db);
            p_dw = fmaf(du, Vb[vt][c] - r, p_dw);
            if (vt < cnt) dv[((t0 + vt) * hv + h) * D + rb * R + c] = bet[vt] * du;
        }
        for (int e = tid; e < R * D; e += 256) p_gs = fmaf(Gb[e / D][e % D], Sb[e / D][e % D], p_gs);
        // U G, dO S0, dU S0 on this wave's d tiles (k: the block's rows).
#pragma unroll
        for (int i = 0; i < TPW; ++i) {
            const int nt = w + 4 * i;
            if (nt < NTD) {
#pragma unroll
                for (int kk = 0; kk < R / 4; ++kk) {
                    const int k = 4 * kk + g4;
                    const float sb = Sb[k][16 * nt + m];
                    accUG[i] = mfma4(Us[m][k], Gb[k][16 * nt + m], accUG[i]);
                    accOS[i] = mfma4(dOb[m][k], sb, accOS[i]);
                    accUS[i] = mfma4(dUs[m][k], sb, accUS[i]);
                }
            }
        }
        if (w >= 2) {   // dO U^T (wave 2), dU U^T (wave 3)
            const float (*X)[BP] = w == 2 ? dOb : dUs;
#pragma unroll
            for (int kk = 0; kk < R / 4; ++kk) {
                const int k = 4 * kk + g4;
                accM = mfma4(X[m][k], Us[m][k], accM);
            }
        }
    }
    // dO U^T and dU U^T to LDS; the row dots a, b, c of this wave's d tiles.
    if (w >= 2) {
        float (*dst)[SP] = w == 2 ? dOU : DUm;
#pragma unroll
        for (int e = 0; e < 4; ++e) dst[4 * g4 + e][m] = accM[e];
    }
    {
        float pa[4] = {0.f, 0.f, 0.f, 0.f}, pbq[4] = {0.f, 0.f, 0.f, 0.f}, pc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < TPW; ++i) {
            const int nt = w + 4 * i;
            if (nt < NTD) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int t = 4 * g4 + e, col = 16 * nt + m;
                    pa[e] = fmaf(accUG[i][e], Kf[t][col], pa[e]);
                    pbq[e] = fmaf(accOS[i][e], Qf[t][col], pbq[e]);
                    pc[e] = fmaf(accUS[i][e], Kf[t][col], pc[e]);
                }
            }
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            pa[e] = group_sum<16>(pa[e]);
            pbq[e] = group_sum<16>(pbq[e]);
            pc[e] = group_sum<16>(pc[e]);
        }
        if (m == 0) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                part[w][0][4 * g4 + e] = pa[e];
                part[w][1][4 * g4 + e] = pbq[e];
                part[w][2][4 * g4 + e] = pc[e];
            }
        }
    }
    // Row sums of dbeta and du . AW per token (16 lanes per token), <G, S0> over the block.
    p_db = group_sum<16>(p_db);
    p_dw = group_sum<16>(p_dw);
    p_gs = group_sum<16>(p_gs);
    p_gs = swap16_sum(p_gs);
    p_gs = swap32_sum(p_gs);
    if (ln == 0) red[w] = p_gs;
    __syncthreads();
    // M4 and M5 (wave 0, lane t builds row t); dg and dbeta (wave 1, lane t).
    if (w == 0 && ln < C) {
        const int t = ln;
        const float bt = bet[t];
        for (int s = 0; s < C; ++s) {
            const float dts = gam[t] - gam[s];
            M4[t][s] = s <= t ? exp_nonpos(dts) * dOU[t][s] : 0.f;
            float m5 = 0.f;
            if (s > t) m5 = exp_nonpos(-dts) * bet[s] * DUm[s][t];
            if (s < t) m5 = bt * exp_nonpos(dts) * DUm[t][s];
            M5[t][s] = m5;
        }
    }
    if (w == 1 && ln < C) {
        const int t = ln;
        const float gs = red[0] + red[1] + red[2] + red[3];
        float a_excl = 0.f, b_incl = 0.f, c_excl = 0.f, rect = 0.f;
        for (int s = 0; s < C; ++s) {
            const float a = Gp[s] * (part[0][0][s] + part[1][0][s] + part[2][0][s] + part[3][0][s]);
            const float b = scale * Gam[s] * (part[0][1][s] + part[1][1][s] + part[2][1][s] + part[3][1][s]);
            const float cc = Gam[s] * bet[s] * (part[0][2][s] + part[1][2][s] + part[2][2][s] + part[3][2][s]);
            if (s < t) a_excl += a;
            if (s >= t) b_incl += b;
            if (s > t) c_excl += cc;
            if (s >= t) {
                for (int tau = 0; tau < t; ++tau) {
                    float x = scale * Pm[s][tau] * dOU[s][tau];
                    if (s > t) x -= bet[s] * At[s][tau] * DUm[s][tau];
                    rect += x;
                }
            }
        }
        dgs[t] = exp_nonpos(gam[C - 1]) * gs + a_excl + b_incl - c_excl + rect;
    }
    __syncthreads();
    // Each token's 16-lane group holds its dbeta and du . AW sums.
    if (vp == 0 && vt < cnt) {
        const int64_t gi = (t0 + vt) * hv + h;
        dbeta[gi] = p_db;
        dg[gi] = dgs[vt] - bet[vt] * p_dw;
    }
    // dQ and dK on this wave's d tiles.
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
        const int nt = w + 4 * i;
        if (nt < NTD) {
            const int col = 16 * nt + m;
            f32x4 q_, k_;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int t = 4 * g4 + e;
                q_[e] = Gam[t] * accOS[i][e];
                k_[e] = Gp[t] * accUG[i][e] - bet[t] * Gam[t] * accUS[i][e];
            }
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                const int k = 4 * kk + g4;
                q_ = mfma4(M4[m][k], Kf[k][col], q_);
                k_ = mfma4(scale * M4[k][m], Qf[k][col], k_);
                k_ = mfma4(-M5[m][k], Kf[k][col], k_);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int t = 4 * g4 + e;
                if (t < cnt) {
                    const int64_t gi = ((t0 + t) * hv + h) * D + col;
                    dq_h[gi] = scale * q_[e];
                    dk_h[gi] = k_[e];
                }
            }
        }
    }
}

// Pass 3, dq and dk of a QK head: the sum of the row-block parts of its V heads.
__global__ void backward_qk_sum_kernel(const float* __restrict__ part, float* __restrict__ dst, int64_t rows,
                                       int32_t num_qk_heads, int32_t group, int32_t split, int32_t d) {
    const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;   // over rows * num_qk_heads * d
    if (e >= rows * num_qk_heads * d) return;
    const int64_t t = e / ((int64_t)num_qk_heads * d);
    const int64_t r = e % ((int64_t)num_qk_heads * d);
    const int hq = (int)(r / d), j = (int)(r % d);
    const float* p = part + ((t * num_qk_heads + hq) * group) * (int64_t)split * d + j;
    float s = 0.f;
    for (int x = 0; x < group * split; ++x) s += p[(int64_t)x * d];
    dst[e] = s;
}

size_t backward_workspace_bytes(int64_t total_tokens, int32_t num_seqs, int32_t num_v_heads, int32_t d) {
    const int64_t slots = total_tokens / kCkpt + num_seqs;
    const size_t ck = (size_t)slots * num_v_heads * d * d * sizeof(float);   // one checkpoint array
    const size_t qk = (size_t)total_tokens * num_v_heads * d * sizeof(float);  // dq or dk per V head
    return 2 * ck + 2 * qk;
}

template <int D, bool BF16>
static hipError_t launch_bwd_t(const BackwardArgs& a, hipStream_t stream) {
    using Sh = BwdShape<D>;
    static_assert(Sh::SPLIT * Sh::ROWS == D && Sh::NT <= 512 && Sh::KPT * Sh::NT == kCkpt * D, "row blocks");
    float* ws = static_cast<float*>(a.workspace);
    const int64_t slots = a.total_tokens / kCkpt + a.num_seqs;
    const size_t ck = (size_t)slots * a.num_v_heads * D * D;
    const size_t qk = (size_t)a.total_tokens * a.num_v_heads * D;
    float* ck_s = ws;
    float* ck_ds = ck_s + ck;
    float* dq_h = ck_ds + ck;
    float* dk_h = dq_h + qk;
    const BwdIn in{a.q, a.k, a.v, a.d_out, a.g, a.beta, a.cu_seqlens, a.total_tokens,
                   a.num_seqs, a.num_qk_heads, a.num_v_heads, a.scale};
    const int64_t P = (int64_t)a.num_seqs * a.num_v_heads * Sh::SPLIT;
    prof::begin(stream, "gdn_backward_scan");
    hipLaunchKernelGGL((backward_scan_kernel<D, BF16>), dim3((unsigned)(2 * P)), dim3(Sh::NT), 0, stream, in,
                       a.initial_state, a.d_final_state, a.d_initial_state, ck_s, ck_ds);
    prof::end(stream);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.total_tokens == 0) return e;
    prof::begin(stream, "gdn_backward_grad");
    hipLaunchKernelGGL((backward_grad_kernel<D, BF16>), dim3((unsigned)(slots * a.num_v_heads)), dim3(256), 0,
                       stream, in, ck_s, ck_ds, dq_h, dk_h, a.dg, a.dbeta, a.dv);
    prof::end(stream);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const int64_t nqk = a.total_tokens * a.num_qk_heads * D;
    const int group = a.num_v_heads / a.num_qk_heads;
    prof::begin(stream, "gdn_backward_sums");
    hipLaunchKernelGGL(backward_qk_sum_kernel, dim3((unsigned)((nqk + 255) / 256)), dim3(256), 0, stream, dq_h, a.dq,
                       a.total_tokens, a.num_qk_heads, group, 1, D);
    hipLaunchKernelGGL(backward_qk_sum_kernel, dim3((unsigned)((nqk + 255) / 256)), dim3(256), 0, stream, dk_h, a.dk,
                       a.total_tokens, a.num_qk_heads, group, 1, D);
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
