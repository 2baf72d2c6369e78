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

// Pass 2: block (slot, V head, row block); slots outside every sequence's range exit.
// The four tokens of a sub-block share one round of cross-wave sums.
template <int D, bool BF16>
__global__ __launch_bounds__(BwdShape<D>::NT) void backward_grad_kernel(
    BwdIn in, const float* __restrict__ ck_s, const float* __restrict__ ck_ds, float* __restrict__ dq_p,
    float* __restrict__ dk_p, float* __restrict__ gb_p, float* __restrict__ dv) {
    using Sh = BwdShape<D>;
    using RB = RowBlock<D, BF16>;
    constexpr int L = Sh::L, SPLIT = Sh::SPLIT, NT = Sh::NT, WL = Sh::WL, NW = Sh::NW;
    __shared__ typename RB::Lds lds;
    __shared__ __align__(16) float red[kSub][NW][2][D];
    __shared__ __align__(16) float reds[kSub][NW][4];
    const int split = blockIdx.x % SPLIT;
    const int h = (blockIdx.x / SPLIT) % in.num_v_heads;
    const int64_t sl = blockIdx.x / (SPLIT * in.num_v_heads);
    // The sequence whose slots hold sl: the last n with ckpt_base(n) <= sl.
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
    if (j < 0 || j >= (eos - bos + kCkpt - 1) / kCkpt) return;   // a gap slot: uniform over the block
    RB rb(in, lds, h, split);
    const int tid = threadIdx.x, c = rb.c, rl = rb.rl, row = rb.row, wv = tid / 64, ln = tid % 64;
    const float scale = in.scale;
    const int64_t off = (sl * in.num_v_heads + h) * (int64_t)D * D;
    const int64_t t0 = bos + j * kCkpt, t1 = (t0 + kCkpt < eos) ? t0 + kCkpt : eos;
    const int cnt = (int)(t1 - t0);
    {
        typename RB::Fetch f;
        rb.fetch(f, t0, t1, true, true, true);
        rb.commit(f, true, true, true);
    }
    Row dS, sub[kCkpt / kSub];
    rb.load_row(ck_ds + off, dS);
    // The state at the start of every sub-block.
    {
        Row S;
        rb.load_row(ck_s + off, S);
#pragma unroll
        for (int sb = 0; sb < kCkpt / kSub; ++sb) {
            RB::copy(sub[sb], S);
            if (sb + 1 < kCkpt / kSub && kSub * (sb + 1) < cnt) {
#pragma unroll
                for (int m = 0; m < kSub; ++m) rb.step(S, kSub * sb + m);
            }
        }
    }
    // Differentiate token tt (slot m of its sub-block) with S the state before it;
    // the rows' column and scalar sums go to red[m], reds[m].
    auto grad = [&](const Row& S, int tt, int m) {
        Row kk, qq;
        rb.lds_row(lds.k, tt, kk);
        rb.lds_row(lds.q, tt, qq);
        const int64_t gb = (t0 + tt) * in.num_v_heads + h;
        const float alpha = lds.a[tt], b = lds.b[tt];
        float w0 = 0.f, w1 = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            w0 = fmaf(S[0][e], kk[0][e], w0);
            w1 = fmaf(S[1][e], kk[1][e], w1);
        }
        const float w = group_sum<L>(w0 + w1);
        const float vm = lds.v[tt][rl];
        const float u = b * (vm - alpha * w);
        const float dom = lds.dout[tt][rl];
        float d0 = 0.f, d1 = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            dS[0][e] = fmaf(scale * dom, qq[0][e], dS[0][e]);
            dS[1][e] = fmaf(scale * dom, qq[1][e], dS[1][e]);
            d0 = fmaf(dS[0][e], kk[0][e], d0);
            d1 = fmaf(dS[1][e], kk[1][e], d1);
        }
        const float du = group_sum<L>(d0 + d1);
        float s_beta = 0.f, s_dw = 0.f, s_udo = 0.f, s_dss = 0.f;
        if (c == 0) {
            dv[gb * D + row] = b * du;
            s_beta = du * (vm - alpha * w);
            s_dw = du * w;
            s_udo = u * dom;
        }
        const float ab = alpha * b;
        Row colA, colB;
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                colA[i][e] = S[i][e] * dom;
                colB[i][e] = dS[i][e] * u - ab * S[i][e] * du;
                s_dss = fmaf(dS[i][e], S[i][e], s_dss);
                dS[i][e] = alpha * dS[i][e] - ab * du * kk[i][e];
            }
        // Sums over the row groups of the wave; the lanes with c == 0 hold the rows' scalar terms.
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                colA[i][e] = rows_sum<L, WL>(colA[i][e]);
                colB[i][e] = rows_sum<L, WL>(colB[i][e]);
            }
        s_dss = group_sum<L>(s_dss);
        s_beta = rows_sum<L, WL>(s_beta);
        s_dw = rows_sum<L, WL>(s_dw);
        s_udo = rows_sum<L, WL>(s_udo);
        s_dss = rows_sum<L, WL>(s_dss);
        if (ln < L) {
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                *reinterpret_cast<f32x4*>(&red[m][wv][0][rb.col(i, 0)]) =
                    f32x4{colA[i][0], colA[i][1], colA[i][2], colA[i][3]};
                *reinterpret_cast<f32x4*>(&red[m][wv][1][rb.col(i, 0)]) =
                    f32x4{colB[i][0], colB[i][1], colB[i][2], colB[i][3]};
            }
        }
        if (ln == 0) *reinterpret_cast<f32x4*>(&reds[m][wv][0]) = f32x4{s_beta, s_dw, s_udo, s_dss};
    };
    // This block's parts of the sub-block's tokens tb .. tb + nt - 1 from the sums of
    // the waves (linear in the sums, so the parts add up).
    auto flush = [&](int tb, int nt) {
        __syncthreads();
        for (int x = tid; x < nt * 2 * D; x += NT) {
            const int m = x / (2 * D), which = (x / D) % 2, jj = x % D;
            const int tt = tb + m;
            const int64_t pb = (((t0 + tt) * in.num_v_heads + h) * SPLIT + split) * D;
            float a = 0.f;
#pragma unroll
            for (int y = 0; y < NW; ++y) a += red[m][y][which][jj];
            if (which == 0) {
                float sudo = 0.f;
#pragma unroll
                for (int y = 0; y < NW; ++y) sudo += reds[m][y][2];
                dq_p[pb + jj] = scale * fmaf(lds.a[tt], a, lds.k[tt][jj] * sudo);
            } else {
                dk_p[pb + jj] = a;
            }
        }
        if (tid < nt) {
            const int tt = tb + tid;
            float sb = 0.f, sdw = 0.f, sdss = 0.f;
#pragma unroll
            for (int y = 0; y < NW; ++y) {
                sb += reds[tid][y][0];
                sdw += reds[tid][y][1];
                sdss += reds[tid][y][3];
            }
            const int64_t gq = (((t0 + tt) * in.num_v_heads + h) * SPLIT + split) * 2;
            gb_p[gq + 0] = lds.a[tt] * (sdss - lds.b[tt] * sdw);
            gb_p[gq + 1] = sb;
        }
        __syncthreads();   // red and reds are free for the next sub-block
    };
    // Sub-blocks in reverse; inside each, its states in registers, then its tokens in reverse.
#pragma unroll
    for (int sb = kCkpt / kSub - 1; sb >= 0; --sb) {
        if (kSub * sb < cnt) {
            Row st[kSub];
            RB::copy(st[0], sub[sb]);
#pragma unroll
            for (int m = 1; m < kSub; ++m) {
                RB::copy(st[m], st[m - 1]);
                if (kSub * sb + m < cnt) rb.step(st[m], kSub * sb + m - 1);
            }
#pragma unroll
            for (int m = kSub - 1; m >= 0; --m)
                if (kSub * sb + m < cnt) grad(st[m], kSub * sb + m, m);
            flush(kSub * sb, min(kSub, cnt - kSub * sb));
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

// Pass 3, dg and dbeta: the sum of the row-block parts.
__global__ void backward_gb_sum_kernel(const float* __restrict__ part, float* __restrict__ dg,
                                       float* __restrict__ dbeta, int64_t n, int32_t split) {
    const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;   // over total_tokens * num_v_heads
    if (e >= n) return;
    float a = 0.f, b = 0.f;
    for (int x = 0; x < split; ++x) {
        a += part[(e * split + x) * 2 + 0];
        b += part[(e * split + x) * 2 + 1];
    }
    dg[e] = a;
    dbeta[e] = b;
}

static int bwd_split(int32_t d) { return d < 32 ? 1 : d / 32; }   // BwdShape<d>::SPLIT

size_t backward_workspace_bytes(int64_t total_tokens, int32_t num_seqs, int32_t num_v_heads, int32_t d) {
    const int64_t slots = total_tokens / kCkpt + num_seqs;
    const int split = bwd_split(d);
    const size_t ck = (size_t)slots * num_v_heads * d * d * sizeof(float);
    const size_t qk = (size_t)total_tokens * num_v_heads * split * d * sizeof(float);
    const size_t gbp = (size_t)total_tokens * num_v_heads * split * 2 * sizeof(float);
    return 2 * ck + 2 * qk + gbp;
}

template <int D, bool BF16>
static hipError_t launch_bwd_t(const BackwardArgs& a, hipStream_t stream) {
    using Sh = BwdShape<D>;
    static_assert(Sh::SPLIT * Sh::ROWS == D && Sh::NT <= 512 && Sh::KPT * Sh::NT == kCkpt * D, "row blocks");
    float* ws = static_cast<float*>(a.workspace);
    const int64_t slots = a.total_tokens / kCkpt + a.num_seqs;
    const size_t ck = (size_t)slots * a.num_v_heads * D * D;
    const size_t qk = (size_t)a.total_tokens * a.num_v_heads * Sh::SPLIT * D;
    float* ck_s = ws;
    float* ck_ds = ck_s + ck;
    float* dq_p = ck_ds + ck;
    float* dk_p = dq_p + qk;
    float* gb_p = dk_p + qk;
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
    hipLaunchKernelGGL((backward_grad_kernel<D, BF16>), dim3((unsigned)(slots * a.num_v_heads * Sh::SPLIT)),
                       dim3(Sh::NT), 0, stream, in, ck_s, ck_ds, dq_p, dk_p, gb_p, a.dv);
    prof::end(stream);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const int64_t nqk = a.total_tokens * a.num_qk_heads * D;
    const int64_t nv = a.total_tokens * a.num_v_heads;
    const int group = a.num_v_heads / a.num_qk_heads;
    prof::begin(stream, "gdn_backward_sums");
    hipLaunchKernelGGL(backward_qk_sum_kernel, dim3((unsigned)((nqk + 255) / 256)), dim3(256), 0, stream, dq_p, a.dq,
                       a.total_tokens, a.num_qk_heads, group, Sh::SPLIT, D);
    hipLaunchKernelGGL(backward_qk_sum_kernel, dim3((unsigned)((nqk + 255) / 256)), dim3(256), 0, stream, dk_p, a.dk,
                       a.total_tokens, a.num_qk_heads, group, Sh::SPLIT, D);
    hipLaunchKernelGGL(backward_gb_sum_kernel, dim3((unsigned)((nv + 255) / 256)), dim3(256), 0, stream, gb_p, a.dg,
                       a.dbeta, nv, Sh::SPLIT);
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
