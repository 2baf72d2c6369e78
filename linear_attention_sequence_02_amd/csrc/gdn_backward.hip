// Gradients of the Gated DeltaNet recurrence in fp32, by chunks of 16 tokens.
//
// Forward rule per (sequence, V head), token t (alpha = exp(g), w = S k):
//     u = beta (v - alpha w)        S_t = alpha S + u k^T        o = scale S_t q
// Reverse, with E_t the gradient of S_t (every later token's contribution and
// the read-out at t included) and S the state before token t:
//     du = E_t k,  dv = beta du,  dbeta = du . (v - alpha w),  dg = alpha <E_t, S> - beta du . (alpha w)
//     dk = E_t^T u - alpha beta S^T du,  dq = scale S_t^T do,
//     E_{t-1} = alpha E_t - alpha beta du k^T + scale do_{t-1} q_{t-1}^T.
// Over a chunk of 16 tokens (gamma the in-chunk cumulative sum of g, padded
// tokens have g = 0, beta = 0 and zero inputs, so they are identity steps),
// with At = exp(gamma_r - gamma_c) (k_r . k_c) strictly below the diagonal,
// P = exp(gamma_r - gamma_c) (q_r . k_c) on and below it, T = (I + diag(beta)
// At)^-1, Gam = exp(gamma), Gp = exp(gamma_last - gamma), S0 the state before
// the chunk and G the gradient of the state after it, the chunk's writes and
// their gradients are (rows are tokens):
//     U  = T diag(beta) (V - diag(Gam) K S0^T)
//     dU = T^T (diag(Gp) K G^T + scale P^T dO)
//     S_after  = exp(gamma_last) S0 + (diag(Gp) U)^T K
//     G_before = exp(gamma_last) G + (scale diag(Gam) dO)^T Q - (diag(Gam beta) dU)^T K
// The passes:
//   1. prep, every (chunk, QK head) in parallel: gamma, beta, At, P and T of its V heads;
//   2. scans, per (sequence, V head, 16 state rows) and direction, chunk by
//      chunk: S0 of every chunk (forward) and G of every chunk (reverse, and the
//      gradient of the initial state);
//   3. gradients, every (chunk, V head) in parallel, in closed form from S0 and G;
//   4. dq and dk of each QK head from its V heads' shares, deterministically: one V
//      head stores its share; two add theirs into the output that pass 1 zeroed
//      (0 + a + b and 0 + b + a are the same float under IEEE addition, and also
//      when subnormal operands are flushed); three or more write their shares to the
//      workspace, which a last launch sums in a fixed order.
// Every product is fp32 MFMA 16x16x4: lane (g, m) = (lane / 16, lane % 16) gives
// A[m][k] and B[k][m] for the step's k and receives D[4 g + e][m], e = 0..3.
// Steps take k = 4 kk + g, which spreads a row-major operand's reads over the
// LDS banks; a contraction may also take its k in any other order that A and B share.
#include "gdn_common.h"
#include "gdn_internal.h"
#include "gdn_mfma.h"

namespace gdn {

typedef float f32x4 __attribute__((ext_vector_type(4)));
constexpr int kC = 16;   // tokens per chunk; also the checkpoint interval

// How dq and dk of a QK head are formed from its V heads' shares:
enum DqkMode {
    kDqkPartial = 0,   // per V head into the workspace, then summed in a fixed order (pass 4)
    kDqkDirect = 1,    // one V head per QK head: stored directly
    kDqkPair = 2,      // two V heads: each adds its share into the output, zeroed by pass 1; with
                       // exactly two addends on 0 the sum does not depend on their order
};

struct BwdIn {
    const void *q, *k, *v, *dout;
    const float *g, *beta;
    const int32_t* cu;
    int64_t total_tokens;
    int32_t num_seqs, num_qk_heads, num_v_heads;
    float scale;
    float *dq, *dk;    // the outputs [T, Hqk, d]
    int32_t dqk_mode;  // DqkMode
};

// Slot of chunk j of sequence n: cu[n] / 16 + n + j. The ranges of different
// sequences are disjoint and below T / 16 + N.
__device__ __forceinline__ int64_t ckpt_base(const int32_t* cu, int n) {
    return cu ? (int64_t)(cu[n] / kC) + n : 0;
}

// The chunk that slot sl holds: its sequence, first token and token count;
// false for a slot between two sequences' ranges.
__device__ __forceinline__ bool slot_chunk(const BwdIn& in, int64_t sl, int& n, int64_t& t0, int& cnt) {
    n = 0;
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
    if (j < 0 || j >= (eos - bos + kC - 1) / kC) return false;
    t0 = bos + j * kC;
    cnt = (int)min((int64_t)kC, eos - t0);
    return true;
}

template <bool BF16>
__device__ __forceinline__ float ld_in(const void* p, int64_t idx) {
    if constexpr (BF16) return bf16_bits_to_float(reinterpret_cast<const uint16_t*>(p)[idx]);
    else return reinterpret_cast<const float*>(p)[idx];
}

// NE (1, 2, 4 or 8) consecutive elements at idx, aligned to their size, as fp32.
template <bool BF16, int NE>
__device__ __forceinline__ void ld_vec(const void* p, int64_t idx, float (&out)[NE]) {
    static_assert(NE == 1 || NE == 2 || NE == 4 || NE == 8, "vector of 1, 2, 4 or 8");
    if constexpr (BF16) {
        const uint16_t* b = reinterpret_cast<const uint16_t*>(p) + idx;
        if constexpr (NE == 1) {
            out[0] = bf16_bits_to_float(*b);
        } else {
            typedef uint32_t u32v __attribute__((ext_vector_type(NE / 2)));
            const u32v v = *reinterpret_cast<const u32v*>(b);
#pragma unroll
            for (int i = 0; i < NE / 2; ++i) {
                out[2 * i] = __uint_as_float(v[i] << 16);
                out[2 * i + 1] = __uint_as_float(v[i] & 0xFFFF0000u);
            }
        }
    } else {
        const float* f = reinterpret_cast<const float*>(p) + idx;
        if constexpr (NE == 1) {
            out[0] = *f;
        } else {
            constexpr int V = NE < 4 ? NE : 4;
            typedef float f32v __attribute__((ext_vector_type(V)));
#pragma unroll
            for (int h = 0; h < NE / V; ++h) {
                const f32v v = *reinterpret_cast<const f32v*>(f + V * h);
#pragma unroll
                for (int i = 0; i < V; ++i) out[V * h + i] = v[i];
            }
        }
    }
}

// The same elements as raw 32-bit words (bf16 pairs or fp32), for loads whose
// values are not used until much later: converting them at once would make the
// wave wait for the load right there.
template <bool BF16, int NE>
struct Raw {
    static constexpr int W = BF16 ? (NE + 1) / 2 : NE;
    uint32_t w[W];
};
template <bool BF16, int NE>
__device__ __forceinline__ void ld_raw(const void* p, int64_t idx, Raw<BF16, NE>& r) {
    static_assert(NE == 1 || NE == 2 || NE == 4 || NE == 8, "vector of 1, 2, 4 or 8");
    if constexpr (BF16 && NE == 1) {
        r.w[0] = reinterpret_cast<const uint16_t*>(p)[idx];
    } else {
        const uint32_t* base = BF16 ? reinterpret_cast<const uint32_t*>(reinterpret_cast<const uint16_t*>(p) + idx)
                                    : reinterpret_cast<const uint32_t*>(reinterpret_cast<const float*>(p) + idx);
        constexpr int W = Raw<BF16, NE>::W, V = W < 4 ? W : 4;
        typedef uint32_t u32v __attribute__((ext_vector_type(V)));
#pragma unroll
        for (int h = 0; h < W / V; ++h) {
            const u32v v = *reinterpret_cast<const u32v*>(base + V * h);
#pragma unroll
            for (int i = 0; i < V; ++i) r.w[V * h + i] = v[i];
        }
    }
}
template <bool BF16, int NE>
__device__ __forceinline__ float raw_at(const Raw<BF16, NE>& r, int i) {
    if constexpr (!BF16) return __uint_as_float(r.w[i]);
    else if constexpr (NE == 1) return __uint_as_float(r.w[0] << 16);
    else return __uint_as_float((i & 1) ? (r.w[i / 2] & 0xFFFF0000u) : (r.w[i / 2] << 16));
}

__device__ __forceinline__ f32x4 mfma4(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

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

// Per (chunk slot, V head): the chunk's factors.
struct alignas(16) ChunkFac {
    float gam[kC], bet[kC];   // in-chunk cumulative g; beta (0 past the chunk's tokens)
    float Gam[kC], Gp[kC];    // exp(gamma), exp(gamma_last - gamma)
    float T[kC][kC];          // (I + diag(beta) At)^-1
    float P[kC][kC];          // exp(gamma_r - gamma_c) (q_r . k_c), c <= r
    float At[kC][kC];         // exp(gamma_r - gamma_c) (k_r . k_c), c < r
};

// Pass 1: one wave per (slot, QK head): K, Q and their Gram products (K K^T,
// Q K^T) once, then the decay-masked factors of each V head of the QK head,
// four V heads at a time (lanes 16 x .. 16 x + 15 take V head x0 + x).
template <int D, bool BF16>
__global__ __launch_bounds__(64) void backward_prep_kernel(BwdIn in, ChunkFac* __restrict__ fac) {
    constexpr int KP = D + 4;
    __shared__ __align__(16) float Kf[kC][KP], Qf[kC][KP];
    __shared__ float gin[4][kC], bet[4][kC], gam[4][kC], At[4][kC][kC + 1];
    const int hv = in.num_v_heads, hqk = in.num_qk_heads, hq = blockIdx.x % hqk, group = hv / hqk;
    const int64_t sl = blockIdx.x / hqk;
    int n, cnt;
    int64_t t0;
    if (!slot_chunk(in, sl, n, t0, cnt)) return;
    const int ln = threadIdx.x, g4 = ln / 16, m = ln % 16;
    if (in.dqk_mode == kDqkPair) {   // the chunk's dq and dk rows of this QK head start at 0
        if (((reinterpret_cast<uintptr_t>(in.dq) | reinterpret_cast<uintptr_t>(in.dk)) & 15) == 0) {
            const f32x4 z = {0.f, 0.f, 0.f, 0.f};
            for (int e = ln; e < cnt * (D / 4); e += 64) {
                const int64_t gi = ((t0 + e / (D / 4)) * hqk + hq) * D + 4 * (e % (D / 4));
                *reinterpret_cast<f32x4*>(in.dq + gi) = z;
                *reinterpret_cast<f32x4*>(in.dk + gi) = z;
            }
        } else {
            for (int e = ln; e < cnt * D; e += 64) {
                const int64_t gi = ((t0 + e / D) * hqk + hq) * D + e % D;
                in.dq[gi] = 0.f;
                in.dk[gi] = 0.f;
            }
        }
    }
    // K and Q rows in pieces of D / 16 elements (the scan reads its rows in the same pieces).
    constexpr int NE = D / 16;
    for (int e = ln; e < kC * 16; e += 64) {
        const int t = e / 16, c = NE * (e % 16);
        const int64_t idx = ((t0 + min(t, cnt - 1)) * hqk + hq) * D + c;
        const float keep = t < cnt ? 1.f : 0.f;
        float kv[NE], qv[NE];
        ld_vec<BF16, NE>(in.k, idx, kv);
        ld_vec<BF16, NE>(in.q, idx, qv);
#pragma unroll
        for (int i = 0; i < NE; ++i) {
            Kf[t][c + i] = keep * kv[i];
            Qf[t][c + i] = keep * qv[i];
        }
    }
    __syncthreads();
    f32x4 kk_ = {0.f, 0.f, 0.f, 0.f}, qk_ = kk_;
    for (int kk = 0; kk < D / 4; ++kk) {
        const int k = 4 * kk + g4;
        const float kv = Kf[m][k];
        kk_ = mfma4(kv, kv, kk_);
        qk_ = mfma4(Qf[m][k], kv, qk_);
    }
    // Lane (x, c) of a round: V head x0 + x, token (or column) c.
    const int x = ln / 16, c16 = ln % 16;
    for (int x0 = 0; x0 < group; x0 += 4) {
        const bool mine = x0 + x < group;
        const int hx = hq * group + x0 + x;   // this lane's V head (if mine)
        if (mine) {
            const int64_t gi = (t0 + min(c16, cnt - 1)) * hv + hx;
            const float keep = c16 < cnt ? 1.f : 0.f;
            gin[x][c16] = keep * in.g[gi];
            bet[x][c16] = keep * in.beta[gi];
        }
        __syncthreads();
        if (mine) {
            float s = 0.f;
            for (int t = 0; t <= c16; ++t) s += gin[x][t];
            gam[x][c16] = s;
        }
        __syncthreads();
        // At and P of every V head of the round, from the Gram tiles in this lane's registers.
        for (int xx = 0; xx < 4 && x0 + xx < group; ++xx) {
            ChunkFac& F = fac[sl * hv + hq * group + x0 + xx];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 4 * g4 + e, c = m;
                const float dec = exp_nonpos(fminf(gam[xx][r] - gam[xx][c], 0.f));
                const float at = c < r ? dec * kk_[e] : 0.f;
                At[xx][r][c] = at;
                F.At[r][c] = at;
                F.P[r][c] = c <= r ? dec * qk_[e] : 0.f;
            }
        }
        if (mine) {
            ChunkFac& F = fac[sl * hv + hx];
            F.gam[c16] = gam[x][c16];
            F.bet[c16] = bet[x][c16];
            F.Gam[c16] = exp_nonpos(gam[x][c16]);
            F.Gp[c16] = exp_nonpos(gam[x][kC - 1] - gam[x][c16]);
        }
        __syncthreads();
        // T by forward substitution, lane (x, c) solving column c of V head x0 + x.
        if (mine) {
            ChunkFac& F = fac[sl * hv + hx];
            const int c = c16;
            float Tc[kC];
#pragma unroll
            for (int r = 0; r < kC; ++r) {
                float s = r == c ? 1.f : 0.f;
                const float br = bet[x][r];
#pragma unroll
                for (int p = 0; p < r; ++p) s = fmaf(-br * At[x][r][p], Tc[p], s);
                Tc[r] = s;
            }
#pragma unroll
            for (int r = 0; r < kC; ++r) F.T[r][c] = Tc[r];
        }
        __syncthreads();   // the round's LDS is reused by the next
    }
}

// Pass 2: blocks [0, P) scan forward, blocks [P, 2P) in reverse, P = N Hv (d / 16);
// a block holds 16 state rows (value tile vt) of one (sequence, V head) as
// transposed 16 x 16 tiles in its waves' MFMA accumulators, wave w the key tiles
// w, w + 4, ... (lane (g, m) of key tile tk: rows 16 vt + m, columns 16 tk + 4 g + e).
// That layout is also the B operand of K S0^T when step (tk, e) takes, in lane
// group g, key 16 tk + 4 g + e, so the state never leaves the registers; each
// wave adds its key tiles' share of K S0^T (or K G^T) and the shares meet in LDS,
// one barrier per chunk. The inputs of later chunks are loaded into two
// register sets ahead of use and kept in a ring of three LDS buffers.
template <int D>
struct ScanShape {
    static constexpr int NTD = D / 16;            // 16-wide tiles over d
    static constexpr int TPW = (NTD + 3) / 4;     // key tiles per wave
    static constexpr int EPT = D / 16;            // staged k (or q) elements per thread: one row piece
};

template <int D>
struct ScanSmem {
    // K, Q rows 16-byte aligned (the commit and the K X^T operands move 16 bytes per
    // access); the odd pitch of the 16 x 16 matrices spreads a column over the banks.
    static constexpr int KP = D + 4, SP = kC + 1;
    float Kc[3][kC][KP], Qc[3][kC][KP];
    float Xc[3][kC][SP], Tc[3][kC][SP], Pc[3][kC][SP], Gc[3][kC], Hc[3][kC], bc[3][kC];   // Hc: Gp
    float part[2][4][kC][SP];
};

// One direction's scan (REV: the gradient, in reverse); b indexes (sequence, V head, value tile).
template <int D, bool BF16, bool REV>
__device__ __forceinline__ void scan_body(ScanSmem<D>& sm, const BwdIn& in, const ChunkFac* __restrict__ fac,
                                          const float* __restrict__ init, float* __restrict__ dinit,
                                          float* __restrict__ ck, int64_t b) {
    using Sh = ScanShape<D>;
    constexpr int NTD = Sh::NTD, TPW = Sh::TPW, EPT = Sh::EPT;
    // Every wave has TPW whole d tiles when the tiles divide evenly among the four waves; the
    // guard below is then a constant (left to the wave index, it put a branch around every
    // tile's products and kept their LDS reads from being batched).
    constexpr bool kAllTiles = (NTD % 4 == 0);
    constexpr bool rev = REV;
    auto& Kc = sm.Kc;
    auto& Qc = sm.Qc;
    auto& Xc = sm.Xc;
    auto& Tc = sm.Tc;
    auto& Pc = sm.Pc;
    auto& Gc = sm.Gc;
    auto& Hc = sm.Hc;
    auto& bc = sm.bc;
    auto& part = sm.part;
    const int hv = in.num_v_heads, hqk = in.num_qk_heads;
    const int vt = (int)(b % NTD);
    const int nh = (int)(b / NTD);
    const int n = nh / hv, h = nh % hv, hq = h / (hv / hqk);
    const int64_t bos = in.cu ? (int64_t)in.cu[n] : 0, eos = in.cu ? (int64_t)in.cu[n + 1] : in.total_tokens;
    const int64_t cbase = ckpt_base(in.cu, n);
    const int nint = (int)((eos - bos + kC - 1) / kC);
    const int tid = threadIdx.x, w = tid / 64, ln = tid % 64, g4 = ln / 16, m = ln % 16;
    const int64_t sbase = ((int64_t)n * hv + h) * D * D;
    const float scale = in.scale;
    const int row = 16 * vt + m;   // this lane's state row

    // One chunk's inputs in registers. Thread tid stages token row tid / 16 of K
    // (and Q), columns EPT (tid % 16) .. + EPT - 1, and element (tid / 16, tid % 16)
    // of the 16 x 16 value tile and of T, P.
    struct Pre {
        Raw<BF16, EPT> k, q;
        Raw<BF16, 1> x;
        float t, p, G, H, b;
        bool keep;   // the thread's token row is inside the chunk (applied at commit, so
                     // that nothing waits for the loads before then)
    };
    const int ktt = tid / 16, kcol = EPT * (tid % 16);
    auto chunk_at = [&](int q) { return rev ? nint - 1 - q : q; };   // q-th chunk in scan order
    auto fetch = [&](Pre& pre, int q) {
        const int c = chunk_at(q);
        const int64_t t0 = bos + (int64_t)c * kC;
        const int cnt = (int)min((int64_t)kC, eos - t0);
        const int rr = min(ktt, cnt - 1);   // rows past the chunk re-read its last row, then read as 0
        pre.keep = ktt < cnt;
        const int64_t kb = (t0 * hqk + hq) * D + (int64_t)rr * hqk * D + kcol;
        ld_raw<BF16, EPT>(in.k, kb, pre.k);
        if constexpr (REV) ld_raw<BF16, EPT>(in.q, kb, pre.q);
        const int64_t xb = (t0 * hv + h) * D + (int64_t)rr * hv * D + 16 * vt + tid % 16;
        ld_raw<BF16, 1>(REV ? in.dout : in.v, xb, pre.x);
        const ChunkFac& F = fac[(cbase + c) * hv + h];
        pre.t = F.T[tid / 16][tid % 16];
        if constexpr (REV) pre.p = F.P[tid / 16][tid % 16];
        pre.G = F.Gam[tid % kC];   // every lane loads (no branch around the loads); tid < 16 keep theirs
        pre.H = F.Gp[tid % kC];
        pre.b = F.bet[tid % kC];
    };
    auto commit = [&](const Pre& pre, int buf) {
#pragma unroll
        for (int i = 0; i < EPT; ++i) {
            Kc[buf][ktt][kcol + i] = pre.keep ? raw_at(pre.k, i) : 0.f;
            if constexpr (REV) Qc[buf][ktt][kcol + i] = pre.keep ? raw_at(pre.q, i) : 0.f;
        }
        Xc[buf][tid / 16][tid % 16] = pre.keep ? raw_at(pre.x, 0) : 0.f;
        Tc[buf][tid / 16][tid % 16] = pre.t;
        if constexpr (REV) Pc[buf][tid / 16][tid % 16] = pre.p;
        if (tid < kC) {
            Gc[buf][tid] = pre.G;
            Hc[buf][tid] = pre.H;
            bc[buf][tid] = pre.b;
        }
    };

    // The state (forward) or its gradient (reverse), transposed tiles.
    f32x4 acc[TPW];
    {
        const float* src = init ? init + sbase : nullptr;
#pragma unroll
        for (int i = 0; i < TPW; ++i) {
            const int tk = w + 4 * i;
            acc[i] = (src && (kAllTiles || tk < NTD)) ? *reinterpret_cast<const f32x4*>(src + row * D + 16 * tk + 4 * g4)
                                       : f32x4{0.f, 0.f, 0.f, 0.f};
        }
        // Let these loads finish here, once: otherwise the compiler, unable to
        // tell whether they are still in flight when the chunk loop starts, waits
        // for every outstanding load (the prefetch included) at each use of the
        // state inside the loop.
        __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0); expcnt, lgkmcnt unconstrained
    }
    // Chunks q and q + 1 sit in LDS when chunk q starts; two register sets hold
    // chunks q + 2 and q + 3 on their way (loaded two chunks ahead of use).
    Pre pa, pb;
    if (nint > 0) {
        fetch(pa, 0);
        commit(pa, 0);
    }
    if (nint > 1) {
        fetch(pb, 1);
        commit(pb, 1);
    }
    mf::lds_barrier();
    if (nint > 2) fetch(pa, 2);
    if (nint > 3) fetch(pb, 3);
    f32x4 zkeep = {0.f, 0.f, 0.f, 0.f};   // reverse: this chunk's Z
    // Each phase below reads all of its LDS operands before its products (a scheduling barrier
    // between the two): left to the scheduler, every product waited for its own operand reads.
    auto chunk = [&](int q, Pre& pre) {
        const int c = chunk_at(q), bb = q % 3, pp = q & 1;
        // This wave's share of K X^T (X: the state or its gradient) and, in reverse, Z = P^T dO
        // (no dependence on the gradient).
        {
            float ka[TPW][4];
#pragma unroll
            for (int i = 0; i < TPW; ++i) {
                const int tk = w + 4 * i;
#pragma unroll
                for (int e = 0; e < 4; ++e) ka[i][e] = (kAllTiles || tk < NTD) ? Kc[bb][m][16 * tk + 4 * g4 + e] : 0.f;
            }
            float pz[4], xz[4];
            if constexpr (REV) {
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) {
                    pz[kk] = Pc[bb][4 * kk + g4][m];
                    xz[kk] = Xc[bb][4 * kk + g4][m];
                }
            }
            __builtin_amdgcn_sched_barrier(0);
            f32x4 ps = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int i = 0; i < TPW; ++i) {
                const int tk = w + 4 * i;
                if (kAllTiles || tk < NTD) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) ps = mfma4(ka[i][e], acc[i][e], ps);
                }
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) part[pp][w][4 * g4 + e][m] = ps[e];
            if constexpr (REV) {
                f32x4 zz = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) zz = mfma4(pz[kk], xz[kk], zz);
                zkeep = zz;
            }
        }
        mf::lds_barrier();
        // Buffer (q + 2) % 3 was last read in chunk q - 1, which every wave has finished.
        if (q + 2 < nint) commit(pre, (q + 2) % 3);
        // Checkpoint: the state at the chunk's start (forward), the gradient at its end (reverse),
        // unchanged until the update below. Stored after the commit: stores count among the
        // outstanding vector memory operations, and the commit's wait for its loads (issued two
        // chunks earlier) would otherwise also wait for these stores to complete.
        {
            float* dst = ck + ((cbase + c) * hv + h) * (int64_t)D * D + row * D;
#pragma unroll
            for (int i = 0; i < TPW; ++i) {
                const int tk = w + 4 * i;
                if (kAllTiles || tk < NTD) *reinterpret_cast<f32x4*>(dst + 16 * tk + 4 * g4) = acc[i];
            }
        }
        if (q + 4 < nint) fetch(pre, q + 4);
        const float GL = Gc[bb][kC - 1];   // exp(gamma_last)
        // The update's K (and Q) operands, read with the phase's other operands. The update takes
        // its reduction index (the token) in the order 4 g + kk, the row order of an accumulator
        // tile, so that U (forward) or dU (reverse) enters it straight from its accumulator.
        float ku[TPW][4], qu[TPW][4];
#pragma unroll
        for (int i = 0; i < TPW; ++i) {
            const int tk = w + 4 * i;
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                const int tau = 4 * g4 + kk;
                ku[i][kk] = (kAllTiles || tk < NTD) ? Kc[bb][tau][16 * tk + m] : 0.f;
                if constexpr (REV) qu[i][kk] = (kAllTiles || tk < NTD) ? Qc[bb][tau][16 * tk + m] : 0.f;
            }
        }
        if constexpr (!REV) {
            // U = T diag(beta) (V - diag(Gam) K S0^T); its accumulator scaled by Gp is the update's operand.
            float pr[4][4], xr[4], gr[4], br[4], tr[4], hr[4];
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                const int tau = 4 * kk + g4;
#pragma unroll
                for (int ww = 0; ww < 4; ++ww) pr[kk][ww] = part[pp][ww][tau][m];
                xr[kk] = Xc[bb][tau][m];
                gr[kk] = Gc[bb][tau];
                br[kk] = bc[bb][tau];
                tr[kk] = Tc[bb][m][tau];
                hr[kk] = Hc[bb][4 * g4 + kk];
            }
            __builtin_amdgcn_sched_barrier(0);
            f32x4 u = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                const float ks = (pr[kk][0] + pr[kk][1]) + (pr[kk][2] + pr[kk][3]);
                u = mfma4(tr[kk], br[kk] * (xr[kk] - gr[kk] * ks), u);
            }
            // S^T <- exp(gamma_last) S^T + K^T (Gp U)
            float uu[4];
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) uu[kk] = hr[kk] * u[kk];
#pragma unroll
            for (int i = 0; i < TPW; ++i) {
                const int tk = w + 4 * i;
                if (kAllTiles || tk < NTD) {
                    f32x4 a = acc[i] * GL;
#pragma unroll
                    for (int kk = 0; kk < 4; ++kk) a = mfma4(ku[i][kk], uu[kk], a);
                    acc[i] = a;
                }
            }
        } else {
            // Y = Gp K G^T + scale Z, dU = T^T Y, then -Gam beta dU. Every product here takes its
            // reduction index in the order 4 g + kk, so Y and dU pass from one product to the next
            // in registers: lane (g, m) holds rows 4 g .. 4 g + 3 of column m of each.
            float pr[4][4], hr[4], gr[4], br[4], tt[4], gx[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int tau = 4 * g4 + e;
#pragma unroll
                for (int ww = 0; ww < 4; ++ww) pr[e][ww] = part[pp][ww][tau][m];
                hr[e] = Hc[bb][tau];
                gr[e] = Gc[bb][tau];
                br[e] = bc[bb][tau];
                tt[e] = Tc[bb][tau][m];
                gx[e] = scale * Gc[bb][tau] * Xc[bb][tau][m];
            }
            __builtin_amdgcn_sched_barrier(0);
            float y[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float kg = (pr[e][0] + pr[e][1]) + (pr[e][2] + pr[e][3]);
                y[e] = fmaf(hr[e], kg, scale * zkeep[e]);
            }
            f32x4 du = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) du = mfma4(tt[kk], y[kk], du);
            // G^T <- exp(gamma_last) G^T + Q^T (scale Gam dO) + K^T (-Gam beta dU)
            float uu[4];
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) uu[kk] = -gr[kk] * br[kk] * du[kk];
#pragma unroll
            for (int i = 0; i < TPW; ++i) {
                const int tk = w + 4 * i;
                if (kAllTiles || tk < NTD) {
                    f32x4 a = acc[i] * GL;
#pragma unroll
                    for (int kk = 0; kk < 4; ++kk) {
                        a = mfma4(qu[i][kk], gx[kk], a);
                        a = mfma4(ku[i][kk], uu[kk], a);
                    }
                    acc[i] = a;
                }
            }
        }
    };
    for (int q = 0; q < nint; q += 2) {
        chunk(q, pa);
        if (q + 1 < nint) chunk(q + 1, pb);
    }
    if (REV && dinit) {
#pragma unroll
        for (int i = 0; i < TPW; ++i) {
            const int tk = w + 4 * i;
            if (kAllTiles || tk < NTD) *reinterpret_cast<f32x4*>(dinit + sbase + row * D + 16 * tk + 4 * g4) = acc[i];
        }
    }
}

template <int D, bool BF16>
__global__ __launch_bounds__(256) void backward_scan_kernel(
    BwdIn in, const ChunkFac* __restrict__ fac, const float* __restrict__ initial_state,
    const float* __restrict__ dfinal, float* __restrict__ dinit, float* __restrict__ ck_s,
    float* __restrict__ ck_ds) {
    __shared__ __align__(16) ScanSmem<D> sm;
    const int64_t P = (int64_t)in.num_seqs * in.num_v_heads * (D / 16);
    if (blockIdx.x >= P) scan_body<D, BF16, true>(sm, in, fac, dfinal, dinit, ck_ds, blockIdx.x - P);
    else scan_body<D, BF16, false>(sm, in, fac, initial_state, nullptr, ck_s, blockIdx.x);
}

// Pass 3, one workgroup (4 waves) per (chunk slot, V head), from the chunk's
// factors, S0 and G. With U, dU as above, AW = diag(Gam) K S0^T + At U (alpha w
// of every token) and the rows' dot products over the value index:
//   dv = diag(beta) dU,   dbeta_t = du_t . (v_t - AW_t)
//   dQ = scale (diag(Gam) dO S0 + M4 K),           M4 = [tau <= t] dec (dO U^T)
//   dK = diag(Gp) U G - diag(beta Gam) dU S0 + scale M4^T Q - M5 K,
//        M5[t][s] = [s > t] dec[s][t] beta_s (dU U^T)[s][t] + [s < t] beta_t dec[t][s] (dU U^T)[t][s]
//   dg_t = exp(gamma_last) <G, S0> + sum_{tau < t} a_tau + sum_{s >= t} b_s - sum_{s > t} c_s
//          + sum_{s >= t, tau < t} scale P[s][tau] (dO U^T)[s][tau]
//          - sum_{s > t, tau < t} beta_s At[s][tau] (dU U^T)[s][tau] - beta_t du_t . AW_t,
//   a = Gp (U G . K), b = scale Gam (dO S0 . Q), c = Gam beta (dU S0 . K) (row dots),
// dec[r][c] = exp(gamma_r - gamma_c). Products over the value index (U G, dO S0,
// dU S0, dO U^T, dU U^T, <G, S0>) run over blocks of 16 state rows staged in LDS
// and accumulate in registers (16-row blocks keep the LDS at 52 KB for d = 128,
// so three workgroups share a CU).
template <int D>
struct ChunkShape {
    static constexpr int R = 16;                // state rows per block
    static constexpr int NB = D / R;            // blocks
    static constexpr int KP = D + 4;            // fp32 row pitch of d-wide rows
    static constexpr int BP = R + 4;            // fp32 row pitch of block-wide rows
    static constexpr int NTD = D / 16;          // 16-column tiles over d
    static constexpr int NTR = R / 16;          // 16-column tiles over a block
    static constexpr int TPW = (NTD + 3) / 4;   // d tiles per wave
};


template <int D, bool BF16>
__global__ __launch_bounds__(256) void backward_grad_kernel(
    BwdIn in, const ChunkFac* __restrict__ fac, const float* __restrict__ ck_s, const float* __restrict__ ck_ds,
    float* __restrict__ dq_h, float* __restrict__ dk_h, float* __restrict__ dg, float* __restrict__ dbeta,
    float* __restrict__ dv) {
    using CS = ChunkShape<D>;
    constexpr int C = kC, R = CS::R, NB = CS::NB, KP = CS::KP, BP = CS::BP, NTD = CS::NTD, NTR = CS::NTR,
                  TPW = CS::TPW;
    constexpr int SP = C + 1;   // pitch of the 16 x 16 matrices
    static_assert(C == 16 && R % 16 == 0, "chunk of 16 tokens, blocks of whole tiles");
    __shared__ __align__(16) float Kf[C][KP], Qf[C][KP];
    __shared__ __align__(16) float Sb[R][KP], Gb[R][KP];
    __shared__ float Vb[C][BP], dOb[C][BP], KSs[C][BP], KGs[C][BP], Us[C][BP], dUs[C][BP], Rs[C][BP];
    __shared__ float At[C][SP], Pm[C][SP], Tm[C][SP], M4[C][SP], M5[C][SP], dOU[C][SP], DUm[C][SP], Rm[C][SP];
    __shared__ float gam[C], Gam[C], Gp[C], bet[C], part[4][3][C], red[4], dgs[C];

    const int hv = in.num_v_heads, hqk = in.num_qk_heads, h = blockIdx.x % hv, hq = h / (hv / hqk);
    const int64_t sl = blockIdx.x / hv;
    int n, cnt;
    int64_t t0;
    if (!slot_chunk(in, sl, n, t0, cnt)) return;   // a gap slot: uniform over the block
    const int tid = threadIdx.x, w = tid / 64, ln = tid % 64, g4 = ln / 16, m = ln % 16;
    const float scale = in.scale;
    const int64_t off = (sl * hv + h) * (int64_t)D * D;
    const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};

    // Stage K, Q (rows past cnt are zero; thread tid: row tid / 16, D / 16 columns)
    // and the chunk's factors.
    {
        constexpr int EPT = D / 16;
        const int t = tid / 16, c0 = EPT * (tid % 16);
        const int64_t idx = ((t0 + min(t, cnt - 1)) * hqk + hq) * D + c0;
        float kv[EPT], qv[EPT];
        ld_vec<BF16, EPT>(in.k, idx, kv);
        ld_vec<BF16, EPT>(in.q, idx, qv);
#pragma unroll
        for (int i = 0; i < EPT; ++i) {
            Kf[t][c0 + i] = t < cnt ? kv[i] : 0.f;
            Qf[t][c0 + i] = t < cnt ? qv[i] : 0.f;
        }
    }
    {
        const ChunkFac& F = fac[sl * hv + h];
        const int r = tid / 16, c = tid % 16;
        Tm[r][c] = F.T[r][c];
        Pm[r][c] = F.P[r][c];
        At[r][c] = F.At[r][c];
        if (tid < C) {
            gam[tid] = F.gam[tid];
            bet[tid] = F.bet[tid];
            Gam[tid] = F.Gam[tid];
            Gp[tid] = F.Gp[tid];
        }
    }
    // Accumulators over the blocks: U G, dO S0, dU S0 for this wave's d tiles; dO U^T
    // (wave 2) and dU U^T (wave 3); row sums for dbeta and du . AW; <G, S0>.
    f32x4 accUG[TPW], accOS[TPW], accUS[TPW], accM = zero4;
#pragma unroll
    for (int i = 0; i < TPW; ++i) accUG[i] = accOS[i] = accUS[i] = zero4;
    float p_db = 0.f, p_dw = 0.f, p_gs = 0.f;
    const int vt = tid / 16, vp = tid % 16;   // token and column phase for the row sums

    // Rows of S0 and G, and columns of V and dO, of block rb + 1 on their way while
    // block rb is processed (raw words, converted when written to LDS).
    constexpr int BV = (R * D + 4 * 256 - 1) / (4 * 256);   // f32x4 pieces per thread and matrix
    constexpr int VV = (C * R + 255) / 256;                 // V (and dO) elements per thread
    f32x4 nS[BV], nG[BV];
    Raw<BF16, 1> nV[VV], nO[VV];
    auto load_block = [&](int rb) {
        const float* s0 = ck_s + off + (int64_t)rb * R * D;
        const float* gg = ck_ds + off + (int64_t)rb * R * D;
#pragma unroll
        for (int i = 0; i < BV; ++i) {
            const int e = min(4 * tid + 4 * 256 * i, R * D - 4);
            nS[i] = *reinterpret_cast<const f32x4*>(s0 + e);
            nG[i] = *reinterpret_cast<const f32x4*>(gg + e);
        }
#pragma unroll
        for (int i = 0; i < VV; ++i) {
            const int e = min(tid + 256 * i, C * R - 1), t = e / R, c = e % R;
            const int64_t idx = ((t0 + min(t, cnt - 1)) * hv + h) * D + rb * R + c;
            ld_raw<BF16, 1>(in.v, idx, nV[i]);
            ld_raw<BF16, 1>(in.dout, idx, nO[i]);
        }
    };
    load_block(0);
    for (int rb = 0; rb < NB; ++rb) {
        mf::lds_barrier();   // the previous block's LDS reads are done (and the factors are staged)
        // Stage this block's rows of S0 and G, and its columns of V and dO.
        {
#pragma unroll
            for (int i = 0; i < BV; ++i) {
                const int e = 4 * tid + 4 * 256 * i;
                if (e < R * D) {
                    *reinterpret_cast<f32x4*>(&Sb[e / D][e % D]) = nS[i];
                    *reinterpret_cast<f32x4*>(&Gb[e / D][e % D]) = nG[i];
                }
            }
#pragma unroll
            for (int i = 0; i < VV; ++i) {
                const int e = tid + 256 * i, t = e / R, c = e % R;
                if (e < C * R) {
                    Vb[t][c] = t < cnt ? raw_at(nV[i], 0) : 0.f;
                    dOb[t][c] = t < cnt ? raw_at(nO[i], 0) : 0.f;
                }
            }
            if (rb + 1 < NB) load_block(rb + 1);
        }
        mf::lds_barrier();
        // K S0^T (waves 0, 2) and K G^T (waves 1, 3) for the block's 16 columns, each wave over
        // one half of the d keys (two chains of D / 8 steps instead of one of D / 4 on two
        // waves). The second halves go to Rs and dUs, which are written only after those
        // halves are read (by the same wave, same elements), and are added where read.
        {
            static_assert(NTR == 1, "one 16-column tile per block");
            const float (*B)[KP] = (w & 1) ? Gb : Sb;
            const int k0 = (w >> 1) * (D / 8);
            f32x4 acc = zero4;
            for (int kk = k0; kk < k0 + D / 8; ++kk) {
                const int k = 4 * kk + g4;
                acc = mfma4(Kf[m][k], B[m][k], acc);
            }
            float (*dst)[BP] = w == 0 ? KSs : w == 1 ? KGs : w == 2 ? Rs : dUs;
#pragma unroll
            for (int e = 0; e < 4; ++e) dst[4 * g4 + e][m] = acc[e];
        }
        float (*KSh)[BP] = Rs;    // K S0^T, second half of the keys
        float (*KGh)[BP] = dUs;   // K G^T, second half of the keys
        mf::lds_barrier();
        // U, then AW = Gam K S0^T + At U and R = V - AW (wave 0); Z = P^T dO, Y = Gp K G^T + scale Z,
        // then dU = T^T Y (wave 2). The second product of each takes its reduction index in the
        // order 4 g + kk, the row order of an accumulator tile, so U and Y reach it in registers.
        if (w < NTR) {
            const int c = 16 * w + m;
            f32x4 u = zero4;
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                const int k = 4 * kk + g4;
                u = mfma4(Tm[m][k], bet[k] * (Vb[k][c] - Gam[k] * (KSs[k][c] + KSh[k][c])), u);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) Us[4 * g4 + e][c] = u[e];
            f32x4 acc = zero4;
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) acc = mfma4(At[m][4 * g4 + kk], u[kk], acc);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int t = 4 * g4 + e;
                Rs[t][c] = Vb[t][c] - fmaf(Gam[t], KSs[t][c] + KSh[t][c], acc[e]);
            }
        } else if (w >= 2 && w < 2 + NTR) {
            const int c = 16 * (w - 2) + m;
            f32x4 z = zero4;
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                const int k = 4 * kk + g4;
                z = mfma4(Pm[k][m], dOb[k][c], z);
            }
            float y[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int t = 4 * g4 + e;
                y[e] = fmaf(Gp[t], KGs[t][c] + KGh[t][c], scale * z[e]);   // Y = Gp K G^T + scale P^T dO
            }
            f32x4 acc = zero4;
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) acc = mfma4(Tm[4 * g4 + kk][m], y[kk], acc);
#pragma unroll
            for (int e = 0; e < 4; ++e) dUs[4 * g4 + e][c] = acc[e];
        }
        mf::lds_barrier();
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
    mf::lds_barrier();
    // M4, M5 and the dg terms, one thread per (row s, column t) of the 16 x 16
    // matrices: thread (s, t) builds M4[s][t], M5[s][t] and row s's share of
    // token t's dg; the shares are then summed per token.
    {
        const int sr = tid / 16, tc = tid % 16;
        const float drc = gam[sr] - gam[tc];
        M4[sr][tc] = tc <= sr ? exp_nonpos(drc) * dOU[sr][tc] : 0.f;
        float m5 = 0.f;
        if (tc > sr) m5 = exp_nonpos(-drc) * bet[tc] * DUm[tc][sr];
        if (tc < sr) m5 = bet[sr] * exp_nonpos(drc) * DUm[sr][tc];
        M5[sr][tc] = m5;
        const float a = Gp[sr] * (part[0][0][sr] + part[1][0][sr] + part[2][0][sr] + part[3][0][sr]);
        const float b = scale * Gam[sr] * (part[0][1][sr] + part[1][1][sr] + part[2][1][sr] + part[3][1][sr]);
        const float c3 = Gam[sr] * bet[sr] * (part[0][2][sr] + part[1][2][sr] + part[2][2][sr] + part[3][2][sr]);
        // rectangle terms of row s >= t: sum over tau < t
        float r1 = 0.f, r2 = 0.f;
#pragma unroll
        for (int tau = 0; tau < C; ++tau) {
            const float on = tau < tc ? 1.f : 0.f;
            r1 = fmaf(on * Pm[sr][tau], dOU[sr][tau], r1);
            r2 = fmaf(on * At[sr][tau], DUm[sr][tau], r2);
        }
        float x = (sr < tc ? a : 0.f) - (sr > tc ? c3 + bet[sr] * r2 : 0.f);
        if (sr >= tc) x += b + scale * r1;
        Rm[sr][tc] = x;
    }
    mf::lds_barrier();
    if (tid < C) {
        float sum = 0.f;
        for (int sr = 0; sr < C; ++sr) sum += Rm[sr][tid];
        dgs[tid] = Gam[C - 1] * (red[0] + red[1] + red[2] + red[3]) + sum;
    }
    mf::lds_barrier();
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
                    if (in.dqk_mode == kDqkPartial) {
                        const int64_t gi = ((t0 + t) * hv + h) * D + col;
                        dq_h[gi] = scale * q_[e];
                        dk_h[gi] = k_[e];
                    } else {
                        const int64_t gi = ((t0 + t) * hqk + hq) * D + col;
                        if (in.dqk_mode == kDqkDirect) {
                            in.dq[gi] = scale * q_[e];
                            in.dk[gi] = k_[e];
                        } else {
                            unsafeAtomicAdd(in.dq + gi, scale * q_[e]);
                            unsafeAtomicAdd(in.dk + gi, k_[e]);
                        }
                    }
                }
            }
        }
    }
}

// Pass 4, dq and dk of a QK head: the sum over its V heads.
__global__ void backward_qk_sum_kernel(const float* __restrict__ part, float* __restrict__ dst, int64_t rows,
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

// The same sums over 16-byte words, dq (blockIdx.y = 0) and dk (1) in one launch:
// output word e4 is word e4 % (d / 4) of row e4 / (d / 4) (d / 4 = 1 << lg), and
// the group's parts of a row are consecutive rows of `part`. The parts are added
// in the same order as above, so the sums are the same.
__global__ void backward_qk_sum4_kernel(const float* __restrict__ part_q, const float* __restrict__ part_k,
                                        float* __restrict__ dq, float* __restrict__ dk, int64_t n4, int32_t group,
                                        int32_t lg) {
    const int64_t e4 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (e4 >= n4) return;
    const f32x4* part = reinterpret_cast<const f32x4*>(blockIdx.y ? part_k : part_q);
    f32x4* dst = reinterpret_cast<f32x4*>(blockIdx.y ? dk : dq);
    const int64_t d4 = (int64_t)1 << lg;
    const f32x4* p = part + (e4 >> lg) * group * d4 + (e4 & (d4 - 1));
    f32x4 s = {0.f, 0.f, 0.f, 0.f};
    for (int x = 0; x < group; ++x) s += p[x * d4];
    dst[e4] = s;
}

size_t backward_workspace_bytes(int64_t total_tokens, int32_t num_seqs, int32_t num_v_heads, int32_t d) {
    const int64_t slots = total_tokens / kC + num_seqs;
    const size_t ck = (size_t)slots * num_v_heads * d * d * sizeof(float);    // one checkpoint array
    const size_t qk = (size_t)total_tokens * num_v_heads * d * sizeof(float);  // dq or dk per V head
    const size_t fc = (size_t)slots * num_v_heads * sizeof(ChunkFac);
    return 2 * ck + 2 * qk + fc;
}

template <int D, bool BF16>
static hipError_t launch_bwd_t(const BackwardArgs& a, hipStream_t stream) {
    static_assert(sizeof(ChunkFac) % 16 == 0, "factor records keep the arrays after them aligned");
    float* ws = static_cast<float*>(a.workspace);
    const int64_t slots = a.total_tokens / kC + a.num_seqs;
    const size_t ck = (size_t)slots * a.num_v_heads * D * D;
    const size_t qk = (size_t)a.total_tokens * a.num_v_heads * D;
    float* ck_s = ws;
    float* ck_ds = ck_s + ck;
    float* dq_h = ck_ds + ck;
    float* dk_h = dq_h + qk;
    ChunkFac* fac = reinterpret_cast<ChunkFac*>(dk_h + qk);
    const int group = a.num_v_heads / a.num_qk_heads;
    const int32_t mode = group == 1 ? kDqkDirect : group == 2 ? kDqkPair : kDqkPartial;
    const BwdIn in{a.q, a.k, a.v, a.d_out, a.g, a.beta, a.cu_seqlens, a.total_tokens,
                   a.num_seqs, a.num_qk_heads, a.num_v_heads, a.scale, a.dq, a.dk, mode};
    const unsigned chunks = (unsigned)(slots * a.num_v_heads);
    hipError_t e;
    if (a.total_tokens > 0) {
        prof::begin(stream, "gdn_backward_prep");
        hipLaunchKernelGGL((backward_prep_kernel<D, BF16>), dim3((unsigned)(slots * a.num_qk_heads)), dim3(64), 0,
                           stream, in, fac);
        prof::end(stream);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    const int64_t P = (int64_t)a.num_seqs * a.num_v_heads * (D / 16);
    prof::begin(stream, "gdn_backward_scan");
    hipLaunchKernelGGL((backward_scan_kernel<D, BF16>), dim3((unsigned)(2 * P)), dim3(256), 0, stream, in, fac,
                       a.initial_state, a.d_final_state, a.d_initial_state, ck_s, ck_ds);
    prof::end(stream);
    if ((e = hipGetLastError()) != hipSuccess || a.total_tokens == 0) return e;
    prof::begin(stream, "gdn_backward_grad");
    hipLaunchKernelGGL((backward_grad_kernel<D, BF16>), dim3(chunks), dim3(256), 0, stream, in, fac, ck_s, ck_ds,
                       dq_h, dk_h, a.dg, a.dbeta, a.dv);
    prof::end(stream);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (mode != kDqkPartial) return hipSuccess;
    const int64_t nqk = a.total_tokens * a.num_qk_heads * D;
    prof::begin(stream, "gdn_backward_sums");
    const bool aligned = ((reinterpret_cast<uintptr_t>(dq_h) | reinterpret_cast<uintptr_t>(dk_h) |
                           reinterpret_cast<uintptr_t>(a.dq) | reinterpret_cast<uintptr_t>(a.dk)) & 15) == 0;
    if (aligned) {
        constexpr int lg = D == 16 ? 2 : D == 32 ? 3 : D == 64 ? 4 : 5;
        static_assert((4 << lg) == D, "d / 4 is a power of two");
        const int64_t n4 = nqk / 4;
        hipLaunchKernelGGL(backward_qk_sum4_kernel, dim3((unsigned)((n4 + 255) / 256), 2), dim3(256), 0, stream, dq_h,
                           dk_h, a.dq, a.dk, n4, group, lg);
    } else {
        hipLaunchKernelGGL(backward_qk_sum_kernel, dim3((unsigned)((nqk + 255) / 256)), dim3(256), 0, stream, dq_h,
                           a.dq, a.total_tokens, a.num_qk_heads, group, D);
        hipLaunchKernelGGL(backward_qk_sum_kernel, dim3((unsigned)((nqk + 255) / 256)), dim3(256), 0, stream, dk_h,
                           a.dk, a.total_tokens, a.num_qk_heads, group, D);
    }
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
