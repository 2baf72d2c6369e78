// Chunked Gated DeltaNet prefill with bf16 MFMA (gfx950), d_k = d_v = 128.
//
// Chunk algebra (chunk of n <= 64 tokens, state S0 on entry; gamma = in-chunk
// cumulative sum of g; Gamma = exp(gamma)):
//   A[r][c] = beta_r exp(gamma_r - gamma_c) (k_r . k_c), c < r      decay-masked Gram
//   Tm      = (I + A)^-1                                            UT transform
//   U       = Tm (beta * (V - Gamma * (K S0^T)))                    the chunk's delta writes
//   O       = scale (Gamma * (Q S0^T) + P U),  P[r][c] = exp(gamma_r - gamma_c) (q_r . k_c), c <= r
//   S_end   = Gamma_last S0 + U^T diag(exp(gamma_last - gamma)) K
// (derivation: unrolling the per-token rule inside the chunk; the write of
// token r sees the decayed entry state plus the chunk's earlier writes, which
// is the unit lower-triangular system (I + A) U = beta * (V - Gamma * K S0^T)).
//
// Two kernels:
//  * prep  - one workgroup per (chunk slot, QK head), fully parallel. K K^T
//            and Q K^T by MFMA once per QK head, then for each V head of the
//            group: decay masks, A, P, and Tm by a blocked forward
//            substitution in fp32 (16 x 16 diagonal blocks per lane column,
//            then three levels of block products). Tm and P go to the
//            workspace as bf16, gamma as fp32.
//  * chain - one workgroup per (sequence, V head, value-column split); walks
//            the sequence's chunks in order with the fp32 state held in MFMA
//            accumulators. Each wave owns 16*NW value columns, so the four
//            waves never exchange state.
//
// State layout in registers: the accumulator tiles hold S^T (rows = key index
// j, columns = value index i). Tile (mt, nt), lane (g = lane/16, m = lane%16),
// element e holds S[i = col0 + 16 nt + m][j = 16 mt + 4 g + e]. Any MFMA whose
// B operand is S^T (or U, or beta * R) is fed straight from such accumulators
// by listing the 32 reduction indices of a k-step in the order the
// accumulators hold them: B-slot s of lane group g stands for index
// 16 (s / 4) + 4 g + (s % 4); the matching A operand reads the same index
// order from LDS (two 8-byte reads). No state transpose goes through LDS.
#include "gdn_common.h"
#include "gdn_internal.h"

namespace gdn {

namespace {

constexpr int D = 128;
constexpr int RP = D + 8;          // padded bf16 row of a 64 x 128 tile
constexpr int CP = kChunk + 8;     // padded bf16 row of a 64 x 64 tile / a transposed K row
constexpr size_t kTBytes = kChunk * kChunk * 2;
constexpr size_t kPBytes = kChunk * kChunk * 2;
constexpr size_t kGamBytes = kChunk * 4;
constexpr size_t kSlotHeadBytes = kTBytes + kPBytes + kGamBytes;   // per (chunk slot, V head)

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
    return (uint32_t)float_to_bf16_bits(lo) | ((uint32_t)float_to_bf16_bits(hi) << 16);
}

// B operand from two accumulator tiles (reduction indices 32k + 4g + e and 32k + 16 + 4g + e).
__device__ __forceinline__ bf16x8 pack_acc_pair(f32x4 lo, f32x4 hi) {
    u32x4 u;
    u.x = pack_bf16(lo[0], lo[1]);
    u.y = pack_bf16(lo[2], lo[3]);
    u.z = pack_bf16(hi[0], hi[1]);
    u.w = pack_bf16(hi[2], hi[3]);
    return __builtin_bit_cast(bf16x8, u);
}

// A operand in the same index order: row `row` of a bf16 LDS tile, columns
// 32 k + 4 g .. +3 and 32 k + 16 + 4 g .. +3.
__device__ __forceinline__ bf16x8 lds_a_perm(const uint16_t* tile, int ld, int row, int k, int g) {
    const uint2 lo = *reinterpret_cast<const uint2*>(tile + row * ld + 32 * k + 4 * g);
    const uint2 hi = *reinterpret_cast<const uint2*>(tile + row * ld + 32 * k + 16 + 4 * g);
    u32x4 u;
    u.x = lo.x; u.y = lo.y; u.z = hi.x; u.w = hi.y;
    return __builtin_bit_cast(bf16x8, u);
}

// Standard-order operand: row `row`, columns 32 k + 8 g .. +7 (one 16-byte read).
__device__ __forceinline__ bf16x8 lds_row8(const uint16_t* tile, int ld, int row, int k, int g) {
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(tile + row * ld + 32 * k + 8 * g));
}

// Chunk slots: sequence n owns slots [f(n), f(n) + ceil(L_n / 64)) with
// f(n) = cu[n] / 64 + n. f is increasing and the ranges are disjoint, and
// every slot is below total_tokens / 64 + num_seqs, so the workspace can be
// sized on the host without reading the device offsets.
__device__ __forceinline__ int64_t slot_base(const int32_t* cu, int n) {
    return cu ? (int64_t)(cu[n] / kChunk) + n : 0;
}

struct SeqRange {
    int64_t bos, eos;
};

__device__ __forceinline__ SeqRange seq_range(const int32_t* cu, int n, int64_t total_tokens) {
    SeqRange r;
    r.bos = cu ? cu[n] : 0;
    r.eos = cu ? cu[n + 1] : total_tokens;
    return r;
}

// Largest n in [0, N) with slot_base(n) <= slot.
__device__ int find_seq_for_slot(const int32_t* cu, int N, int64_t slot) {
    if (!cu) return 0;
    int lo = 0, hi = N - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (slot_base(cu, mid) <= slot) lo = mid;
        else hi = mid - 1;
    }
    return lo;
}

// Cooperative load of a 64 x 128 bf16 tile (rows t0 .. t0 + nc - 1 of head `hd`
// in a [T, H, 128] array) into an LDS tile with padded rows; missing rows are 0.
__device__ __forceinline__ void load_tile_64x128(uint16_t* dst, const uint16_t* src, int64_t t0, int nc,
                                                 int heads, int hd, int tid) {
#pragma unroll
    for (int p = tid; p < kChunk * (D / 8); p += 256) {
        const int row = p >> 4, c8 = p & 15;
        u32x4 val = {0u, 0u, 0u, 0u};
        if (row < nc) val = *reinterpret_cast<const u32x4*>(src + ((t0 + row) * heads + hd) * D + c8 * 8);
        *reinterpret_cast<u32x4*>(dst + row * RP + c8 * 8) = val;
    }
}

struct PrepSmem {
    uint16_t K[kChunk][RP];
    uint16_t Q[kChunk][RP];
    float Gkk[kChunk][kChunk + 1];
    float Gqk[kChunk][kChunk + 1];
    float A[kChunk][kChunk + 1];
    float T[kChunk][kChunk + 1];
    float X[3][16][17];
    float graw[kChunk], gam[kChunk], bet[kChunk];
};

__global__ __launch_bounds__(256) void prep_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const float* __restrict__ g,
    const float* __restrict__ beta, const int32_t* __restrict__ cu, int32_t num_seqs, int64_t total_tokens,
    int32_t num_qk_heads, int32_t num_v_heads, uint8_t* __restrict__ ws) {
    __shared__ PrepSmem sm;
    const int64_t slot = blockIdx.x;
    const int hq = blockIdx.y;
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63, lg = lane >> 4, lm = lane & 15;

    const int n = find_seq_for_slot(cu, num_seqs, slot);
    const SeqRange sr = seq_range(cu, n, total_tokens);
    const int64_t c = slot - slot_base(cu, n);
    const int64_t t0 = sr.bos + c * kChunk;
    if (c < 0 || t0 >= sr.eos) return;   // slot not used by any sequence
    const int nc = (int)((sr.eos - t0) < kChunk ? (sr.eos - t0) : kChunk);

    load_tile_64x128(&sm.K[0][0], k, t0, nc, num_qk_heads, hq, tid);
    load_tile_64x128(&sm.Q[0][0], q, t0, nc, num_qk_heads, hq, tid);
    __syncthreads();

    // K K^T and Q K^T, lower block triangle (10 tiles each), 5 tiles per wave.
    for (int job = wave; job < 20; job += 4) {
        const int which = job / 10, ti = job % 10;
        const int mt = (ti >= 6) ? 3 : (ti >= 3) ? 2 : (ti >= 1) ? 1 : 0;
        const int nt = ti - mt * (mt + 1) / 2;
        const uint16_t* Asrc = which ? &sm.Q[0][0] : &sm.K[0][0];
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
            acc = mfma16(lds_row8(Asrc, RP, 16 * mt + lm, kk, lg), lds_row8(&sm.K[0][0], RP, 16 * nt + lm, kk, lg), acc);
        float(*G)[kChunk + 1] = which ? sm.Gqk : sm.Gkk;
#pragma unroll
        for (int e = 0; e < 4; ++e) G[16 * mt + 4 * lg + e][16 * nt + lm] = acc[e];
    }

    const int group = num_v_heads / num_qk_heads;
    for (int vh = 0; vh < group; ++vh) {
        const int hv = hq * group + vh;
        if (tid < kChunk) {
            const bool in = tid < nc;
            sm.graw[tid] = in ? g[(t0 + tid) * num_v_heads + hv] : 0.f;
            sm.bet[tid] = in ? beta[(t0 + tid) * num_v_heads + hv] : 0.f;
        }
        __syncthreads();
        if (tid < kChunk) {
            float acc = 0.f;
            for (int cc = 0; cc <= tid; ++cc) acc += sm.graw[cc];
            sm.gam[tid] = acc;
        }
        __syncthreads();
        uint8_t* base = ws + ((size_t)slot * num_v_heads + hv) * kSlotHeadBytes;
        uint16_t* Tout = reinterpret_cast<uint16_t*>(base);
        uint16_t* Pout = reinterpret_cast<uint16_t*>(base + kTBytes);
        float* gout = reinterpret_cast<float*>(base + kTBytes + kPBytes);
        for (int e = tid; e < kChunk * kChunk; e += 256) {
            const int r = e >> 6, cc = e & 63;
            float a = 0.f, p = 0.f;
            if (cc <= r) {
                const float dec = exp_nonpos(sm.gam[r] - sm.gam[cc]);
                p = dec * sm.Gqk[r][cc];
                if (cc < r) a = sm.bet[r] * dec * sm.Gkk[r][cc];
            }
            sm.A[r][cc] = a;
            sm.T[r][cc] = 0.f;
            Pout[e] = float_to_bf16_bits(p);
        }
        if (tid < kChunk) gout[tid] = sm.gam[tid];
        __syncthreads();
        // Diagonal 16 x 16 blocks: lane = 16 b + col, forward substitution on its column.
        if (wave == 0) {
            const int b = lg, col = lm;
            float t[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float acc = 0.f;
#pragma unroll
                for (int j = 0; j < r; ++j) acc = fmaf(sm.A[16 * b + r][16 * b + j], t[j], acc);
                t[r] = (r == col ? 1.f : 0.f) - acc;
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) sm.T[16 * b + r][16 * b + col] = t[r];
        }
        __syncthreads();
        // Off-diagonal blocks, by distance from the diagonal:
        // T[bi][bj] = -T[bi][bi] * (A[bi rows][16 bj : 16 bi] * T[16 bj : 16 bi][bj cols]).
        for (int lev = 1; lev < 4; ++lev) {
            const int nblk = 4 - lev;
            for (int e = tid; e < nblk * 256; e += 256) {
                const int bj = e >> 8, ii = (e >> 4) & 15, jj = e & 15;
                const int bi = bj + lev;
                float acc = 0.f;
                for (int kk = 16 * bj; kk < 16 * bi; ++kk) acc = fmaf(sm.A[16 * bi + ii][kk], sm.T[kk][16 * bj + jj], acc);
                sm.X[bj][ii][jj] = acc;
            }
            __syncthreads();
            for (int e = tid; e < nblk * 256; e += 256) {
                const int bj = e >> 8, ii = (e >> 4) & 15, jj = e & 15;
                const int bi = bj + lev;
                float acc = 0.f;
#pragma unroll
                for (int kk = 0; kk < 16; ++kk) acc = fmaf(sm.T[16 * bi + ii][16 * bi + kk], sm.X[bj][kk][jj], acc);
                sm.T[16 * bi + ii][16 * bj + jj] = -acc;
            }
            __syncthreads();
        }
        for (int e = tid; e < kChunk * kChunk; e += 256) Tout[e] = float_to_bf16_bits(sm.T[e >> 6][e & 63]);
        __syncthreads();
    }
}

template <int NW>
struct ChainSmem {
    uint16_t K[kChunk][RP];
    uint16_t KT[D][CP];
    uint16_t Q[kChunk][RP];
    uint16_t T[kChunk][CP];
    uint16_t P[kChunk][CP];
    uint16_t V[kChunk][64 * NW + 8];
    float gam[kChunk], bet[kChunk];
};

// NW = value-column tiles (16 wide) per wave; a workgroup covers 64 * NW columns.
template <int NW>
__global__ __launch_bounds__(256) void chain_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const float* __restrict__ beta, const float* initial_state, const int32_t* __restrict__ cu,
    float* final_state, uint16_t* __restrict__ out, const uint8_t* __restrict__ ws, int64_t total_tokens,
    int32_t num_qk_heads, int32_t num_v_heads, float scale) {
    constexpr int NSPLIT = D / (64 * NW);
    constexpr int VW = 64 * NW;   // value columns per workgroup
    __shared__ ChainSmem<NW> sm;

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63, lg = lane >> 4, lm = lane & 15;
    const int split = blockIdx.x % NSPLIT;
    const int h = (blockIdx.x / NSPLIT) % num_v_heads;
    const int n = blockIdx.x / (NSPLIT * num_v_heads);
    const int hq = h / (num_v_heads / num_qk_heads);
    const int colw = wave * 16 * NW;         // first value column of this wave inside the WG tile
    const int col0 = split * VW + colw;      // first value column of this wave in the head
    const SeqRange sr = seq_range(cu, n, total_tokens);
    const int64_t sb = slot_base(cu, n);

    f32x4 ST[8][NW];
    const int64_t sbase = ((int64_t)n * num_v_heads + h) * D * D;
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
#pragma unroll
        for (int nt = 0; nt < NW; ++nt) {
            f32x4 s = {0.f, 0.f, 0.f, 0.f};
            if (initial_state)
                s = *reinterpret_cast<const f32x4*>(initial_state + sbase + (int64_t)(col0 + 16 * nt + lm) * D + 16 * mt + 4 * lg);
            ST[mt][nt] = s;
        }

    int64_t c = 0;
    for (int64_t t0 = sr.bos; t0 < sr.eos; t0 += kChunk, ++c) {
        const int nc = (int)((sr.eos - t0) < kChunk ? (sr.eos - t0) : kChunk);
        const uint8_t* base = ws + ((size_t)(sb + c) * num_v_heads + h) * kSlotHeadBytes;
        // ---- stage the chunk in LDS
        load_tile_64x128(&sm.Q[0][0], q, t0, nc, num_qk_heads, hq, tid);
#pragma unroll
        for (int p = tid; p < kChunk * (D / 8); p += 256) {
            const int row = p >> 4, c8 = p & 15;
            u32x4 val = {0u, 0u, 0u, 0u};
            if (row < nc) val = *reinterpret_cast<const u32x4*>(k + ((t0 + row) * num_qk_heads + hq) * D + c8 * 8);
            *reinterpret_cast<u32x4*>(&sm.K[row][c8 * 8]) = val;
#pragma unroll
            for (int s = 0; s < 8; ++s)
                sm.KT[c8 * 8 + s][row] = (uint16_t)((s & 1) ? (val[s >> 1] >> 16) : (val[s >> 1] & 0xFFFFu));
        }
        for (int p = tid; p < kChunk * kChunk / 8; p += 256) {
            const int row = p >> 3, c8 = p & 7;
            *reinterpret_cast<u32x4*>(&sm.T[row][c8 * 8]) = reinterpret_cast<const u32x4*>(base)[p];
            *reinterpret_cast<u32x4*>(&sm.P[row][c8 * 8]) = reinterpret_cast<const u32x4*>(base + kTBytes)[p];
        }
        for (int p = tid; p < kChunk * VW / 8; p += 256) {
            const int row = p / (VW / 8), c8 = p % (VW / 8);
            u32x4 val = {0u, 0u, 0u, 0u};
            if (row < nc) val = *reinterpret_cast<const u32x4*>(v + ((t0 + row) * num_v_heads + h) * D + split * VW + c8 * 8);
            *reinterpret_cast<u32x4*>(&sm.V[row][c8 * 8]) = val;
        }
        if (tid < kChunk) {
            sm.gam[tid] = reinterpret_cast<const float*>(base + kTBytes + kPBytes)[tid];
            sm.bet[tid] = tid < nc ? beta[(t0 + tid) * num_v_heads + h] : 0.f;
        }
        __syncthreads();

        // ---- Z = K S0^T and Y = Q S0^T (64 tokens x this wave's value columns)
        bf16x8 Sb[4][NW];
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
#pragma unroll
            for (int nt = 0; nt < NW; ++nt) Sb[kk][nt] = pack_acc_pair(ST[2 * kk][nt], ST[2 * kk + 1][nt]);
        f32x4 Z[4][NW], Y[4][NW];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
            for (int nt = 0; nt < NW; ++nt) {
                Z[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
                Y[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                const bf16x8 ak = lds_a_perm(&sm.K[0][0], RP, 16 * mt + lm, kk, lg);
                const bf16x8 aq = lds_a_perm(&sm.Q[0][0], RP, 16 * mt + lm, kk, lg);
#pragma unroll
                for (int nt = 0; nt < NW; ++nt) {
                    Z[mt][nt] = mfma16(ak, Sb[kk][nt], Z[mt][nt]);
                    Y[mt][nt] = mfma16(aq, Sb[kk][nt], Y[mt][nt]);
                }
            }
        }
        // ---- beta * R = beta * (V - Gamma * Z); U = Tm (beta R)
        f32x4 BR[4][NW];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 16 * mt + 4 * lg + e;
                const float Gr = exp_nonpos(sm.gam[r]);
                const float br = sm.bet[r];
#pragma unroll
                for (int nt = 0; nt < NW; ++nt) {
                    const float vv = bf16_bits_to_float(sm.V[r][colw + 16 * nt + lm]);
                    BR[mt][nt][e] = br * (vv - Gr * Z[mt][nt][e]);
                }
            }
        bf16x8 Bb[2][NW];
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
            for (int nt = 0; nt < NW; ++nt) Bb[kk][nt] = pack_acc_pair(BR[2 * kk][nt], BR[2 * kk + 1][nt]);
        f32x4 U[4][NW];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
            for (int nt = 0; nt < NW; ++nt) U[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk <= mt / 2; ++kk) {
                const bf16x8 at = lds_a_perm(&sm.T[0][0], CP, 16 * mt + lm, kk, lg);
#pragma unroll
                for (int nt = 0; nt < NW; ++nt) U[mt][nt] = mfma16(at, Bb[kk][nt], U[mt][nt]);
            }
        }
        // ---- O = scale (Gamma * Y + P U)
        bf16x8 Ub[2][NW];
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
            for (int nt = 0; nt < NW; ++nt) Ub[kk][nt] = pack_acc_pair(U[2 * kk][nt], U[2 * kk + 1][nt]);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
            f32x4 O[NW];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float Gr = exp_nonpos(sm.gam[16 * mt + 4 * lg + e]);
#pragma unroll
                for (int nt = 0; nt < NW; ++nt) O[nt][e] = Gr * Y[mt][nt][e];
            }
#pragma unroll
            for (int kk = 0; kk <= mt / 2; ++kk) {
                const bf16x8 ap = lds_a_perm(&sm.P[0][0], CP, 16 * mt + lm, kk, lg);
#pragma unroll
                for (int nt = 0; nt < NW; ++nt) O[nt] = mfma16(ap, Ub[kk][nt], O[nt]);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 16 * mt + 4 * lg + e;
                if (r < nc) {
#pragma unroll
                    for (int nt = 0; nt < NW; ++nt)
                        out[((t0 + r) * num_v_heads + h) * D + col0 + 16 * nt + lm] = float_to_bf16_bits(scale * O[nt][e]);
                }
            }
        }
        // ---- S = Gamma_last S0 + U^T diag(exp(gamma_last - gamma)) K  (as S^T += K^T U')
        const float glast = sm.gam[kChunk - 1];
        bf16x8 Wb[2][NW];
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            f32x4 lo[NW], hi[NW];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float dlo = exp_nonpos(glast - sm.gam[32 * kk + 4 * lg + e]);
                const float dhi = exp_nonpos(glast - sm.gam[32 * kk + 16 + 4 * lg + e]);
#pragma unroll
                for (int nt = 0; nt < NW; ++nt) {
                    lo[nt][e] = dlo * U[2 * kk][nt][e];
                    hi[nt][e] = dhi * U[2 * kk + 1][nt][e];
                }
            }
#pragma unroll
            for (int nt = 0; nt < NW; ++nt) Wb[kk][nt] = pack_acc_pair(lo[nt], hi[nt]);
        }
        const float Glast = exp_nonpos(glast);
#pragma unroll
        for (int mt = 0; mt < 8; ++mt) {
#pragma unroll
            for (int nt = 0; nt < NW; ++nt) ST[mt][nt] *= Glast;
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                const bf16x8 akt = lds_a_perm(&sm.KT[0][0], CP, 16 * mt + lm, kk, lg);
#pragma unroll
                for (int nt = 0; nt < NW; ++nt) ST[mt][nt] = mfma16(akt, Wb[kk][nt], ST[mt][nt]);
            }
        }
        __syncthreads();
    }

    if (final_state) {
#pragma unroll
        for (int mt = 0; mt < 8; ++mt)
#pragma unroll
            for (int nt = 0; nt < NW; ++nt)
                *reinterpret_cast<f32x4*>(final_state + sbase + (int64_t)(col0 + 16 * nt + lm) * D + 16 * mt + 4 * lg) = ST[mt][nt];
    }
}

}  // namespace

size_t prefill_bf16_workspace_bytes(int64_t total_tokens, int32_t num_seqs, int32_t num_qk_heads,
                                    int32_t num_v_heads) {
    (void)num_qk_heads;
    const int64_t slots = total_tokens / kChunk + num_seqs;
    return (size_t)slots * (size_t)num_v_heads * kSlotHeadBytes;
}

hipError_t launch_prefill_bf16(const PrefillArgs& a, hipStream_t stream) {
    const int64_t slots = a.total_tokens / kChunk + a.num_seqs;
    uint8_t* ws = static_cast<uint8_t*>(a.workspace);
    if (a.total_tokens > 0) {
        prof::begin(stream, "gdn_chunk_prep");
        hipLaunchKernelGGL(prep_kernel, dim3((unsigned)slots, (unsigned)a.num_qk_heads), dim3(256), 0, stream,
                           (const uint16_t*)a.q, (const uint16_t*)a.k, a.g, a.beta, a.cu_seqlens, a.num_seqs,
                           a.total_tokens, a.num_qk_heads, a.num_v_heads, ws);
        prof::end(stream);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    // Fewer than ~2 workgroups per CU with whole heads: split the value columns in two.
    const int64_t units = (int64_t)a.num_seqs * a.num_v_heads;
    prof::begin(stream, "gdn_chunk_chain");
    if (units >= 512) {
        hipLaunchKernelGGL((chain_kernel<2>), dim3((unsigned)units), dim3(256), 0, stream,
                           (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v, a.beta,
                           a.initial_state, a.cu_seqlens, a.final_state, (uint16_t*)a.out, ws, a.total_tokens,
                           a.num_qk_heads, a.num_v_heads, a.scale);
    } else {
        hipLaunchKernelGGL((chain_kernel<1>), dim3((unsigned)(units * 2)), dim3(256), 0, stream,
                           (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v, a.beta,
                           a.initial_state, a.cu_seqlens, a.final_state, (uint16_t*)a.out, ws, a.total_tokens,
                           a.num_qk_heads, a.num_v_heads, a.scale);
    }
    prof::end(stream);
    return hipGetLastError();
}

}  // namespace gdn
