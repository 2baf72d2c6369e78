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

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Two floats -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
    const f32x2 x = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf16x2));
}

// exp(x) for x <= 0 with the raw hardware exp2 (results below 2^-126 may flush to 0).
__device__ __forceinline__ float fast_exp(float x) { return __builtin_amdgcn_exp2f(x * 1.4426950408889634f); }

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

// Prep: one workgroup per (chunk slot, QK head) and its group of V heads
// (at most kMaxGroup; larger groups loop). LDS holds K and Q while the Gram
// products run, then the same bytes hold Tm; A and the level scratch have
// their own space, so two workgroups fit on a CU.
constexpr int kMaxGroup = 2;

struct PrepSmem {
    union {
        struct {
            uint16_t K[kChunk][RP];
            uint16_t Q[kChunk][RP];
        } kq;
        float T[kMaxGroup][kChunk][kChunk + 1];
    } u;
    float A[kMaxGroup][kChunk][kChunk + 1];
    float X[kMaxGroup][3][16][17];
    float gam[kMaxGroup][kChunk], bet[kMaxGroup][kChunk];
};

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ float wave_inclusive_scan(float x, int lane) {
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const float y = __shfl_up(x, d, 64);
        if (lane >= d) x += y;
    }
    return x;
}

// Off-diagonal blocks at distance L from the diagonal, for every head of the
// group: T[bi][bj] = -T[bi][bi] (A[bi rows][16 bj : 16 bi] T[16 bj : 16 bi][bj cols]).
template <int L>
__device__ __forceinline__ void tsolve_level(PrepSmem& sm, int nh, int tid) {
    constexpr int NB = 4 - L;
    for (int e = tid; e < nh * NB * 256; e += 256) {
        const int hh = e / (NB * 256), bj = (e >> 8) % NB, ii = (e >> 4) & 15, jj = e & 15;
        const int bi = bj + L;
        const float* arow = &sm.A[hh][16 * bi + ii][16 * bj];
        float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < 16 * L; ++kk) acc[kk & 3] = fmaf(arow[kk], sm.u.T[hh][16 * bj + kk][16 * bj + jj], acc[kk & 3]);
        sm.X[hh][bj][ii][jj] = (acc[0] + acc[1]) + (acc[2] + acc[3]);
    }
    __syncthreads();
    for (int e = tid; e < nh * NB * 256; e += 256) {
        const int hh = e / (NB * 256), bj = (e >> 8) % NB, ii = (e >> 4) & 15, jj = e & 15;
        const int bi = bj + L;
        float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < 16; ++kk) acc[kk & 3] = fmaf(sm.u.T[hh][16 * bi + ii][16 * bi + kk], sm.X[hh][bj][kk][jj], acc[kk & 3]);
        sm.u.T[hh][16 * bi + ii][16 * bj + jj] = -((acc[0] + acc[1]) + (acc[2] + acc[3]));
    }
    __syncthreads();
}

__global__ __launch_bounds__(256, 2) void prep_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const float* __restrict__ g,
    const float* __restrict__ beta, const int32_t* __restrict__ cu, int32_t num_seqs, int64_t total_tokens,
    int32_t num_qk_heads, int32_t num_v_heads, uint8_t* __restrict__ ws) {
    __shared__ PrepSmem sm;
    const int64_t slot = blockIdx.x;
    const int hq = blockIdx.y;
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, lg = lane >> 4, lm = lane & 15;

    const int n = find_seq_for_slot(cu, num_seqs, slot);
    const SeqRange sr = seq_range(cu, n, total_tokens);
    const int64_t c = slot - slot_base(cu, n);
    const int64_t t0 = sr.bos + c * kChunk;
    if (c < 0 || t0 >= sr.eos) return;   // slot not used by any sequence
    const int nc = (int)((sr.eos - t0) < kChunk ? (sr.eos - t0) : kChunk);
    const int group = num_v_heads / num_qk_heads;

    load_tile_64x128(&sm.u.kq.K[0][0], k, t0, nc, num_qk_heads, hq, tid);
    load_tile_64x128(&sm.u.kq.Q[0][0], q, t0, nc, num_qk_heads, hq, tid);

    for (int h0 = 0; h0 < group; h0 += kMaxGroup) {
        const int nh = (group - h0) < kMaxGroup ? (group - h0) : kMaxGroup;
        if (h0 > 0) {   // later head pairs: K and Q again (their LDS held Tm)
            __syncthreads();
            load_tile_64x128(&sm.u.kq.K[0][0], k, t0, nc, num_qk_heads, hq, tid);
            load_tile_64x128(&sm.u.kq.Q[0][0], q, t0, nc, num_qk_heads, hq, tid);
        }
        // gamma (in-chunk cumulative g) and beta; padded rows have g = beta = 0.
        if (wave < nh) {
            const int hv = hq * group + h0 + wave;
            const bool in = lane < nc;
            const float gl = in ? g[(t0 + lane) * num_v_heads + hv] : 0.f;
            const float gm = wave_inclusive_scan(gl, lane);
            sm.gam[wave][lane] = gm;
            sm.bet[wave][lane] = in ? beta[(t0 + lane) * num_v_heads + hv] : 0.f;
            uint8_t* base = ws + ((size_t)slot * num_v_heads + hv) * kSlotHeadBytes;
            reinterpret_cast<float*>(base + kTBytes + kPBytes)[lane] = gm;
        }
        __syncthreads();

        // Gram tiles (lower block triangle) by MFMA, masked straight into A (LDS) and P (workspace).
        for (int job = wave; job < 20; job += 4) {
            const int which = job / 10, ti = job % 10;
            const int mt = (ti >= 6) ? 3 : (ti >= 3) ? 2 : (ti >= 1) ? 1 : 0;
            const int nt = ti - mt * (mt + 1) / 2;
            const uint16_t* Asrc = which ? &sm.u.kq.Q[0][0] : &sm.u.kq.K[0][0];
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < 4; ++kk)
                acc = mfma16(lds_row8(Asrc, RP, 16 * mt + lm, kk, lg), lds_row8(&sm.u.kq.K[0][0], RP, 16 * nt + lm, kk, lg), acc);
            const int cc = 16 * nt + lm;
            for (int hh = 0; hh < nh; ++hh) {
                const float gc = sm.gam[hh][cc];
                uint16_t* Pout = reinterpret_cast<uint16_t*>(
                    ws + ((size_t)slot * num_v_heads + hq * group + h0 + hh) * kSlotHeadBytes + kTBytes);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = 16 * mt + 4 * lg + e;
                    const float dec = (cc <= r) ? fast_exp(sm.gam[hh][r] - gc) : 0.f;
                    if (which) Pout[r * kChunk + cc] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(dec * acc[e]));
                    else sm.A[hh][r][cc] = (cc < r) ? sm.bet[hh][r] * dec * acc[e] : 0.f;
                }
            }
        }
        // Upper block triangle of P is zero.
        for (int e = tid; e < nh * 6 * 256; e += 256) {
            const int hh = e / 1536, ti = (e >> 8) % 6, ii = (e >> 4) & 15, jj = e & 15;
            const int nt = (ti >= 3) ? 3 : (ti >= 1) ? 2 : 1;          // (0,1) (0,2) (1,2) (0,3) (1,3) (2,3)
            const int mt = ti - (nt * (nt - 1)) / 2;
            uint16_t* Pout = reinterpret_cast<uint16_t*>(
                ws + ((size_t)slot * num_v_heads + hq * group + h0 + hh) * kSlotHeadBytes + kTBytes);
            Pout[(16 * mt + ii) * kChunk + 16 * nt + jj] = 0;
        }
        __syncthreads();   // A complete; K and Q no longer needed

        // Diagonal 16 x 16 blocks of Tm, one wave per head: lane = 16 b + col holds
        // column col of block b and substitutes down its 16 rows.
        if (wave < nh) {
            const int b = lg, col = lm;
            float t[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float* arow = &sm.A[wave][16 * b + r][16 * b];
                float p0 = 0.f, p1 = 0.f, p2 = 0.f, p3 = 0.f;
#pragma unroll
                for (int j = 0; j < r; ++j) {
                    const float term = arow[j] * t[j];
                    if ((j & 3) == 0) p0 += term;
                    else if ((j & 3) == 1) p1 += term;
                    else if ((j & 3) == 2) p2 += term;
                    else p3 += term;
                }
                t[r] = (r == col ? 1.f : 0.f) - ((p0 + p1) + (p2 + p3));
            }
            for (int r = 0; r < 64; ++r) sm.u.T[wave][r][lane] = 0.f;
#pragma unroll
            for (int r = 0; r < 16; ++r) sm.u.T[wave][16 * b + r][16 * b + col] = t[r];
        }
        __syncthreads();
        tsolve_level<1>(sm, nh, tid);
        tsolve_level<2>(sm, nh, tid);
        tsolve_level<3>(sm, nh, tid);
        // Tm as bf16 (rows of 8 values per 16-byte store).
        for (int e = tid; e < nh * kChunk * 8; e += 256) {
            const int hh = e >> 9, r = (e >> 3) & 63, c8 = e & 7;
            uint16_t* Tout = reinterpret_cast<uint16_t*>(ws + ((size_t)slot * num_v_heads + hq * group + h0 + hh) * kSlotHeadBytes);
            u32x4 u;
#pragma unroll
            for (int s2 = 0; s2 < 4; ++s2) u[s2] = pack_bf16(sm.u.T[hh][r][8 * c8 + 2 * s2], sm.u.T[hh][r][8 * c8 + 2 * s2 + 1]);
            *reinterpret_cast<u32x4*>(Tout + r * kChunk + 8 * c8) = u;
        }
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


// ---------------------------------------------------------------------------
// Chain kernel for few (sequence, head) pairs: each workgroup owns 16 value
// columns of one head (8 workgroups per head). Per chunk every wave computes
// Z = K S^T and U = Tm (beta R) for all 64 tokens (redundantly, in registers,
// so no exchange is needed for them), then its own share of the rest: the
// output rows of token tile w, and the state's key rows 32 w .. 32 w + 31.
// The only exchange is the bf16 copy of S in LDS, so a chunk costs one
// barrier. The next chunk's operands are loaded into registers during the
// chunk and written to the other half of a double buffer before the barrier;
// the new bf16 S goes to the other half of its own double buffer.
struct SliceBuf {
    uint16_t K[kChunk][RP];
    uint16_t Q[kChunk][RP];
    uint16_t T[kChunk][CP];
    uint16_t P[kChunk][CP];
    uint16_t Vt[16][CP];   // V of the 16 value columns, [value col][token]
    float Gam[kChunk];     // exp(gamma_r)
    float Dec[kChunk];     // exp(gamma_last - gamma_r)
    float bet[kChunk];
};

struct SliceSmem {
    SliceBuf buf[2];
    uint16_t SBt[2][16][D + 8];   // bf16 S for the 16 value columns: [value col][key index], double-buffered
};

struct SlicePrefetch {
    u32x4 k[4], q[4], t[2], p[2], v;
    float s;
};

// Per-thread, chunk-invariant offsets of the staging loads.
struct SliceOffsets {
    int k[4];      // element offset inside a chunk of q / k (row * ldk + col)
    int v;         // element offset inside a chunk of v (waves 0-1)
    int s;         // gamma index (wave 2) or beta row offset (waves 0, 1, 3)
};

__device__ __forceinline__ void slice_fetch(SlicePrefetch& pf, const SliceOffsets& o, const uint16_t* kc,
                                            const uint16_t* qc, const uint16_t* vc, const float* sc,
                                            const uint8_t* base, int tid) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        pf.k[i] = *reinterpret_cast<const u32x4*>(kc + o.k[i]);
        pf.q[i] = *reinterpret_cast<const u32x4*>(qc + o.k[i]);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        pf.t[i] = reinterpret_cast<const u32x4*>(base)[tid + 256 * i];
        pf.p[i] = reinterpret_cast<const u32x4*>(base + kTBytes)[tid + 256 * i];
    }
    pf.v = *reinterpret_cast<const u32x4*>(vc + o.v);
    pf.s = sc[o.s];
}

// Offsets for a chunk of nc tokens; rows past nc re-read row nc - 1 (they are
// zeroed when stored), so no load leaves the sequence.
__device__ __forceinline__ SliceOffsets slice_offsets(int nc, int tid, int w, int ldk, int ldv, int num_v_heads) {
    SliceOffsets o;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int p = tid + 256 * i, row = p >> 4;
        o.k[i] = (row < nc ? row : nc - 1) * ldk + (p & 15) * 8;
    }
    const int vrow = (tid & 127) >> 1;
    o.v = (vrow < nc ? vrow : nc - 1) * ldv + 8 * (tid & 1);
    const int r = tid & 63;
    o.s = (w == 2) ? r : (r < nc ? r : nc - 1) * num_v_heads;
    return o;
}

__device__ __forceinline__ void slice_store(SliceBuf& b, const SlicePrefetch& pf, int nc, int tid, int w) {
    const u32x4 z = {0u, 0u, 0u, 0u};
    const bool full = nc == kChunk;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int p = tid + 256 * i, row = p >> 4, c8 = p & 15;
        const bool in = full || row < nc;
        *reinterpret_cast<u32x4*>(&b.K[row][c8 * 8]) = in ? pf.k[i] : z;
        *reinterpret_cast<u32x4*>(&b.Q[row][c8 * 8]) = in ? pf.q[i] : z;
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int p = tid + 256 * i, row = p >> 3, c8 = p & 7;
        *reinterpret_cast<u32x4*>(&b.T[row][c8 * 8]) = pf.t[i];
        *reinterpret_cast<u32x4*>(&b.P[row][c8 * 8]) = pf.p[i];
    }
    if (w < 2) {
        const int row = tid >> 1, c0 = 8 * (tid & 1);
        const u32x4 val = (full || row < nc) ? pf.v : z;
#pragma unroll
        for (int s = 0; s < 8; ++s)
            b.Vt[c0 + s][row] = (uint16_t)((s & 1) ? (val[s >> 1] >> 16) : (val[s >> 1] & 0xFFFFu));
    } else if (w == 2) {
        // gamma of padded rows repeats the last real value (g = 0 there).
        const float glast = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, pf.s), 63));
        b.Gam[tid - 128] = fast_exp(pf.s);
        b.Dec[tid - 128] = fast_exp(glast - pf.s);
    } else {
        b.bet[tid - 192] = (full || (tid - 192) < nc) ? pf.s : 0.f;
    }
}

// A operand of K^T for key-row tile t and token k-step kk, in the accumulator
// order of U (token 32 kk + 16 (s / 4) + 4 g + (s % 4) for slot s).
__device__ __forceinline__ bf16x8 lds_kt_perm(const uint16_t (*K)[RP], int t, int kk, int g, int m) {
    u32x4 u;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        const int r = 32 * kk + 16 * (s >> 1) + 4 * g + 2 * (s & 1);
        u[s] = (uint32_t)K[r][16 * t + m] | ((uint32_t)K[r + 1][16 * t + m] << 16);
    }
    return __builtin_bit_cast(bf16x8, u);
}

__device__ __forceinline__ void store_bf16x4(uint16_t* dst, f32x4 x) {
    uint2 w;
    w.x = pack_bf16(x[0], x[1]);
    w.y = pack_bf16(x[2], x[3]);
    *reinterpret_cast<uint2*>(dst) = w;
}

__device__ __forceinline__ f32x4 unpack_bf16x4(uint2 u) {
    f32x4 r;
    r[0] = __uint_as_float(u.x << 16);
    r[1] = __uint_as_float(u.x & 0xFFFF0000u);
    r[2] = __uint_as_float(u.y << 16);
    r[3] = __uint_as_float(u.y & 0xFFFF0000u);
    return r;
}

__global__ __launch_bounds__(256) void chain_slice_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const float* __restrict__ beta, const float* initial_state, const int32_t* __restrict__ cu,
    float* final_state, uint16_t* __restrict__ out, const uint8_t* __restrict__ ws, int64_t total_tokens,
    int32_t num_seqs, int32_t num_qk_heads, int32_t num_v_heads, float scale) {
    __shared__ SliceSmem sm;
    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index, kept in a scalar register
    const int lane = tid & 63, g = lane >> 4, m = lane & 15;
    // XCD-aware placement: workgroups are dealt round-robin to the 8 XCDs
    // (bid % 8), each with its own L2. All 8 * group workgroups of one
    // (sequence, QK head) group - which read the same K, Q and, per V head, the
    // same Tm, P - are placed on the XCD (group index) % 8.
    const int group = num_v_heads / num_qk_heads;
    const int per = 8 * group;                          // workgroups per (sequence, QK head)
    const int xcd = blockIdx.x & 7;
    const int kx = blockIdx.x >> 3;
    const int sidx = kx % per;
    const int64_t qg = 8 * (int64_t)(kx / per) + xcd;   // (sequence, QK head) group index
    if (qg >= (int64_t)num_seqs * num_qk_heads) return;
    const int n = (int)(qg / num_qk_heads);
    const int hq = (int)(qg % num_qk_heads);
    const int h = hq * group + sidx / 8;
    const int col0 = 16 * (sidx & 7);                   // first value column of this slice
    const SeqRange sr = seq_range(cu, n, total_tokens);
    const int64_t sb = slot_base(cu, n);
    const int64_t nch = (sr.eos - sr.bos + kChunk - 1) / kChunk;
    const int ldk = num_qk_heads * D, ldv = num_v_heads * D;

    // State: this wave's key rows 32 w .. 32 w + 31 (tiles 2w, 2w+1) for value columns col0 .. col0+15.
    f32x4 ST[2];
    const int64_t sbase = ((int64_t)n * num_v_heads + h) * D * D;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int t = 2 * w + i;
        f32x4 s = {0.f, 0.f, 0.f, 0.f};
        if (initial_state)
            s = *reinterpret_cast<const f32x4*>(initial_state + sbase + (int64_t)(col0 + m) * D + 16 * t + 4 * g);
        ST[i] = s;
        store_bf16x4(&sm.SBt[0][m][16 * t + 4 * g], s);
    }

    auto fetch = [&](SlicePrefetch& pf, int64_t c, int nc) {
        const int64_t t0 = sr.bos + c * kChunk;
        const uint8_t* base = ws + ((size_t)(sb + c) * num_v_heads + h) * kSlotHeadBytes;
        const float* sc = (w == 2) ? reinterpret_cast<const float*>(base + kTBytes + kPBytes)
                                   : beta + t0 * num_v_heads + h;
        const SliceOffsets o = slice_offsets(nc, tid, w, ldk, ldv, num_v_heads);
        slice_fetch(pf, o, k + t0 * ldk + hq * D, q + t0 * ldk + hq * D, v + t0 * ldv + h * D + col0, sc, base, tid);
    };

    SlicePrefetch pf;
    if (nch > 0) {
        const int nc0 = (int)((sr.eos - sr.bos) < kChunk ? (sr.eos - sr.bos) : kChunk);
        fetch(pf, 0, nc0);
        slice_store(sm.buf[0], pf, nc0, tid, w);
    }
    __syncthreads();

    for (int64_t c = 0; c < nch; ++c) {
        const SliceBuf& b = sm.buf[c & 1];
        const int64_t t0 = sr.bos + c * kChunk;
        const int nc = (int)((sr.eos - t0) < kChunk ? (sr.eos - t0) : kChunk);
        // The fetch and its store are unconditional (the last chunk re-reads
        // itself into the unused buffer) so that no load is outstanding on
        // any path into the next iteration.
        const bool more = c + 1 < nch;
        const int64_t c1 = more ? c + 1 : c;
        const int nc1 = more ? (int)((sr.eos - t0 - kChunk) < kChunk ? (sr.eos - t0 - kChunk) : kChunk) : nc;
        fetch(pf, c1, nc1);

        // Z = K S^T for all tokens, Y = Q S^T for token tile w.
        bf16x8 sbop[4];
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) sbop[kk] = lds_row8(&sm.SBt[c & 1][0][0], D + 8, m, kk, g);
        f32x4 Z[4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
            Z[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) Z[mt] = mfma16(lds_row8(&b.K[0][0], RP, 16 * mt + m, kk, g), sbop[kk], Z[mt]);
        }
        f32x4 Y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) Y = mfma16(lds_row8(&b.Q[0][0], RP, 16 * w + m, kk, g), sbop[kk], Y);

        // beta R = beta (V - Gamma Z), all tokens, as B operands in accumulator order.
        f32x4 BR[4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
            const int r = 16 * mt + 4 * g;
            const f32x4 Gr = *reinterpret_cast<const f32x4*>(&b.Gam[r]);
            const f32x4 Br = *reinterpret_cast<const f32x4*>(&b.bet[r]);
            const f32x4 Vv = unpack_bf16x4(*reinterpret_cast<const uint2*>(&b.Vt[m][r]));
            BR[mt] = Br * (Vv - Gr * Z[mt]);
        }
        const bf16x8 Bb0 = pack_acc_pair(BR[0], BR[1]), Bb1 = pack_acc_pair(BR[2], BR[3]);
        // U = Tm (beta R): token tiles 0, 1 need reduction step 0 only (Tm is lower triangular).
        f32x4 U[4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
            U[mt] = mfma16(lds_a_perm(&b.T[0][0], CP, 16 * mt + m, 0, g), Bb0, f32x4{0.f, 0.f, 0.f, 0.f});
            if (mt >= 2) U[mt] = mfma16(lds_a_perm(&b.T[0][0], CP, 16 * mt + m, 1, g), Bb1, U[mt]);
        }
        const bf16x8 Ub0 = pack_acc_pair(U[0], U[1]), Ub1 = pack_acc_pair(U[2], U[3]);
        f32x4 Ud[4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) Ud[mt] = *reinterpret_cast<const f32x4*>(&b.Dec[16 * mt + 4 * g]) * U[mt];
        const bf16x8 Udb0 = pack_acc_pair(Ud[0], Ud[1]), Udb1 = pack_acc_pair(Ud[2], Ud[3]);

        // State rows of this wave: S^T = Gamma_last S^T + K^T U'.
        const float Glast = b.Gam[kChunk - 1];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int t = 2 * w + i;
            f32x4 acc = ST[i] * Glast;
            acc = mfma16(lds_kt_perm(b.K, t, 0, g, m), Udb0, acc);
            acc = mfma16(lds_kt_perm(b.K, t, 1, g, m), Udb1, acc);
            ST[i] = acc;
        }
        // Output rows of this wave: O = scale (Gamma Y + P U).
        f32x4 O = *reinterpret_cast<const f32x4*>(&b.Gam[16 * w + 4 * g]) * Y;
        O = mfma16(lds_a_perm(&b.P[0][0], CP, 16 * w + m, 0, g), Ub0, O);
        if (w >= 2) O = mfma16(lds_a_perm(&b.P[0][0], CP, 16 * w + m, 1, g), Ub1, O);

#pragma unroll
        for (int i = 0; i < 2; ++i) store_bf16x4(&sm.SBt[(c + 1) & 1][m][16 * (2 * w + i) + 4 * g], ST[i]);
        uint16_t* orow = out + (t0 + 16 * w + 4 * g) * ldv + h * D + col0 + m;
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if (nc == kChunk || 16 * w + 4 * g + e < nc)
                orow[e * ldv] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(scale * O[e]));
        slice_store(sm.buf[(c + 1) & 1], pf, nc1, tid, w);
        __syncthreads();
    }

    if (final_state) {
#pragma unroll
        for (int i = 0; i < 2; ++i)
            *reinterpret_cast<f32x4*>(final_state + sbase + (int64_t)(col0 + m) * D + 16 * (2 * w + i) + 4 * g) = ST[i];
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
    // Whole-head workgroups only when there are enough (sequence, head) pairs to
    // fill the chip; otherwise 8 workgroups per head, 16 value columns each.
    const int64_t units = (int64_t)a.num_seqs * a.num_v_heads;
    prof::begin(stream, "gdn_chunk_chain");
    if (units >= 512) {
        hipLaunchKernelGGL((chain_kernel<2>), dim3((unsigned)units), dim3(256), 0, stream,
                           (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v, a.beta,
                           a.initial_state, a.cu_seqlens, a.final_state, (uint16_t*)a.out, ws, a.total_tokens,
                           a.num_qk_heads, a.num_v_heads, a.scale);
    } else {
        const int64_t groups = (int64_t)a.num_seqs * a.num_qk_heads;
        const int64_t per = 8 * (int64_t)(a.num_v_heads / a.num_qk_heads);
        const int64_t blocks = ((groups + 7) / 8) * 8 * per;   // groups padded to a multiple of 8
        hipLaunchKernelGGL(chain_slice_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                           (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v, a.beta,
                           a.initial_state, a.cu_seqlens, a.final_state, (uint16_t*)a.out, ws, a.total_tokens,
                           a.num_seqs, a.num_qk_heads, a.num_v_heads, a.scale);
    }
    prof::end(stream);
    return hipGetLastError();
}

}  // namespace gdn
