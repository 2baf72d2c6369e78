// Chunked bf16 prefill, segment-parallel: the whole prefill in three launches.
//
// Chunk algebra (chunk of n <= 64 tokens, entry state S (d_v x d_k), gamma =
// in-chunk cumulative sum of g, Gamma = exp(gamma)):
//   A[r][c] = beta_r exp(gamma_r - gamma_c) (k_r . k_c)   c < r   decay-masked Gram
//   U       solves (I + A) U = beta * (V - Gamma * (K S^T))       the chunk's delta writes
//   O       = scale (Gamma * (Q S^T) + P U),  P[r][c] = exp(gamma_r - gamma_c) (q_r . k_c), c <= r
//   S_end   = Gamma_last S + U^T diag(exp(gamma_last - gamma)) K
// (unrolling the per-token rule inside the chunk: the write of token r sees
// the decayed entry state plus the chunk's earlier writes, which is the unit
// lower-triangular system above). The system is solved by 16-row blocks:
// U_b = (I + A_bb)^-1 (X_b - sum_{b' < b} A_bb' U_b'), so only the four 16 x 16
// diagonal blocks are inverted; the off-diagonal blocks are applied by MFMA.
//
// Segments. S_end is affine in the entry state: over a segment of L chunks,
// S_end = S_in M_seg + H_seg, where H_seg is the segment run from S_in = 0 and
// M_seg (d_k x d_k) the run from S_in = I with V = 0. The launches:
//   pass A   every segment but a sequence's last: H (segment 0 starts from
//            the sequence's initial state, so its H is its end state) and,
//            for segments >= 1, M.
//   combine  S_in(1) = H_0, S_in(j+1) = S_in(j) M_j + H_j, fp32 values (products
//            split into bf16 parts on MFMA, fp32 accumulation).
//   pass C   every segment from its true entry state: outputs and, for the
//            last segment, the final state.
//
// Work split inside a workgroup (one (segment, V head)):
//   chain waves     each owns 32 value columns of a 128 x 128 fp32 state (pass
//                   C: one state; pass A: H and M, each wave running both),
//                   held in MFMA accumulators, and runs chunk c.
//   producer waves  (4) meanwhile build chunk c + 1's factors (masked Gram
//                   blocks, diagonal-block inverses, decay vectors) and stage
//                   chunk c + 2's K and Q (pass C) or K and V (pass A) tiles
//                   from registers into LDS.
// The tiles are triple-buffered (K and Q with keys and rows reordered, see
// kq_row) and the factors double-buffered, so one workgroup barrier per chunk
// separates producers from consumers. In pass C values and outputs go straight
// between HBM and the chain waves' registers.
#include "gdn_mfma.h"

namespace gdn {

using namespace mf;

namespace {

enum { kModeOut = 0, kModeHM = 1 };
constexpr size_t kSegMat = (size_t)D * D;   // floats in one 128 x 128 matrix
constexpr int kSegMats = 3;                 // H, M, S_in per (segment, V head)
constexpr int kProd = 4;                    // producer waves per workgroup
constexpr int TP = 24;                      // bf16 pitch of the 16 x 16 factor blocks (48 bytes)
constexpr int AP = 20;                      // fp32 row pitch of a diagonal A block
constexpr int AB = 16 * AP + 8;             // fp32 stride between diagonal A blocks (bank offset 8)

template <int MODE>
struct ChainWaves {
    static constexpr int n = 4;
};

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

// One chunk's factors. A 16 x 16 block X is stored column-major, blk[c][r] =
// X[r][c] (r: the chunk's token 16 b + r), so that producers write four rows
// of a column with one 8-byte store and the chain reads its 16x16x16 MFMA A
// operand with the LDS transpose read.
struct __attribute__((aligned(16))) ChunkFactors {
    uint16_t Td[4][16][TP];     // (I + A_bb)^-1
    uint16_t Tw[4][16][TP];     // diag(exp(gamma_last - gamma)) (I + A_bb)^-1: the state update's rows
    uint16_t Ob[17][16][TP];    // 0..5: -A_bb' (b > b') at b (b - 1) / 2 + b'; 6..15: scale * P
                                // blocks (mt >= nt, output pass) at 6 + mt (mt + 1) / 2 + nt; 16: unused
    float Gam[kChunk], Gs[kChunk], bet[kChunk];   // Gamma, scale * Gamma, beta
};

// Second tile set: queries (output pass) or values (map pass). Map-pass values
// are held per 4-row group and value-column pair: V[rg][p][e] is the bf16 pair
// (columns 2 p, 2 p + 1) of token row 4 rg + e, so that a chain lane reads its
// four rows of one column pair as one 16-byte word.
template <int MODE>
struct QVTiles {
    uint16_t Q[3][kChunk][RP];
};
template <>
struct QVTiles<kModeHM> {
    uint32_t V[3][kChunk / 4][D / 2][4];
};

template <int MODE>
struct __attribute__((aligned(16))) SegSmem {
    uint16_t K[3][kChunk][RP];                          // keys, token-major (layout: kq_row, kq_col)
    QVTiles<MODE> qv;
    ChunkFactors F[2];
    float Ad[4 * AB];                                   // producer scratch: the diagonal blocks of A
    float Dec[kChunk];                                  // producer scratch: exp(gamma_last - gamma)
    float pg[kProd][kChunk], pb[kProd][kChunk];         // producer scratch: gamma, beta
};

// A pointer the compiler must keep in SGPRs (so that per-row bases are not
// folded into per-lane 64-bit addresses).
template <class T>
__device__ __forceinline__ T* uniform_ptr(T* p) {
    const uint64_t u = reinterpret_cast<uint64_t>(p);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
    return reinterpret_cast<T*>(((uint64_t)hi << 32) | lo);
}

// Raw buffer access to one chunk's rows (word 3 of the resource: 32-bit data
// format, as the GFX9 buffer resource layout requires for untyped access).
// Reads at or past `bytes` return 0 and stores there are dropped, so a partial
// last chunk needs neither clamped rows nor guarded stores, and no access can
// leave the chunk's valid rows.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t chunk_rsrc(const void* base, int64_t bytes) {
    const uint32_t n = bytes > 0 ? (uint32_t)bytes : 0u;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)n, 0x00020000);
}
__device__ __forceinline__ uint32_t buf_ld_b32(rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0);
}
__device__ __forceinline__ u32x4 buf_ld_b128(rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}
__device__ __forceinline__ void buf_st_b32(uint32_t x, rsrc_t r, uint32_t off) {
    __builtin_amdgcn_raw_buffer_store_b32(x, r, (int)off, 0, 0);
}

// Producer registers: K and Q (output pass) or V (map pass) pieces of the chunk
// two ahead, and g, beta (row = lane) of the chunk one ahead. Map pass: q[i][e]
// holds the value-column pair pl % 64 of row 4 (pl / 64 + 4 i) + e.
struct ProdRegs {
    u32x4 k[4], q[4];
    float g, b;     // the chunk whose factors are built next
    float gn, bn;   // the chunk after it, requested a whole chunk step ahead
};

// Rows past the end of a chunk re-read its last row (they are zeroed when
// staged), so no load leaves the sequence and none is branched.
// Piece i of producer lane pl: row 16 i + pl / 16, 16-byte column block pl %
// 16. Rows past nc read as zero.
template <int MODE>
__device__ __forceinline__ void prod_fetch_kq(ProdRegs& pr, const uint16_t* kc, const uint16_t* qc, const uint16_t* vc,
                                              int nc, int ldk, int ldv, int pl) {
    const rsrc_t rk = chunk_rsrc(uniform_ptr(kc), (int64_t)nc * ldk * 2);
    if constexpr (MODE == kModeOut) {
        const rsrc_t rq = chunk_rsrc(uniform_ptr(qc), (int64_t)nc * ldk * 2);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t off = (uint32_t)(((pl >> 4) + 16 * i) * ldk + (pl & 15) * 8) * 2u;
            pr.k[i] = buf_ld_b128(rk, off);
            pr.q[i] = buf_ld_b128(rq, off);
        }
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            pr.k[i] = buf_ld_b128(rk, (uint32_t)(((pl >> 4) + 16 * i) * ldk + (pl & 15) * 8) * 2u);
        // one wave's load: 64 consecutive column pairs of one row (256 bytes)
        const rsrc_t rv = chunk_rsrc(uniform_ptr(vc), (int64_t)nc * ldv * 2);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                pr.q[i][e] = buf_ld_b32(rv, (uint32_t)((4 * ((pl >> 6) + 4 * i) + e) * ldv + 2 * (pl & 63)) * 2u);
    }
}

__device__ __forceinline__ void prod_fetch_gb(ProdRegs& pr, const float* gc, const float* bc, int nc, int hv,
                                              int lane) {
    const uint32_t off = (uint32_t)(lane * hv) * 4u;
    pr.gn = __builtin_bit_cast(float, buf_ld_b32(chunk_rsrc(uniform_ptr(gc), (int64_t)nc * hv * 4), off));
    pr.bn = __builtin_bit_cast(float, buf_ld_b32(chunk_rsrc(uniform_ptr(bc), (int64_t)nc * hv * 4), off));
}

// In-kernel L2 normalisation of N 8-element pieces of k or q rows (a row's 16
// pieces sit in 16 consecutive lanes): each lane sums its piece's squares, the
// N row sums are completed over the 16 lanes together (the cross-lane steps of
// different pieces interleaved, so none waits on its own previous step), and
// every element is scaled and rounded back to bf16 (a zero row stays zero).
template <int N>
__device__ __forceinline__ void l2norm_pieces(u32x4 (&x)[N]) {
    float ss[N];
#pragma unroll
    for (int p = 0; p < N; ++p) {
        float s = 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float lo = __uint_as_float(x[p][j] << 16), hi = __uint_as_float(x[p][j] & 0xFFFF0000u);
            s = fmaf(lo, lo, s);
            s = fmaf(hi, hi, s);
        }
        ss[p] = s;
    }
#pragma unroll
    for (int p = 0; p < N; ++p) ss[p] += dpp_quad_xor1(ss[p]);
#pragma unroll
    for (int p = 0; p < N; ++p) ss[p] += dpp_quad_xor2(ss[p]);
#pragma unroll
    for (int p = 0; p < N; ++p) ss[p] += dpp_half_mirror(ss[p]);
#pragma unroll
    for (int p = 0; p < N; ++p) ss[p] += dpp_row_mirror(ss[p]);
#pragma unroll
    for (int p = 0; p < N; ++p) {
        const float r = rsqrtf(ss[p] + kQkNormEps);
#pragma unroll
        for (int j = 0; j < 4; ++j)
            x[p][j] = pack_bf16(__uint_as_float(x[p][j] << 16) * r, __uint_as_float(x[p][j] & 0xFFFF0000u) * r);
    }
}

// K and Q tiles. Within each 32-key block the keys are held in the
// order 4 g .. 4 g + 3, 16 + 4 g .. 16 + 4 g + 3 for g = 0..3 (the key order of
// the state's MFMA B operand), so that the chain's K S^T and Q S^T operands are
// single 16-byte reads instead of two 8-byte ones; products that reduce over
// the keys (the Gram blocks) read both operands in this order and are
// unchanged. Token row r is stored at row kq_row(r), which transposes 4 x 4
// within each 16 rows (r = 16 i + 4 a + b -> 16 i + 4 b + a): with the 136-wide
// rows, the 16-byte reads of 16 consecutive rows and the transposed reads of
// the state update (4 rows x 4 key blocks per 16 lanes) then fall on distinct
// banks.
__device__ __forceinline__ int kq_row(int r) { return (r & ~15) | ((r & 3) << 2) | ((r >> 2) & 3); }

// Column of natural keys 8 c8 .. 8 c8 + 3 (keys 8 c8 + 4 .. + 7 follow eight columns further).
__device__ __forceinline__ int kq_col(int c8) { return 32 * (c8 >> 2) + 16 * (c8 & 1) + 4 * ((c8 >> 1) & 1); }

// MFMA operand (lane (g, m) of a 16x16x32 step kk): token row `row`, keys
// 32 kk + 4 g .. + 3 and 32 kk + 16 + 4 g .. + 3.
__device__ __forceinline__ bf16x8 kq_row8(const uint16_t* tile, int row, int kk, int g) {
    return lds_row8(tile, RP, kq_row(row), kk, g);
}

// A operand of K^T (row = key 16 t + m, reduction = tokens) in accumulator
// order: slots 0..3 are tokens 32 kk + 4 g + 0..3 and slots 4..7 tokens
// 32 kk + 16 + 4 g + 0..3. Lane (g, m) addresses token row 32 kk + 4 g + m / 4
// at natural keys 16 t + 4 (m % 4) .. + 3; the row 16 tokens later is 16 rows
// further. lane_off is this lane's part of the address, kq_kt_tr_lane(g, m).
__device__ __forceinline__ int kq_kt_tr_lane(int g, int m) { return kq_row(4 * g + (m >> 2)) * RP + 8 * (m & 3); }
__device__ __forceinline__ bf16x8 kq_kt_tr(const uint16_t* K, int t, int kk, int lane_off) {
    const uint16_t* p = K + 32 * kk * RP + lane_off + 32 * (t >> 1) + 4 * (t & 1);
    const i16x4 lo = lds_read_tr16(p);
    const i16x4 hi = lds_read_tr16(p + 16 * RP);
    u32x4 u;
    u.x = __builtin_bit_cast(u32x2, lo).x;
    u.y = __builtin_bit_cast(u32x2, lo).y;
    u.z = __builtin_bit_cast(u32x2, hi).x;
    u.w = __builtin_bit_cast(u32x2, hi).y;
    return __builtin_bit_cast(bf16x8, u);
}

// Rows past the end of a partial chunk were read as zero. QKN: k (and q) rows
// are L2-normalised on the way.
template <int MODE, bool QKN>
__device__ __forceinline__ void prod_stage_kq(SegSmem<MODE>& sm, int buf, const ProdRegs& pr, int pl) {
    constexpr int NP = MODE == kModeOut ? 8 : 4;   // pieces 0..3: k; 4..7: q (output pass)
    u32x4 x[NP];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        x[i] = pr.k[i];
        if constexpr (MODE == kModeOut) x[4 + i] = pr.q[i];
    }
    if constexpr (QKN) l2norm_pieces<NP>(x);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int p = pl + 256 * i;
        const int row = p >> 4, c8 = p & 15;
        const u32x4 kv = x[i];
        const int pr_ = kq_row(row), col = kq_col(c8);
        *reinterpret_cast<u32x2*>(&sm.K[buf][pr_][col]) = u32x2{kv[0], kv[1]};
        *reinterpret_cast<u32x2*>(&sm.K[buf][pr_][col + 8]) = u32x2{kv[2], kv[3]};
        if constexpr (MODE == kModeOut) {
            const u32x4 qv = x[4 + i];
            *reinterpret_cast<u32x2*>(&sm.qv.Q[buf][pr_][col]) = u32x2{qv[0], qv[1]};
            *reinterpret_cast<u32x2*>(&sm.qv.Q[buf][pr_][col + 8]) = u32x2{qv[2], qv[3]};
        } else {
            *reinterpret_cast<u32x4*>(&sm.qv.V[buf][(pl >> 6) + 4 * i][pl & 63][0]) = pr.q[i];
        }
    }
}

// Inclusive prefix sum over the 64 lanes of a wave with DPP: shifts inside
// rows of 16 lanes, then the row totals carried by the GFX9 row broadcasts.
__device__ __forceinline__ float wave_prefix_sum(float x) {
    // row_shr:d (DPP control 0x110 + d); lanes below d in their row add 0.
    x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x111, 0xF, 0xF, false));
    x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x112, 0xF, 0xF, false));
    x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x114, 0xF, 0xF, false));
    x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x118, 0xF, 0xF, false));
    x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x142, 0xA, 0xF, false));
    x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x143, 0xC, 0xF, false));
    return x;
}

// 16 x 16 Gram block: rows 16 mt .. of X times rows 16 nt .. of K, transposed;
// lane (g, m) gets element [16 mt + 4 g + e][16 nt + m].
__device__ __forceinline__ f32x4 gram_block(const uint16_t* X, const uint16_t* K, int mt, int nt, int g, int m) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
        acc = mfma16(kq_row8(X, 16 * mt + m, kk, g), kq_row8(K, 16 * nt + m, kk, g), acc);
    return acc;
}

// Accumulator tile (lane (g, m): rows 4 g .. 4 g + 3 of column m) into a
// column-major block.
__device__ __forceinline__ void store_block_bf16(uint16_t (*blk)[TP], const f32x4& v, int g, int m) {
    u32x2 u;
    u.x = pack_bf16(v[0], v[1]);
    u.y = pack_bf16(v[2], v[3]);
    *reinterpret_cast<u32x2*>(&blk[m][4 * g]) = u;
}

// Factors of one chunk (its K/Q tiles in buffer kb) into F. Producer wave 0
// builds the four diagonal blocks of A and inverts them (lane group g: block
// g, lane m: column m) and, in the output pass, the last diagonal P block (job
// 15); waves 1..3 take the off-diagonal A blocks (jobs 0..5) and the other P
// blocks (jobs 6..14) in turn.
template <int MODE>
__device__ __forceinline__ void prod_factors(SegSmem<MODE>& sm, int kb, ChunkFactors& F, const ProdRegs& pr, int nc,
                                             float scale, int pw, int lane) {
    const uint16_t* K = &sm.K[kb][0][0];
    const uint16_t* Q = K;
    if constexpr (MODE == kModeOut) Q = &sm.qv.Q[kb][0][0];
    const int g = lane >> 4, m = lane & 15;

    // gamma = in-chunk inclusive prefix sum of g; rows past nc add 0 and have beta 0.
    const float x = wave_prefix_sum(lane < nc ? pr.g : 0.f);
    const float bt = lane < nc ? pr.b : 0.f;
    sm.pg[pw][lane] = x;
    sm.pb[pw][lane] = bt;

    if (pw == 0) {
        const float glast = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 63));
        const float G = fast_exp(x);
        F.Gam[lane] = G;
        F.Gs[lane] = scale * G;
        F.bet[lane] = bt;
        sm.Dec[lane] = fast_exp(glast - x);
        // Diagonal blocks of A, fp32, strictly lower: block b = rows/cols 16 b ..
        // The four blocks are independent and each uses one operand on both sides:
        // all operand reads first, then the four MFMA chains interleaved.
        // Output pass: wave 0 also builds the last diagonal P block (Q K^T of rows
        // 48..63, whose K operand it already holds), so that waves 1..3 share the
        // other fifteen jobs evenly.
        float* Ad = sm.Ad;
        bf16x8 kd[4][4], q3[4];
        f32x4 grd[4], brd[4];
        float gcd[4];
#pragma unroll
        for (int b = 0; b < 4; ++b) {
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) kd[b][kk] = kq_row8(K, 16 * b + m, kk, g);
            grd[b] = *reinterpret_cast<const f32x4*>(&sm.pg[0][16 * b + 4 * g]);
            brd[b] = *reinterpret_cast<const f32x4*>(&sm.pb[0][16 * b + 4 * g]);
            gcd[b] = sm.pg[0][16 * b + m];
        }
        if constexpr (MODE == kModeOut) {
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) q3[kk] = kq_row8(Q, 48 + m, kk, g);
        }
        __builtin_amdgcn_sched_barrier(0);
        f32x4 accd[4], accp = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int b = 0; b < 4; ++b) accd[b] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
            for (int b = 0; b < 4; ++b) accd[b] = mfma16(kd[b][kk], kd[b][kk], accd[b]);
            if constexpr (MODE == kModeOut) accp = mfma16(q3[kk], kd[3][kk], accp);
        }
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (MODE == kModeOut) {
            f32x4 v;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float x = scale * fast_exp(grd[3][e] - gcd[3]) * accp[e];
                v[e] = (m <= 4 * g + e) ? x : 0.f;
            }
            store_block_bf16(F.Ob[15], v, g, m);
        }
#pragma unroll
        for (int b = 0; b < 4; ++b) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float a = brd[b][e] * fast_exp(grd[b][e] - gcd[b]) * accd[b][e];
                Ad[b * AB + (4 * g + e) * AP + m] = (m < 4 * g + e) ? a : 0.f;
            }
        }
        // (I + A_gg)^-1, column m, by forward substitution in batches of four
        // rows: a batch reads its rows as 16-byte pieces, takes the part of
        // each row's sum over earlier batches in parallel, then the four rows
        // in order.
        const float* Ag = Ad + g * AB;
        float t[16];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            f32x4 a[4][4];
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int c4 = 0; c4 <= q; ++c4) a[i][c4] = *reinterpret_cast<const f32x4*>(Ag + (4 * q + i) * AP + 4 * c4);
            float sacc[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 4 * q + i;
                float p0 = (r == m) ? 1.f : 0.f, p1 = 0.f, p2 = 0.f, p3 = 0.f;
#pragma unroll
                for (int c4 = 0; c4 < q; ++c4) {
                    p0 -= a[i][c4][0] * t[4 * c4];
                    p1 -= a[i][c4][1] * t[4 * c4 + 1];
                    p2 -= a[i][c4][2] * t[4 * c4 + 2];
                    p3 -= a[i][c4][3] * t[4 * c4 + 3];
                }
                sacc[i] = (p0 + p1) + (p2 + p3);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float v = sacc[i];
#pragma unroll
                for (int jj = 0; jj < i; ++jj) v -= a[i][q][jj] * t[4 * q + jj];
                t[4 * q + i] = v;
            }
        }
        // Column m of both blocks: 16 contiguous bf16 each (two 16-byte stores).
        u32x4 td[2], tw[2];
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
            const f32x4 dec = *reinterpret_cast<const f32x4*>(&sm.Dec[16 * g + 4 * r4]);
            td[r4 >> 1][2 * (r4 & 1)] = pack_bf16(t[4 * r4], t[4 * r4 + 1]);
            td[r4 >> 1][2 * (r4 & 1) + 1] = pack_bf16(t[4 * r4 + 2], t[4 * r4 + 3]);
            tw[r4 >> 1][2 * (r4 & 1)] = pack_bf16(dec[0] * t[4 * r4], dec[1] * t[4 * r4 + 1]);
            tw[r4 >> 1][2 * (r4 & 1) + 1] = pack_bf16(dec[2] * t[4 * r4 + 2], dec[3] * t[4 * r4 + 3]);
        }
        *reinterpret_cast<u32x4*>(&F.Td[g][m][0]) = td[0];
        *reinterpret_cast<u32x4*>(&F.Td[g][m][8]) = td[1];
        *reinterpret_cast<u32x4*>(&F.Tw[g][m][0]) = tw[0];
        *reinterpret_cast<u32x4*>(&F.Tw[g][m][8]) = tw[1];
        return;
    }

    if constexpr (MODE == kModeOut) {
        // Output pass: off-diagonal A blocks (stored negated) and P blocks
        // (scaled). Waves 1..3 take jobs pw - 1, pw + 2, ...: fifteen jobs in
        // five rounds each (block 16 of the factor set stays unused).
        constexpr uint64_t kRow = 0x3333222110333221ull, kCol = 0x3210210100210100ull;
        constexpr int NJOBS = 15;   // job 15 (P block (3, 3)) is built by wave 0
        constexpr int ROUNDS = NJOBS / 3;
#pragma unroll
        for (int jj = 0; jj < ROUNDS; ++jj) {
            const int job = (pw - 1) + 3 * jj;
            const int jt = job < NJOBS ? job : NJOBS - 1;
            const int mt = (int)((kRow >> (4 * jt)) & 15), nt = (int)((kCol >> (4 * jt)) & 15);
            const bool isP = jt >= 6;
            const f32x4 acc = gram_block(isP ? Q : K, K, mt, nt, g, m);
            const f32x4 gr = *reinterpret_cast<const f32x4*>(&sm.pg[pw][16 * mt + 4 * g]);
            const f32x4 br = *reinterpret_cast<const f32x4*>(&sm.pb[pw][16 * mt + 4 * g]);
            const float gc = sm.pg[pw][16 * nt + m];
            f32x4 v;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float x = (isP ? scale : -br[e]) * fast_exp(gr[e] - gc) * acc[e];
                v[e] = (mt > nt || m <= 4 * g + e) ? x : 0.f;
            }
            store_block_bf16(F.Ob[job < NJOBS ? job : 16], v, g, m);
        }
    } else {
        // Map pass: only the six off-diagonal A blocks (stored negated), grouped
        // by block column so that each wave reads its K column tile once.
        bf16x8 kc[4];
        auto job = [&](int mt, int nt) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) acc = mfma16(kq_row8(K, 16 * mt + m, kk, g), kc[kk], acc);
            const f32x4 gr = *reinterpret_cast<const f32x4*>(&sm.pg[pw][16 * mt + 4 * g]);
            const f32x4 br = *reinterpret_cast<const f32x4*>(&sm.pb[pw][16 * mt + 4 * g]);
            const float gc = sm.pg[pw][16 * nt + m];
            f32x4 v;
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = -(br[e] * fast_exp(gr[e] - gc) * acc[e]);
            store_block_bf16(F.Ob[mt * (mt - 1) / 2 + nt], v, g, m);
        };
        const int nt = pw - 1;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) kc[kk] = kq_row8(K, 16 * nt + m, kk, g);
        if (pw == 1) {
            job(1, 0);
            job(2, 0);
            job(3, 0);
        } else if (pw == 2) {
            job(2, 1);
            job(3, 1);
        } else {
            job(3, 2);
        }
    }
}

// 16x16x16 A operand (lane (g, m): X[m][4 g .. 4 g + 3]) of a column-major
// block: a transpose read, lane i of group g addressing blk[4 g + i / 4][4 (i % 4)].
__device__ __forceinline__ i16x4 lds_blk_a(const uint16_t (*blk)[TP], int g, int m) {
    return lds_read_tr16(&blk[4 * g + (m >> 2)][4 * (m & 3)]);
}

__device__ __forceinline__ f32x4 mfma_x16(i16x4 a, i16x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

// Accumulator tile -> 16x16x16 B operand (reduction index 4 g + e).
__device__ __forceinline__ i16x4 pack4(const f32x4& v) {
    u32x2 u;
    u.x = pack_bf16(v[0], v[1]);
    u.y = pack_bf16(v[2], v[3]);
    return __builtin_bit_cast(i16x4, u);
}

// Chain-wave values: rows 16 mt + 4 g + e, columns cb + 2 m, cb + 2 m + 1 of
// the chunk whose (row 0, column cb) element vc points at (wave-uniform);
// rows past nc read as zero.
__device__ __forceinline__ void chain_fetch_v(uint32_t (&vr)[16], const uint16_t* vc, int nc, int ldv, int g, int m) {
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
        const rsrc_t r = chunk_rsrc(uniform_ptr(vc + (int64_t)16 * mt * ldv), (int64_t)(nc - 16 * mt) * ldv * 2);
#pragma unroll
        for (int e = 0; e < 4; ++e) vr[4 * mt + e] = buf_ld_b32(r, (uint32_t)((4 * g + e) * ldv + 2 * m) * 2u);
    }
}

// One chunk of one chain for this wave's 32 value columns; lane (g, m) holds
// columns cb + 2 m (tile nt = 0) and cb + 2 m + 1 (nt = 1). ST[t][nt] element e
// is S[column][key 16 t + 4 g + e]. vin holds this chunk's values; the next
// chunk's (from vnext) are requested into vout.
// Values: the output pass holds them in registers (vin; the next chunk's go to
// vout); the map pass reads this chunk's from LDS (vl: this lane's column pair
// of row group 0).
// Output pass: one chunk of the chain from its entry state (values straight from
// HBM into registers, outputs straight back).
__device__ __forceinline__ void chain_step(const uint16_t* K, const uint16_t* Q, const ChunkFactors& F,
                                           f32x4 (&ST)[8][2], const uint32_t (&vin)[16], uint32_t (&vout)[16],
                                           const uint16_t* vnext, int ncn,
                                           uint16_t* orow0, int ldv, int nc, float scale, int g, int m) {
    // Z = K S^T and, for the output, Y = Q S^T: one pass over the S^T operands.
    f32x4 X[4][2], Y[4][2];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
            X[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
            Y[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
    // Software-pipelined over the key steps: step kk + 1's operand rows
    // are requested before step kk's products are issued (the scheduler
    // alone keeps too few LDS reads in flight here).
    bf16x8 ka[2][4], qa[2][4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
        ka[0][mt] = kq_row8(K, 16 * mt + m, 0, g);
        qa[0][mt] = kq_row8(Q, 16 * mt + m, 0, g);
    }
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
        const int cur = kk & 1;
        if (kk < 3) {
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
                ka[cur ^ 1][mt] = kq_row8(K, 16 * mt + m, kk + 1, g);
                qa[cur ^ 1][mt] = kq_row8(Q, 16 * mt + m, kk + 1, g);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
        const bf16x8 sb0 = pack_acc_pair(ST[2 * kk][0], ST[2 * kk + 1][0]);
        const bf16x8 sb1 = pack_acc_pair(ST[2 * kk][1], ST[2 * kk + 1][1]);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
            X[mt][0] = mfma16(ka[cur][mt], sb0, X[mt][0]);
            X[mt][1] = mfma16(ka[cur][mt], sb1, X[mt][1]);
            Y[mt][0] = mfma16(qa[cur][mt], sb0, Y[mt][0]);
            Y[mt][1] = mfma16(qa[cur][mt], sb1, Y[mt][1]);
        }
        __builtin_amdgcn_sched_barrier(0);
    }
    // X = beta (V - Gamma Z); then the next chunk's values are requested.
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
        const f32x4 Gr = *reinterpret_cast<const f32x4*>(&F.Gam[16 * mt + 4 * g]);
        const f32x4 Br = *reinterpret_cast<const f32x4*>(&F.bet[16 * mt + 4 * g]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const uint32_t x = vin[4 * mt + e];
            const float v0 = __uint_as_float(x << 16), v1 = __uint_as_float(x & 0xFFFF0000u);
            X[mt][0][e] = Br[e] * (v0 - Gr[e] * X[mt][0][e]);
            X[mt][1][e] = Br[e] * (v1 - Gr[e] * X[mt][1][e]);
        }
    }
    // The next chunk's values are requested only after this chunk's are
    // consumed: global loads complete in order, so a load hoisted above the
    // uses of the previous ones would make those uses wait for it.
    __builtin_amdgcn_sched_barrier(0);
    chain_fetch_v(vout, vnext, ncn, ldv, g, m);
    // U by 16-row blocks: U_b = Td_b (X_b - sum A_bb' U_b'), and the state
    // update's exp(gamma_last - gamma) U_b = Tw_b (same right-hand side),
    // packed as soon as a pair of blocks is done.
    i16x4 Ub[4][2];
    bf16x8 Wb[2][2];
    f32x4 Wprev[2];
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        f32x4 acc0 = X[b][0], acc1 = X[b][1];
#pragma unroll
        for (int bp = 0; bp < b; ++bp) {
            const i16x4 a = lds_blk_a(F.Ob[b * (b - 1) / 2 + bp], g, m);
            acc0 = mfma_x16(a, Ub[bp][0], acc0);
            acc1 = mfma_x16(a, Ub[bp][1], acc1);
        }
        const i16x4 r0 = pack4(acc0), r1 = pack4(acc1);
        const i16x4 a = lds_blk_a(F.Td[b], g, m);
        const i16x4 aw = lds_blk_a(F.Tw[b], g, m);
        const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
        Ub[b][0] = pack4(mfma_x16(a, r0, zero));
        Ub[b][1] = pack4(mfma_x16(a, r1, zero));
        const f32x4 w0 = mfma_x16(aw, r0, zero);
        const f32x4 w1 = mfma_x16(aw, r1, zero);
        if (b & 1) {
            Wb[b >> 1][0] = pack_acc_pair(Wprev[0], w0);
            Wb[b >> 1][1] = pack_acc_pair(Wprev[1], w1);
        } else {
            Wprev[0] = w0;
            Wprev[1] = w1;
        }
    }
    {
        // O = scale Gamma (Q S^T) + (scale P) U
        uint32_t ob[4][4];   // bf16 pairs: row 16 mt + 4 g + e, columns cb + 2 m, cb + 2 m + 1
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
            const f32x4 Gr = *reinterpret_cast<const f32x4*>(&F.Gs[16 * mt + 4 * g]);
            f32x4 y0 = Gr * Y[mt][0], y1 = Gr * Y[mt][1];
#pragma unroll
            for (int b = 0; b <= mt; ++b) {
                const i16x4 a = lds_blk_a(F.Ob[6 + mt * (mt + 1) / 2 + b], g, m);
                y0 = mfma_x16(a, Ub[b][0], y0);
                y1 = mfma_x16(a, Ub[b][1], y1);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) ob[mt][e] = pack_bf16(y0[e], y1[e]);
        }
        // Rows past nc fall outside the chunk's buffer range and are dropped.
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
            const rsrc_t r = chunk_rsrc(uniform_ptr(orow0 + (int64_t)16 * mt * ldv), (int64_t)(nc - 16 * mt) * ldv * 2);
#pragma unroll
            for (int e = 0; e < 4; ++e) buf_st_b32(ob[mt][e], r, (uint32_t)((4 * g + e) * ldv + 2 * m) * 2u);
        }
    }
    // S^T = Gamma_last S^T + K^T (exp(gamma_last - gamma) U)
    const float Glast = F.Gam[kChunk - 1];
    const int tro = kq_kt_tr_lane(g, m);
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        const bf16x8 a0 = kq_kt_tr(K, t, 0, tro);
        const bf16x8 a1 = kq_kt_tr(K, t, 1, tro);
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
            f32x4 acc = ST[t][nt] * Glast;
            acc = mfma16(a0, Wb[0][nt], acc);
            ST[t][nt] = mfma16(a1, Wb[1][nt], acc);
        }
    }
}

// Map pass: the H chain (from 0, with the chunk's values) and the M chain (from I,
// no values) advanced together over one chunk. The two chains use the same K rows,
// factor blocks and K^T operands, so each is read from LDS once and feeds both
// chains' products, and the two independent dependency chains interleave.
__device__ __forceinline__ void chain_step_hm(const uint16_t* K, const ChunkFactors& F, f32x4 (&ST)[8][2],
                                              f32x4 (&SM)[8][2], int g, int m, const uint32_t* vl) {
    // Z = K S^T for both states, the K S^T loop software-pipelined over the key steps.
    f32x4 XH[4][2], XM[4][2];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
            XH[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
            XM[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
    {
        bf16x8 ka[2][4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) ka[0][mt] = kq_row8(K, 16 * mt + m, 0, g);
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            const int cur = kk & 1;
            if (kk < 3) {
#pragma unroll
                for (int mt = 0; mt < 4; ++mt) ka[cur ^ 1][mt] = kq_row8(K, 16 * mt + m, kk + 1, g);
            }
            __builtin_amdgcn_sched_barrier(0);
            const bf16x8 h0 = pack_acc_pair(ST[2 * kk][0], ST[2 * kk + 1][0]);
            const bf16x8 h1 = pack_acc_pair(ST[2 * kk][1], ST[2 * kk + 1][1]);
            const bf16x8 m0 = pack_acc_pair(SM[2 * kk][0], SM[2 * kk + 1][0]);
            const bf16x8 m1 = pack_acc_pair(SM[2 * kk][1], SM[2 * kk + 1][1]);
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
                XH[mt][0] = mfma16(ka[cur][mt], h0, XH[mt][0]);
                XM[mt][0] = mfma16(ka[cur][mt], m0, XM[mt][0]);
                XH[mt][1] = mfma16(ka[cur][mt], h1, XH[mt][1]);
                XM[mt][1] = mfma16(ka[cur][mt], m1, XM[mt][1]);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    // X = beta (V - Gamma Z) for H, -beta Gamma Z for M (the chunk's values from LDS).
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
        const u32x4 vw = *reinterpret_cast<const u32x4*>(vl + (4 * mt + g) * (D / 2) * 4);
        const f32x4 Gr = *reinterpret_cast<const f32x4*>(&F.Gam[16 * mt + 4 * g]);
        const f32x4 Br = *reinterpret_cast<const f32x4*>(&F.bet[16 * mt + 4 * g]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float v0 = __uint_as_float(vw[e] << 16), v1 = __uint_as_float(vw[e] & 0xFFFF0000u);
            XH[mt][0][e] = Br[e] * (v0 - Gr[e] * XH[mt][0][e]);
            XH[mt][1][e] = Br[e] * (v1 - Gr[e] * XH[mt][1][e]);
            XM[mt][0][e] = Br[e] * (0.f - Gr[e] * XM[mt][0][e]);
            XM[mt][1][e] = Br[e] * (0.f - Gr[e] * XM[mt][1][e]);
        }
    }
    // Both solves by 16-row blocks, each factor block read once for the two chains.
    i16x4 UH[4][2], UM[4][2];
    bf16x8 WH[2][2], WM[2][2];
    f32x4 PH[2], PM[2];
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        f32x4 h0 = XH[b][0], h1 = XH[b][1], k0 = XM[b][0], k1 = XM[b][1];
#pragma unroll
        for (int bp = 0; bp < b; ++bp) {
            const i16x4 a = lds_blk_a(F.Ob[b * (b - 1) / 2 + bp], g, m);
            h0 = mfma_x16(a, UH[bp][0], h0);
            k0 = mfma_x16(a, UM[bp][0], k0);
            h1 = mfma_x16(a, UH[bp][1], h1);
            k1 = mfma_x16(a, UM[bp][1], k1);
        }
        const i16x4 rh0 = pack4(h0), rh1 = pack4(h1), rm0 = pack4(k0), rm1 = pack4(k1);
        const i16x4 a = lds_blk_a(F.Td[b], g, m);
        const i16x4 aw = lds_blk_a(F.Tw[b], g, m);
        const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
        UH[b][0] = pack4(mfma_x16(a, rh0, zero));
        UM[b][0] = pack4(mfma_x16(a, rm0, zero));
        UH[b][1] = pack4(mfma_x16(a, rh1, zero));
        UM[b][1] = pack4(mfma_x16(a, rm1, zero));
        const f32x4 wh0 = mfma_x16(aw, rh0, zero), wm0 = mfma_x16(aw, rm0, zero);
        const f32x4 wh1 = mfma_x16(aw, rh1, zero), wm1 = mfma_x16(aw, rm1, zero);
        if (b & 1) {
            WH[b >> 1][0] = pack_acc_pair(PH[0], wh0);
            WH[b >> 1][1] = pack_acc_pair(PH[1], wh1);
            WM[b >> 1][0] = pack_acc_pair(PM[0], wm0);
            WM[b >> 1][1] = pack_acc_pair(PM[1], wm1);
        } else {
            PH[0] = wh0;
            PH[1] = wh1;
            PM[0] = wm0;
            PM[1] = wm1;
        }
    }
    // S^T = Gamma_last S^T + K^T (exp(gamma_last - gamma) U) for both states, each K^T
    // operand read once. The lane offset is hidden from loop-invariant code motion (hoisted
    // out of the chunk loop, the addresses derived from it would hold registers throughout).
    const float Glast = F.Gam[kChunk - 1];
    int tro = kq_kt_tr_lane(g, m);
    asm volatile("" : "+v"(tro));
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        const bf16x8 a0 = kq_kt_tr(K, t, 0, tro);
        const bf16x8 a1 = kq_kt_tr(K, t, 1, tro);
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
            f32x4 hs = ST[t][nt] * Glast, ms = SM[t][nt] * Glast;
            hs = mfma16(a0, WH[0][nt], hs);
            ms = mfma16(a0, WM[0][nt], ms);
            ST[t][nt] = mfma16(a1, WH[1][nt], hs);
            SM[t][nt] = mfma16(a1, WM[1][nt], ms);
        }
    }
}

// The chain waves' chunk loop (one barrier per chunk, matching the producers).
// Output pass: one chain with values and outputs. Map pass: the H chain (with
// values) and the M chain (no values) for the same columns, advanced together.
template <int MODE>
__device__ __forceinline__ void chain_loop(SegSmem<MODE>& sm, f32x4 (&ST)[8][2], f32x4 (&SM)[8][2],
                                           const uint16_t* vcol, uint16_t* ocol, int64_t bos, int64_t eos,
                                           int64_t c_begin, int64_t nchunks, int ldv, float scale, int lg, int lm,
                                           int cb) {
    auto chunk_nc = [&](int64_t c) {
        const int64_t rem = eos - (bos + c * kChunk);
        return (int)(rem < kChunk ? rem : kChunk);
    };
    uint32_t va[16];
    if constexpr (MODE == kModeOut)
        if (nchunks > 0) chain_fetch_v(va, vcol + (bos + c_begin * kChunk) * ldv, chunk_nc(c_begin), ldv, lg, lm);
    // The entry state and the first values have arrived before the chunk loop
    // starts; otherwise the loop header's wait for the values would also cover
    // every later global access (the previous chunk's output stores included).
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
    lds_barrier();   // prologue: chunks 0 and 1 staged
    lds_barrier();   // prologue: chunk 0's factors
    if constexpr (MODE == kModeOut) {
        for (int64_t i = 0; i < nchunks; ++i) {
            const int64_t c = c_begin + i;
            const int kb = (int)(i % 3);
            const int64_t cn = (i + 1 < nchunks) ? c + 1 : c;
            const int64_t t0 = bos + c * kChunk;
            const uint16_t* vnext = vcol + (bos + cn * kChunk) * ldv;
            chain_step(&sm.K[kb][0][0], &sm.qv.Q[kb][0][0], sm.F[i & 1], ST, va, va, vnext, chunk_nc(cn),
                       ocol + t0 * ldv, ldv, chunk_nc(c), scale, lg, lm);
            lds_barrier();
        }
    } else {
        for (int64_t i = 0; i < nchunks; ++i) {
            const int64_t c = c_begin + i;
            const int kb = (int)(i % 3);
            const uint32_t* vl = &sm.qv.V[kb][0][cb / 2 + lm][0];
            chain_step_hm(&sm.K[kb][0][0], sm.F[i & 1], ST, SM, lg, lm, vl);
            lds_barrier();
        }
    }
}

// One workgroup's task: segment j (of nseg) of sequence n, for V head h.
struct SegTask {
    SeqRange sr;
    int64_t sg, j, nseg, c_begin, c_end, nchunks;
    int n, h, hq;
};

struct SegArgs {
    const uint16_t* q;
    const uint16_t* k;
    const uint16_t* v;
    const float* g;
    const float* beta;
    const float* initial_state;
    float* final_state;
    uint16_t* out;
    float* segws;
    const int32_t* state_indices;   // null: sequence n's state row is n
    const int32_t* has_initial;     // null: read the entry state whenever initial_state is given
    int32_t num_slots;
    int32_t num_qk_heads, num_v_heads;
    float scale;
};

// QKN: L2-normalise k and q rows as they are staged.
template <int MODE, bool QKN>
__device__ __forceinline__ void segment_body(SegSmem<MODE>& sm, const SegArgs& A, const SegTask& tk) {
    constexpr int NCW = ChainWaves<MODE>::n;
    const uint16_t* __restrict__ q = A.q;
    const uint16_t* __restrict__ k = A.k;
    const uint16_t* __restrict__ v = A.v;
    const float* __restrict__ g = A.g;
    const float* __restrict__ beta = A.beta;
    const int32_t num_qk_heads = A.num_qk_heads, num_v_heads = A.num_v_heads;
    const float scale = A.scale;
    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, lg = lane >> 4, lm = lane & 15;
    const SeqRange sr = tk.sr;
    const int64_t j = tk.j, nseg = tk.nseg, c_begin = tk.c_begin, c_end = tk.c_end, nchunks = tk.nchunks;
    const int n = tk.n, h = tk.h, hq = tk.hq;
    float* segmat = A.segws + ((size_t)tk.sg * num_v_heads + h) * kSegMats * kSegMat;

    const bool producer = w >= NCW;
    const int pw = w - NCW;
    const int pl = tid - 64 * NCW;
    // Chain waves (0-3): pass C: the state from its true entry value; pass A:
    // the H map (from the initial state in segment 0, else from 0) and, from
    // segment 1 on, the M map (from I, without values).
    const int cb = 32 * (w & 3);

    const int ldk = num_qk_heads * D, ldv = num_v_heads * D;
    auto chunk_t0 = [&](int64_t c) { return sr.bos + c * kChunk; };
    auto chunk_nc = [&](int64_t c) {
        const int64_t rem = sr.eos - chunk_t0(c);
        return (int)(rem < kChunk ? rem : kChunk);
    };
    auto clampc = [&](int64_t c) { return c < c_end ? c : c_end - 1; };
    ProdRegs pr;
    auto fetch_kq = [&](int64_t c) {
        const int64_t t0 = chunk_t0(c);
        prod_fetch_kq<MODE>(pr, k + t0 * ldk + hq * D, q + t0 * ldk + hq * D, v + t0 * ldv + h * D, chunk_nc(c), ldk,
                            ldv, pl);
    };
    auto fetch_gb = [&](int64_t c) {
        const int64_t t0 = chunk_t0(c);
        prod_fetch_gb(pr, g + t0 * num_v_heads + h, beta + t0 * num_v_heads + h, chunk_nc(c), num_v_heads, lane);
    };
    if (producer) {
        // Prologue: chunks 0 and 1 of the segment staged, chunk 0's factors built.
        if (nchunks > 0) {
            fetch_kq(c_begin);
            fetch_gb(c_begin);
            pr.g = pr.gn;
            pr.b = pr.bn;
            prod_stage_kq<MODE, QKN>(sm, 0, pr, pl);
            fetch_kq(clampc(c_begin + 1));
            if (nchunks > 1) prod_stage_kq<MODE, QKN>(sm, 1, pr, pl);
        }
        lds_barrier();
        if (nchunks > 0) {
            fetch_gb(clampc(c_begin + 1));
            prod_factors<MODE>(sm, 0, sm.F[0], pr, chunk_nc(c_begin), scale, pw, lane);
            fetch_kq(clampc(c_begin + 2));
            pr.g = pr.gn;
            pr.b = pr.bn;
        }
        lds_barrier();
        for (int64_t i = 0; i < nchunks; ++i) {
            const int64_t c = c_begin + i;
            // g and beta of chunk c + 2, a whole step before its factors; then
            // chunk c + 1: factors (its tiles were staged two steps ago);
            // chunk c + 2: tiles from registers to LDS; then the next K/Q loads.
            fetch_gb(clampc(c + 2));
            if (i + 1 < nchunks)
                prod_factors<MODE>(sm, (int)((i + 1) % 3), sm.F[(i + 1) & 1], pr, chunk_nc(c + 1), scale, pw,
                                   lane);
            if (i + 2 < nchunks) prod_stage_kq<MODE, QKN>(sm, (int)((i + 2) % 3), pr, pl);
            fetch_kq(clampc(c + 3));
            pr.g = pr.gn;
            pr.b = pr.bn;
            lds_barrier();
        }
        return;
    }
    // Chain waves.
    f32x4 ST[8][2], SM[8][2];
    {
        const float* src = nullptr;
        if (MODE == kModeOut) {
            if (j == 0) {
                // Entry state: the sequence's state row (a pool slot; none for a
                // padding entry, or when the sequence starts from zeros).
                const int64_t srow = state_row(A.state_indices, A.num_slots, n);
                if (A.initial_state && srow >= 0 && (A.has_initial == nullptr || A.has_initial[n] != 0))
                    src = A.initial_state + (srow * num_v_heads + h) * kSegMat;
            } else {
                src = segmat + 2 * kSegMat;
            }
        }
#pragma unroll
        for (int t = 0; t < 8; ++t)
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) {
                const int col = cb + 2 * lm + nt;
                f32x4 s = {0.f, 0.f, 0.f, 0.f}, e1;
                if (src) s = *reinterpret_cast<const f32x4*>(src + (int64_t)col * D + 16 * t + 4 * lg);
                ST[t][nt] = s;
#pragma unroll
                for (int e = 0; e < 4; ++e) e1[e] = (16 * t + 4 * lg + e == col) ? 1.f : 0.f;
                SM[t][nt] = e1;
            }
    }
    chain_loop<MODE>(sm, ST, SM, v + h * D + cb, A.out + h * D + cb, sr.bos, sr.eos, c_begin,
                     nchunks, ldv, scale, lg, lm, cb);

    if (MODE == kModeOut) {
        // The last segment's end state is the sequence's final state; segment
        // 0's (when more follow) is H_0 = S_in(1), kept for the combine.
        float* dst = nullptr;
        if (j == nseg - 1) {
            const int64_t srow = state_row(A.state_indices, A.num_slots, n);
            if (A.final_state && srow >= 0) dst = A.final_state + (srow * num_v_heads + h) * kSegMat;
        } else if (j == 0) {
            dst = segmat;
        }
        if (dst) {
#pragma unroll
            for (int t = 0; t < 8; ++t)
#pragma unroll
                for (int nt = 0; nt < 2; ++nt)
                    *reinterpret_cast<f32x4*>(dst + (int64_t)(cb + 2 * lm + nt) * D + 16 * t + 4 * lg) = ST[t][nt];
        }
    } else {
#pragma unroll
        for (int t = 0; t < 8; ++t)
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) {
                const int64_t o = (int64_t)(cb + 2 * lm + nt) * D + 16 * t + 4 * lg;
                *reinterpret_cast<f32x4*>(segmat + o) = ST[t][nt];
                *reinterpret_cast<f32x4*>(segmat + kSegMat + o) = SM[t][nt];
            }
    }
}

// Both launches of the segment schedule. Phase 0: segment 0 of every sequence
// runs the output pass from the initial state (its end state is H_0), and
// segments 1 .. nseg - 2 build their maps (H from 0, M from I). Phase 1:
// segments >= 1 run the output pass from the combined entry states. QKN: k and
// q rows are L2-normalised in the kernel.
template <bool QKN>
__global__ __launch_bounds__(64 * (4 + kProd)) void segment_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const float* __restrict__ g, const float* __restrict__ beta, const float* initial_state,
    const int32_t* __restrict__ cu, float* final_state, uint16_t* __restrict__ out, float* __restrict__ segws,
    int64_t total_tokens, int32_t num_seqs, int32_t num_qk_heads, int32_t num_v_heads, int32_t L, int64_t num_segs,
    float scale, int32_t phase, const int32_t* state_indices, const int32_t* has_initial, int32_t num_slots) {
    static_assert(sizeof(SegSmem<kModeHM>) <= sizeof(SegSmem<kModeOut>), "the map pass reuses the output pass's LDS");
    __shared__ SegSmem<kModeOut> sm;

    // XCD-aware placement: workgroups are dealt round-robin to the 8 XCDs
    // (bid % 8). The V heads of one (segment, QK head) - which read the same K
    // and Q - get consecutive slots on the XCD (segment * Hqk + QK head) % 8.
    const int group = num_v_heads / num_qk_heads;
    const int xcd = blockIdx.x & 7;
    const int64_t kx = blockIdx.x >> 3;
    const int vh = (int)(kx % group);
    const int64_t u = 8 * (kx / group) + xcd;            // (segment, QK head) unit
    if (u >= num_segs * num_qk_heads) return;
    SegTask tk;
    tk.sg = u / num_qk_heads;
    tk.hq = (int)(u % num_qk_heads);
    tk.h = tk.hq * group + vh;
    tk.n = find_seq_for_seg(cu, num_seqs, tk.sg, L);
    tk.sr = seq_range(cu, tk.n, total_tokens);
    tk.j = tk.sg - seg_base(cu, tk.n, L);
    const int64_t nch = (tk.sr.eos - tk.sr.bos + kChunk - 1) / kChunk;
    tk.nseg = nch > 0 ? (nch + L - 1) / L : 1;               // an empty sequence still copies its state
    if (tk.j < 0 || tk.j >= tk.nseg) return;                  // unused segment index
    tk.c_begin = tk.j * L;
    tk.c_end = (tk.c_begin + L < nch) ? tk.c_begin + L : nch;
    tk.nchunks = tk.c_end - tk.c_begin;
    const SegArgs A = {q, k, v, g, beta, initial_state, final_state, out, segws, state_indices, has_initial,
                       num_slots, num_qk_heads, num_v_heads, scale};
    if (phase == 0) {
        if (tk.j == 0) segment_body<kModeOut, QKN>(sm, A, tk);
        else if (tk.j < tk.nseg - 1)
            segment_body<kModeHM, QKN>(*reinterpret_cast<SegSmem<kModeHM>*>(&sm), A, tk);
    } else if (tk.j > 0) {
        segment_body<kModeOut, QKN>(sm, A, tk);
    }
}


// Combine: for each (sequence, V head, block of 16 state rows), walk the
// sequence's segments: S_in(1) = H_0, S_in(j+1) = S_in(j) M_j + H_j; S_in(j) is
// stored for pass C. Each wave computes 32 of the 128 columns with the products
// split into bf16 parts on MFMA 16x16x32 (fp32 accumulation; S_in, M and H stay
// fp32 in memory and the split keeps about fp32 accuracy);
// M_{j+1} and H_{j+1} do not depend on the recurrence and are loaded during
// step j, so only the 16 rows of S_in pass through LDS between steps. The row
// blocks of one (sequence, head) are consecutive in units of the head count,
// which puts them on one XCD (blocks go round-robin to the 8 XCDs) when the
// head count is a multiple of 8: M_j then comes from HBM once.
// x = hi + lo in bf16 (hi = x rounded to nearest even, lo = the rest rounded): the products below
// take hi·hi + hi·lo + lo·hi, which leaves out lo·lo (at most 2^-18 of the product); with the
// rounding of lo the error stays near 1e-5 of each product, on bf16 MFMA.
__device__ __forceinline__ void split_bf16x8(const float (&x)[8], bf16x8& hi, bf16x8& lo) {
    u32x4 h, l;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t ph = pack_bf16(x[2 * i], x[2 * i + 1]);
        const float r0 = x[2 * i] - __uint_as_float(ph << 16);
        const float r1 = x[2 * i + 1] - __uint_as_float(ph & 0xFFFF0000u);
        h[i] = ph;
        l[i] = pack_bf16(r0, r1);
    }
    hi = __builtin_bit_cast(bf16x8, h);
    lo = __builtin_bit_cast(bf16x8, l);
}

__global__ __launch_bounds__(256) void combine_kernel(const int32_t* __restrict__ cu, float* __restrict__ segws,
                                                      int64_t total_tokens, int32_t num_seqs, int32_t num_v_heads,
                                                      int32_t L) {
    __shared__ float Srow[16][D + 4];
    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, g = lane >> 4, m = lane & 15;
    const int64_t nh = (int64_t)num_seqs * num_v_heads;
    const int64_t u = blockIdx.x % nh;
    const int rb = (int)(blockIdx.x / nh);
    const int h = (int)(u % num_v_heads), n = (int)(u / num_v_heads);
    const SeqRange sr = seq_range(cu, n, total_tokens);
    const int64_t nch = (sr.eos - sr.bos + kChunk - 1) / kChunk;
    const int64_t nseg = (nch + L - 1) / L;
    if (nseg < 2) return;
    const int64_t s0 = seg_base(cu, n, L);
    auto mat = [&](int64_t jseg, int which) {
        return segws + (((size_t)(s0 + jseg) * num_v_heads + h) * kSegMats + which) * kSegMat;
    };
    const int r0 = 16 * rb, cb = 32 * w;
    // Lane (g, m) of tile ct: rows r0 + 4 g + e, column cb + 16 ct + m.
    auto load_rows = [&](const float* X, f32x4 (&t)[2]) {
#pragma unroll
        for (int ct = 0; ct < 2; ++ct)
#pragma unroll
            for (int e = 0; e < 4; ++e) t[ct][e] = X[(size_t)(r0 + 4 * g + e) * D + cb + 16 * ct + m];
    };
    // B operand of M (16x16x32 bf16 layout): rows 32 kk + 8 g + i, column cb + 16 ct + m.
    auto load_m = [&](const float* M, float (&b)[4][2][8]) {
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
#pragma unroll
            for (int ct = 0; ct < 2; ++ct)
#pragma unroll
                for (int i = 0; i < 8; ++i) b[kk][ct][i] = M[(size_t)(32 * kk + 8 * g + i) * D + cb + 16 * ct + m];
    };
    f32x4 acc[2], hn[2];
    float bm[4][2][8];
    load_rows(mat(0, 0), acc);                 // S_in(1) = H_0
    if (nseg > 2) {
        load_m(mat(1, 1), bm);
        load_rows(mat(1, 0), hn);
    }
    for (int64_t jj = 1; jj < nseg; ++jj) {
        float* Sin = mat(jj, 2);
#pragma unroll
        for (int ct = 0; ct < 2; ++ct)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                Sin[(size_t)(r0 + 4 * g + e) * D + cb + 16 * ct + m] = acc[ct][e];
                Srow[4 * g + e][cb + 16 * ct + m] = acc[ct][e];
            }
        if (jj == nseg - 1) break;
        __syncthreads();
        // S_in(jj + 1) = S_in(jj) M_jj + H_jj
        acc[0] = hn[0];
        acc[1] = hn[1];
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            float a8[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) a8[i] = Srow[m][32 * kk + 8 * g + i];
            bf16x8 ah, al;
            split_bf16x8(a8, ah, al);
#pragma unroll
            for (int ct = 0; ct < 2; ++ct) {
                bf16x8 bh, bl;
                split_bf16x8(bm[kk][ct], bh, bl);
                acc[ct] = mfma16(al, bh, acc[ct]);
                acc[ct] = mfma16(ah, bl, acc[ct]);
                acc[ct] = mfma16(ah, bh, acc[ct]);
            }
        }
        if (jj + 1 < nseg - 1) {
            load_m(mat(jj + 1, 1), bm);
            load_rows(mat(jj + 1, 0), hn);
        }
        __syncthreads();
    }
}

int64_t num_segments(int64_t total_tokens, int32_t num_seqs, int L) {
    return total_tokens / ((int64_t)kChunk * L) + num_seqs;
}

}  // namespace

// Chunks per segment. Each of the two segment launches holds about one
// (segment, V head) task per CU (one workgroup fits a CU): a sequence with G
// segments contributes G - 1 tasks per V head to each launch, so G - 1 =
// CUs / Hv segments per sequence, with enough chunks per segment to amortise
// the map work (at least 8).
int cp_segment_chunks(int64_t total_tokens, int32_t num_seqs, int32_t num_v_heads) {
    // The compute-unit count of the current device, looked up on every call (the runtime answers
    // from its own per-device table), so that each device gets its own segment length.
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
        cus = 256;
    const int64_t chunks = (total_tokens + kChunk - 1) / kChunk;
    const int64_t per_head = cus / num_v_heads > 1 ? cus / num_v_heads : 1;
    int64_t L = (chunks + per_head + num_seqs - 1) / (per_head + num_seqs);
    if (L < 8) L = 8;
    if (L > (1 << 24)) L = 1 << 24;
    return (int)L;
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
    // Phase 0 (segment 0's outputs and the other segments' maps) always runs;
    // the combine and phase 1 only when some sequence spans more than one segment.
    const bool multi = a.num_seqs > 1 || a.total_tokens > (int64_t)kChunk * L;
    auto kern = a.qk_norm ? segment_kernel<true> : segment_kernel<false>;
    prof::begin(stream, multi ? "gdn_segment_maps" : "gdn_segment_out");
    hipLaunchKernelGGL(kern, grid, dim3(64 * (4 + kProd)), 0, stream, q, k, v, a.g, a.beta, a.initial_state,
                       a.cu_seqlens, a.final_state, (uint16_t*)a.out, seg_ws, a.total_tokens, a.num_seqs,
                       a.num_qk_heads, a.num_v_heads, L, segs, a.scale, 0, a.state_indices, a.has_initial,
                       a.num_slots);
    prof::end(stream);
    if (multi) {
        prof::begin(stream, "gdn_segment_combine");
        hipLaunchKernelGGL(combine_kernel, dim3((unsigned)((int64_t)a.num_seqs * a.num_v_heads * 8)), dim3(256), 0,
                           stream, a.cu_seqlens, seg_ws, a.total_tokens, a.num_seqs, a.num_v_heads, L);
        prof::end(stream);
        prof::begin(stream, "gdn_segment_out");
        hipLaunchKernelGGL(kern, grid, dim3(64 * (4 + kProd)), 0, stream, q, k, v, a.g, a.beta,
                           a.initial_state, a.cu_seqlens, a.final_state, (uint16_t*)a.out, seg_ws, a.total_tokens,
                           a.num_seqs, a.num_qk_heads, a.num_v_heads, L, segs, a.scale, 1, a.state_indices,
                           a.has_initial, a.num_slots);
        prof::end(stream);
    }
    return hipGetLastError();
}

size_t prefill_bf16_workspace_bytes(int64_t total_tokens, int32_t num_seqs, int32_t num_qk_heads,
                                    int32_t num_v_heads) {
    (void)num_qk_heads;
    return cp_segment_workspace_bytes(total_tokens, num_seqs, num_v_heads);
}

}  // namespace gdn
