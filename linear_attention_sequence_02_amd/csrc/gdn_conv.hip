// Input prologue of the mixer: the short depthwise causal convolution over the
// q, k and v channels (the causal-conv1d step the model card points to beside
// flash-linear-attention), an optional SiLU, the split into the q, k and v
// arrays the mixer reads, and optionally the per-head L2 normalisation of q
// and k. HBM-bound: every input is read once (plus K - 1 rows of history per
// 64-token tile) and every output written once.
//
// Channel c of a token row: q for c < Hqk d, then k, then v. Per channel,
//   y_t[c] = sum_{i < K} w[c][i] x_{t-K+1+i}[c]
// with x before a sequence's first token taken from its history rows (the K-1
// inputs of an earlier call, oldest first) or zero.
//
// Launch 1 (one workgroup per (64-token tile of a sequence, 2048 channels),
// eight channels per lane): outputs. The token rows are read and the outputs
// written with non-temporal accesses (each is touched once; 0.436 -> 0.393 ms
// at T = 65536, and 64-token tiles instead of 32, which halves the re-read
// history rows, 0.389 ms). Launch 2 (one lane per (sequence, eight
// channels)): each sequence's new history, its last K - 1 inputs; every lane
// reads all its rows before writing any, so the new history may overwrite the
// old one in place.
#include "gdn_common.h"
#include "gdn_internal.h"

namespace gdn {

namespace {

constexpr int kTile = 64;            // tokens per tile
constexpr int kLaneCh = 8;           // channels per lane
constexpr int kBlock = 256;          // threads per workgroup
constexpr int kGroupCh = kBlock * kLaneCh;

typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef unsigned int u32x4v __attribute__((ext_vector_type(4)));

struct ConvArgs {
    const void* x;
    const float* w;
    const void* hist_in;
    void* hist_out;
    const int32_t* cu;
    void* q;
    void* k;
    void* v;
    int64_t total_tokens;
    int32_t num_seqs, hqk, hv, d, K, C;
    bool silu, qk_norm;
};

// Sequence n's first and last token: from cu_seqlens, else equal-length sequences.
__device__ __forceinline__ void seq_bounds(const ConvArgs& a, int n, int64_t& bos, int64_t& eos) {
    if (a.cu) {
        bos = a.cu[n];
        eos = a.cu[n + 1];
    } else {
        const int64_t len = a.total_tokens / a.num_seqs;
        bos = (int64_t)n * len;
        eos = bos + len;
    }
}

// Tiles of sequence n occupy slots [base(n), base(n) + ceil(len / 32)), base(n) = bos / 32 + n:
// disjoint ranges below total_tokens / 32 + num_seqs.
__device__ __forceinline__ int64_t tile_base(const ConvArgs& a, int n) {
    int64_t bos, eos;
    seq_bounds(a, n, bos, eos);
    return bos / kTile + n;
}

// One lane's eight channels of a row as loaded (bf16: one 16-byte word; fp32: two).
template <bool BF16>
struct RawRow {
    u32x4v u[BF16 ? 1 : 2];
};

template <bool BF16>
__device__ __forceinline__ RawRow<BF16> load_raw(const void* p, int64_t elem) {
    RawRow<BF16> r;
    if constexpr (BF16) {
        r.u[0] = __builtin_nontemporal_load(reinterpret_cast<const u32x4v*>(reinterpret_cast<const uint16_t*>(p) + elem));
    } else {
        r.u[0] = __builtin_nontemporal_load(reinterpret_cast<const u32x4v*>(reinterpret_cast<const float*>(p) + elem));
        r.u[1] = __builtin_nontemporal_load(reinterpret_cast<const u32x4v*>(reinterpret_cast<const float*>(p) + elem + 4));
    }
    return r;
}

template <bool BF16>
__device__ __forceinline__ f32x8 widen(const RawRow<BF16>& r) {
    f32x8 f;
    if constexpr (BF16) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            f[2 * j] = __uint_as_float(r.u[0][j] << 16);
            f[2 * j + 1] = __uint_as_float(r.u[0][j] & 0xFFFF0000u);
        }
    } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            f[j] = __uint_as_float(r.u[0][j]);
            f[4 + j] = __uint_as_float(r.u[1][j]);
        }
    }
    return f;
}

template <bool BF16>
__device__ __forceinline__ f32x8 load8(const void* p, int64_t elem) {
    f32x8 r;
    if constexpr (BF16) {
        const u32x4v u = *reinterpret_cast<const u32x4v*>(reinterpret_cast<const uint16_t*>(p) + elem);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            r[2 * j] = __uint_as_float(u[j] << 16);
            r[2 * j + 1] = __uint_as_float(u[j] & 0xFFFF0000u);
        }
    } else {
        const float4 a = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(p) + elem);
        const float4 b = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(p) + elem + 4);
        r[0] = a.x; r[1] = a.y; r[2] = a.z; r[3] = a.w;
        r[4] = b.x; r[5] = b.y; r[6] = b.z; r[7] = b.w;
    }
    return r;
}

typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
typedef float f32x2v __attribute__((ext_vector_type(2)));

// Two floats -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack2_bf16(float lo, float hi) {
    const f32x2v x = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf16x2v));
}

template <bool BF16>
__device__ __forceinline__ void store8(void* p, int64_t elem, const f32x8& y) {
    if constexpr (BF16) {
        u32x4v u;
#pragma unroll
        for (int j = 0; j < 4; ++j) u[j] = pack2_bf16(y[2 * j], y[2 * j + 1]);
        __builtin_nontemporal_store(u, reinterpret_cast<u32x4v*>(reinterpret_cast<uint16_t*>(p) + elem));
    } else {
        float* f = reinterpret_cast<float*>(p) + elem;
        *reinterpret_cast<float4*>(f) = make_float4(y[0], y[1], y[2], y[3]);
        *reinterpret_cast<float4*>(f + 4) = make_float4(y[4], y[5], y[6], y[7]);
    }
}

// Sum over the d / 8 lanes that hold one head's channels.
__device__ __forceinline__ float head_sum(float x, int d) {
    if (d == 16) return group_sum<2>(x);
    if (d == 32) return group_sum<4>(x);
    if (d == 64) return group_sum<8>(x);
    return group_sum<16>(x);
}

template <bool BF16, int K>
__global__ __launch_bounds__(kBlock) void conv_out_kernel(ConvArgs a) {
    // The tile: its sequence (binary search over the slot bases) and tokens.
    const int64_t slot = blockIdx.x;
    int lo = 0, hi = a.num_seqs - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (tile_base(a, mid) <= slot) lo = mid;
        else hi = mid - 1;
    }
    const int n = lo;
    int64_t bos, eos;
    seq_bounds(a, n, bos, eos);
    const int64_t t0 = bos + (slot - tile_base(a, n)) * kTile;
    if (t0 >= eos) return;   // a slot between two sequences' ranges (whole workgroup)
    const int64_t t1 = t0 + kTile < eos ? t0 + kTile : eos;

    const int c0 = blockIdx.y * kGroupCh + threadIdx.x * kLaneCh;
    const bool active = c0 < a.C;
    const int cc = active ? c0 : 0;   // idle lanes (past the last channel) read channel 0 and store nothing

    float w[K][kLaneCh];
#pragma unroll
    for (int j = 0; j < kLaneCh; ++j)
#pragma unroll
        for (int i = 0; i < K; ++i) w[i][j] = a.w[(int64_t)(cc + j) * K + i];

    // Window: win[i] = x_{t-K+1+i} for the next token t.
    f32x8 win[K];
#pragma unroll
    for (int i = 0; i < K - 1; ++i) {
        const int64_t s = t0 - (K - 1) + i;
        if (s >= bos) {
            win[i] = load8<BF16>(a.x, s * a.C + cc);
        } else if (a.hist_in) {
            win[i] = load8<BF16>(a.hist_in, ((int64_t)n * (K - 1) + (s - bos + K - 1)) * a.C + cc);
        } else {
#pragma unroll
            for (int j = 0; j < kLaneCh; ++j) win[i][j] = 0.f;
        }
    }

    const int nq = a.hqk * a.d;
    const bool is_qk = cc < 2 * nq;
    void* dst;
    int64_t dst_ld, dst_c;
    if (cc < nq) {
        dst = a.q; dst_ld = nq; dst_c = cc;
    } else if (cc < 2 * nq) {
        dst = a.k; dst_ld = nq; dst_c = cc - nq;
    } else {
        dst = a.v; dst_ld = (int64_t)a.hv * a.d; dst_c = cc - 2 * nq;
    }

    // Batches of eight tokens: the batch's rows are all requested before the first is used.
    for (int64_t tb = t0; tb < t1; tb += 8) {
        RawRow<BF16> raw[8];
#pragma unroll
        for (int u = 0; u < 8; ++u)
            if (tb + u < t1) raw[u] = load_raw<BF16>(a.x, (tb + u) * a.C + cc);
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            if (tb + u >= t1) break;
            win[K - 1] = widen<BF16>(raw[u]);
            f32x8 y;
#pragma unroll
            for (int j = 0; j < kLaneCh; ++j) {
                float acc = 0.f;
#pragma unroll
                for (int i = 0; i < K; ++i) acc = fmaf(w[i][j], win[i][j], acc);
                y[j] = acc;
            }
            if (a.silu) {
                // y * sigmoid(y) = y / (1 + e^-y), with the hardware exp2 and reciprocal (about 1 ulp
                // each); for y below about -88 the exponential overflows and the result is -0.
#pragma unroll
                for (int j = 0; j < kLaneCh; ++j)
                    y[j] = y[j] * __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(y[j] * -1.4426950408889634f));
            }
            if (a.qk_norm) {
                // Every lane takes part in the head-wide sums; only q and k heads are scaled.
                float ss = 0.f;
#pragma unroll
                for (int j = 0; j < kLaneCh; ++j) ss = fmaf(y[j], y[j], ss);
                const float r = rsqrtf(head_sum(ss, a.d) + kQkNormEps);
                if (is_qk) {
#pragma unroll
                    for (int j = 0; j < kLaneCh; ++j) y[j] *= r;
                }
            }
            if (active) store8<BF16>(dst, (tb + u) * dst_ld + dst_c, y);
#pragma unroll
            for (int i = 0; i < K - 1; ++i) win[i] = win[i + 1];
        }
    }
}

// New history of sequence n: row j is the input at relative position len - (K - 1) + j, from x when
// it is >= 0, else from the old history (row len + j) or zero.
template <bool BF16, int K>
__global__ __launch_bounds__(kBlock) void conv_hist_kernel(ConvArgs a) {
    const int n = blockIdx.x;
    const int c0 = blockIdx.y * kGroupCh + threadIdx.x * kLaneCh;
    if (c0 >= a.C || K < 2) return;
    int64_t bos, eos;
    seq_bounds(a, n, bos, eos);
    const int64_t len = eos - bos;
    f32x8 rows[K > 1 ? K - 1 : 1];
#pragma unroll
    for (int j = 0; j < K - 1; ++j) {
        const int64_t rel = len - (K - 1) + j;
        if (rel >= 0) {
            rows[j] = load8<BF16>(a.x, (bos + rel) * a.C + c0);
        } else if (a.hist_in) {
            rows[j] = load8<BF16>(a.hist_in, ((int64_t)n * (K - 1) + (len + j)) * a.C + c0);
        } else {
#pragma unroll
            for (int i = 0; i < kLaneCh; ++i) rows[j][i] = 0.f;
        }
    }
#pragma unroll
    for (int j = 0; j < K - 1; ++j) store8<BF16>(a.hist_out, ((int64_t)n * (K - 1) + j) * a.C + c0, rows[j]);
}

template <bool BF16, int K>
hipError_t launch_conv_k(const ConvArgs& a, hipStream_t stream) {
    const unsigned groups = (unsigned)((a.C + kGroupCh - 1) / kGroupCh);
    if (a.total_tokens > 0) {
        const int64_t slots = a.total_tokens / kTile + a.num_seqs;
        prof::begin(stream, "gdn_conv_prologue");
        hipLaunchKernelGGL((conv_out_kernel<BF16, K>), dim3((unsigned)slots, groups), dim3(kBlock), 0, stream, a);
        prof::end(stream);
    }
    if (a.hist_out && K > 1) {
        prof::begin(stream, "gdn_conv_history");
        hipLaunchKernelGGL((conv_hist_kernel<BF16, K>), dim3((unsigned)a.num_seqs, groups), dim3(kBlock), 0, stream, a);
        prof::end(stream);
    }
    return hipGetLastError();
}

template <bool BF16>
hipError_t launch_conv_t(const ConvArgs& a, hipStream_t stream) {
    switch (a.K) {
        case 1: return launch_conv_k<BF16, 1>(a, stream);
        case 2: return launch_conv_k<BF16, 2>(a, stream);
        case 3: return launch_conv_k<BF16, 3>(a, stream);
        default: return launch_conv_k<BF16, 4>(a, stream);
    }
}

}  // namespace

hipError_t launch_conv_prologue(const ConvPrologueArgs& p, hipStream_t stream) {
    ConvArgs a;
    a.x = p.x; a.w = p.weight; a.hist_in = p.conv_state_in; a.hist_out = p.conv_state_out; a.cu = p.cu_seqlens;
    a.q = p.q; a.k = p.k; a.v = p.v; a.total_tokens = p.total_tokens; a.num_seqs = p.num_seqs;
    a.hqk = p.num_qk_heads; a.hv = p.num_v_heads; a.d = p.d; a.K = p.kernel_size;
    a.C = 2 * p.num_qk_heads * p.d + p.num_v_heads * p.d;
    a.silu = p.silu; a.qk_norm = p.qk_norm;
    return p.bf16 ? launch_conv_t<true>(a, stream) : launch_conv_t<false>(a, stream);
}

}  // namespace gdn
