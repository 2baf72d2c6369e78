// MFMA / LDS helpers for the bf16 prefill kernels (gfx950, wave64,
// v_mfma_f32_16x16x32_bf16).
//
// MFMA 16x16x32 bf16 operand layout (lane l, g = l / 16, m = l % 16):
//   A (16 x 32): row m, reduction indices 8 g .. 8 g + 7
//   B (32 x 16): column m, reduction indices 8 g .. 8 g + 7
//   D (16 x 16): column m, rows 4 g .. 4 g + 3
// Because only the pairing of A and B reduction slots matters, an operand can
// be fed straight from accumulator tiles by listing a k-step's 32 reduction
// indices in accumulator order: slot s of lane group g stands for index
// 16 (s / 4) + 4 g + (s % 4) (two accumulator tiles, four rows each).
#pragma once

#include "gdn_common.h"
#include "gdn_internal.h"

namespace gdn {
namespace mf {

constexpr int D = 128;
constexpr int RP = D + 8;          // padded bf16 row of a 64 x 128 tile
constexpr int CP = kChunk + 8;     // padded bf16 row of a 64 x 64 tile / a transposed K row

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// Workgroup barrier that orders LDS only. The waves of these kernels exchange
// data through LDS alone, so global loads (the next chunk's prefetch) and
// stores stay in flight across it; __syncthreads() would wait for them.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

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

// Standard-order operand: row `row`, columns 32 k + 8 g .. +7 (one 16-byte read).
__device__ __forceinline__ bf16x8 lds_row8(const uint16_t* tile, int ld, int row, int k, int g) {
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(tile + row * ld + 32 * k + 8 * g));
}

typedef short i16x4 __attribute__((ext_vector_type(4)));

// LDS transpose read (ds_read_b64_tr_b16): within each group of 16 lanes, lane
// i addresses 4 consecutive 16-bit values D[i][0..3]; lane j receives
// D[4 e + j / 4][j % 4] for e = 0..3.
__device__ __forceinline__ i16x4 lds_read_tr16(const uint16_t* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(p));
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

}  // namespace mf
}  // namespace gdn
