// Internal helpers shared by the libgdn kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

// Widening of a bfloat16 bit pattern (exact).
__device__ __forceinline__ float bf16_bits_to_float(uint16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// fp32 -> bf16 bits, round to nearest even (inputs are finite here).
__device__ __forceinline__ uint16_t float_to_bf16_bits(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return static_cast<uint16_t>(u >> 16);
}

// exp of a non-positive argument through the hardware exp2.
__device__ __forceinline__ float exp_nonpos(float x) {
    return exp2f(x * 1.4426950408889634f);
}

// DPP lane exchanges inside a row of 16 lanes. Sums over groups of 2, 4 or 8
// adjacent lanes: after the quad-level steps every lane of a quad holds the
// quad sum, and the half-row mirror pairs each lane with one of the other quad.
__device__ __forceinline__ float dpp_quad_xor1(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false));
}
__device__ __forceinline__ float dpp_quad_xor2(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, false));
}
// Mirror inside the row of 16 (lane i <-> 15 - i): after the 8-lane sums it
// pairs each lane with one of the other half row.
__device__ __forceinline__ float dpp_row_mirror(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x140, 0xF, 0xF, false));
}

__device__ __forceinline__ float dpp_half_mirror(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x141, 0xF, 0xF, false));
}

template <int L>
__device__ __forceinline__ float group_sum(float x) {
    static_assert(L == 1 || L == 2 || L == 4 || L == 8 || L == 16, "group of 1, 2, 4, 8 or 16 lanes");
    if constexpr (L >= 2) x += dpp_quad_xor1(x);
    if constexpr (L >= 4) x += dpp_quad_xor2(x);
    if constexpr (L >= 8) x += dpp_half_mirror(x);
    if constexpr (L >= 16) x += dpp_row_mirror(x);
    return x;
}

}  // namespace gdn
