// Device helpers for the affine group-quantized matvec kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qmv_kernels.hpp"

namespace agq {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// bfloat16 is the high half of a binary32: widening is a shift and is exact.
__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xFFFF0000u); }

// binary32 -> bfloat16, round to nearest even; NaN stays NaN (quieted).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// c + a.lo*b.lo + a.hi*b.hi on bfloat16 pairs (v_dot2c_f32_bf16), fp32 accumulate.
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c,
                                           false);
}

// A 4-bit code q placed in the low mantissa bits of bfloat16 0x4300 (= 128.0)
// reads as the exact value 128 + q. For packed word `w` (codes q0..q7 of eight
// consecutive columns, low-first) this yields the bfloat16 pair
// (128 + q_i, 128 + q_{i+4}) with one shift and one AND-OR.
template <int I>
__device__ __forceinline__ uint32_t nibble_pair(uint32_t w) {
    return ((w >> (4 * I)) & 0x000F000Fu) | 0x43004300u;
}

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

__device__ __forceinline__ float readlane_f32(float v, int lane) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

// Sum over the 64 lanes of a wave, the same bits in every lane. DPP butterflies
// (quad swaps, then half-row and row mirrors) leave each 16-lane row holding its
// row sum in every lane; the four row sums are then added in a fixed order.
// Every lane of the wave must be active.
__device__ __forceinline__ float wave_sum(float v) {
    v += dpp_f32<0xB1>(v);   // quad_perm [1,0,3,2]
    v += dpp_f32<0x4E>(v);   // quad_perm [2,3,0,1]
    v += dpp_f32<0x141>(v);  // row_half_mirror
    v += dpp_f32<0x140>(v);  // row_mirror
    return (readlane_f32(v, 0) + readlane_f32(v, 16)) + (readlane_f32(v, 32) + readlane_f32(v, 48));
}

}  // namespace agq
