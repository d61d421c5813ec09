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

typedef float f32x2 __attribute__((ext_vector_type(2)));

// Both bfloat16 values of a pair times rs and times the matching norm weight,
// each product rounded once to bfloat16: (x * rs) * g in fp32, then to nearest
// even (one v_cvt_pk_bf16_f32 for the pair).
__device__ __forceinline__ uint32_t norm_pair(uint32_t x, uint32_t g, float rs) {
    const f32x2 v = {bf16_lo(x) * rs * bf16_lo(g), bf16_hi(x) * rs * bf16_hi(g)};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// c + a.lo*b.lo + a.hi*b.hi on bfloat16 pairs (v_dot2c_f32_bf16), fp32 accumulate.
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c,
                                           false);
}

// A 4-bit code q placed in the low mantissa bits of bfloat16 0x4300 (= 128.0)
// reads as the exact value 128 + q. For a packed word w holding the codes
// q0..q7 of eight consecutive columns (low-first), lo = w & 0x0F0F0F0F has
// bytes (q0, q2, q4, q6) and hi = (w >> 4) & 0x0F0F0F0F has (q1, q3, q5, q7).
// One byte permute against 0x43 bytes then yields the bfloat16 pair
// (128 + q_a, 128 + q_b):
//   perm(.., lo, kSelEven) = (q0, q4)   perm(.., lo, kSelOdd) = (q2, q6)
//   perm(.., hi, kSelEven) = (q1, q5)   perm(.., hi, kSelOdd) = (q3, q7)
// That is 7 VALU ops for 8 codes (and, shift, and, 4 v_perm_b32).
constexpr uint32_t kMagic43 = 0x43434343u;
constexpr uint32_t kSelEven = 0x04020400u;  // bytes: lo.b0, 0x43, lo.b2, 0x43
constexpr uint32_t kSelOdd = 0x04030401u;   // bytes: lo.b1, 0x43, lo.b3, 0x43

__device__ __forceinline__ uint32_t byte_perm(uint32_t hi_src, uint32_t lo_src, uint32_t sel) {
    return __builtin_amdgcn_perm(hi_src, lo_src, sel);
}

// Wave index within the block, as a wave-uniform (scalar) value.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// One halving step of a transposed wave reduction. For lanes l < 32 the swap
// returns (a[l], a[l+32]); for l >= 32 it returns (b[l-32], b[l]). The sum
// therefore holds a's 32 pair sums in the low half and b's in the high half:
// two vectors fold into one with one swap and one add.
__device__ __forceinline__ float fold32(float a, float b) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// The same step inside each 32-lane half: lanes [0,16) of a half get a's sums
// l + (l+16), lanes [16,32) get b's.
__device__ __forceinline__ float fold16(float a, float b) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Sum over the 16 lanes of each row, the same bits in every lane of the row:
// DPP butterflies over lane pairs l^1, l^2, then the half-row and row mirrors.
__device__ __forceinline__ float row_sum16(float v) {
    v += dpp_f32<0xB1>(v);   // quad_perm [1,0,3,2]
    v += dpp_f32<0x4E>(v);   // quad_perm [2,3,0,1]
    v += dpp_f32<0x141>(v);  // row_half_mirror
    v += dpp_f32<0x140>(v);  // row_mirror
    return v;
}

// Wave sums of V lane-partial vectors at once. Value i ends up in every lane of
// 16-lane row rho of t[i / 4], where i % 4 == sum_slot(rho). Every value is
// summed by the same tree (pairs l^32, l^16, l^1, l^2, then the mirrors) and
// floating-point addition is commutative, so a value's bits do not depend on
// its slot. Every lane of the wave must be active.
constexpr int sum_regs(int V) { return (V + 3) / 4; }
__device__ __forceinline__ int sum_slot(int rho) { return ((rho & 1) << 1) | (rho >> 1); }

template <int V>
__device__ __forceinline__ void wave_sums(const float (&v)[V], float (&t)[sum_regs(V)]) {
    constexpr int NU = (V + 1) / 2;
    float u[NU];
#pragma unroll
    for (int i = 0; i < NU; ++i) u[i] = fold32(v[2 * i], 2 * i + 1 < V ? v[2 * i + 1] : 0.f);
#pragma unroll
    for (int j = 0; j < sum_regs(V); ++j) t[j] = row_sum16(fold16(u[2 * j], 2 * j + 1 < NU ? u[2 * j + 1] : 0.f));
}

}  // namespace agq
