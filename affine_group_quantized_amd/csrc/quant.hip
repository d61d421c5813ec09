// Affine group quantizer on the GPU: weights (fp32 or bf16) [N, K] to U32-packed
// 2-, 3-, 4-, 5-, 6- or 8-bit codes with BF16 scale and bias per group of 32,
// 64 or 128 columns, the format the products read: each row's codes form one
// low-first bit stream (code k at stream bits bits*k .. bits*k + bits - 1). It moves the quantization step onto the device
// ("MLX CUDA Cleanup Plan", Phase 5: repeated host-side quantization is one of
// the per-op overheads to remove; the epic's Phase 5 quantized KV cache, #635,
// quantizes on the device too).
//
// The recipe, per row and group, in binary32:
//   scale = bf16((max - min) / (2^bits - 1)),  bias = bf16(min),
//   q = clamp(rint((w - bias) / scale), 0, 2^bits - 1)    (q = 0 where scale is 0)
// with correctly rounded division, rint rounding half to even, and the
// rounded scale and bias. Every step is a single IEEE operation, so the codes
// are bit-identical to any other correct implementation of the recipe.
//
// One thread per group: a first pass over the group's values finds max and
// min, a second (from cache) forms the codes and stores each packed word as
// the stream fills it (a group is a whole number of words: 32 * bits bits per
// 32 columns).

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qmv_device.hpp"

namespace agq {

namespace {

template <typename IN>
__device__ __forceinline__ float load_w(const IN *p);
template <>
__device__ __forceinline__ float load_w<float>(const float *p) {
    return *p;
}
template <>
__device__ __forceinline__ float load_w<uint16_t>(const uint16_t *p) {
    return bf16_lo(*p);
}

}  // namespace

template <int BITS, typename IN>
__global__ __launch_bounds__(256) void quantize_kernel(const IN *__restrict__ w, int64_t groups, int64_t K,
                                                       int gs, uint32_t *__restrict__ wq,
                                                       uint16_t *__restrict__ sc, uint16_t *__restrict__ bi) {
    constexpr float kLevels = (float)((1 << BITS) - 1);
    const int64_t gpr = K / gs;  // groups per row
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < groups;
         i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t row = i / gpr, g = i - row * gpr;
        const IN *src = w + row * K + g * gs;
        float mx = load_w(src), mn = mx;
        for (int j = 1; j < gs; ++j) {
            const float v = load_w(src + j);
            mx = v > mx ? v : mx;
            mn = v < mn ? v : mn;
        }
        const uint16_t s16 = f32_to_bf16(__fdiv_rn(mx - mn, kLevels));
        const uint16_t b16 = f32_to_bf16(mn);
        sc[i] = s16;
        bi[i] = b16;
        const float s = bf16_lo(s16), b = bf16_lo(b16);
        uint32_t *dst = wq + row * (K / 32 * BITS) + g * (gs / 32 * BITS);
        uint64_t bitbuf = 0;  // stream bits not yet stored, low-first
        int nbits = 0;
        for (int j = 0; j < gs; ++j) {
            uint32_t q = 0;
            if (s != 0.f) {
                const float r = rintf(__fdiv_rn(load_w(src + j) - b, s));
                q = r <= 0.f ? 0u : r >= kLevels ? (uint32_t)kLevels : (uint32_t)r;
            }
            bitbuf |= (uint64_t)q << nbits;
            nbits += BITS;
            if (nbits >= 32) {
                *dst++ = (uint32_t)bitbuf;
                bitbuf >>= 32;
                nbits -= 32;
            }
        }
    }
}

template <int BITS>
static const void *quantize_pick(bool bf16_in) {
    return bf16_in ? reinterpret_cast<const void *>(&quantize_kernel<BITS, uint16_t>)
                   : reinterpret_cast<const void *>(&quantize_kernel<BITS, float>);
}

const void *quantize_kernel_for(int bits, bool bf16_in) {
    switch (bits) {
        case 2: return quantize_pick<2>(bf16_in);
        case 3: return quantize_pick<3>(bf16_in);
        case 4: return quantize_pick<4>(bf16_in);
        case 5: return quantize_pick<5>(bf16_in);
        case 6: return quantize_pick<6>(bf16_in);
        case 8: return quantize_pick<8>(bf16_in);
    }
    return nullptr;
}

}  // namespace agq
