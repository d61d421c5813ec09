// Argument block and kernel lookup of the fused decode-MoE kernels (moe_mfma.hip).
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace agq {

constexpr int kMoeMaxTokens = 256;  // tokens per call

// Passed by value as the single kernel argument of both launches.
struct MoeArgs {
    const uint16_t *x;        // tokens [T, H] bf16
    uint16_t *h;              // workspace [2P, F] bf16: per pair the hi and lo rows of silu(gate) * up
    float *o;                 // workspace [P, H] fp32: per pair the router-weighted down projection
    uint16_t *y;              // [T, H] bf16
    const uint32_t *wg;       // gate planes [E, F, H/8] (4-bit codes)
    const uint16_t *sg, *bg;  // [E, F, H/64]
    const uint32_t *wu;       // up planes [E, F, H/8]
    const uint16_t *su, *bu;
    const uint32_t *wd;       // down planes [E, H, F/8]
    const uint16_t *sd, *bd;  // [E, H, F/64]
    const uint32_t *experts;  // [T, k] expert per pair (pair p = t*k + j)
    const float *weights;     // [T, k] router weight per pair
    int32_t T, k, P, E;
    int64_t H, F;
    int32_t S1, SPW1, BPG1;   // gate/up launch: waves per block, segments per wave, bands per block
    int32_t S2, SPW2, BPG2;   // down launch: the same
};

// stage 0: moe_gate_up_kernel; 1: moe_down_kernel with bands of 16*tiles rows;
// 2: moe_combine_kernel.
const void *moe_kernel(int stage, int tiles);

// Bytes of the per-device scratch array of the allocation-free MoE call
// (agq_moe_decode_noalloc): 8 MiB, room for 4*T*k*(F + H) bytes of h and o
// (16 tokens top-2 at H = 4096, F = 14336 take 2.3 MiB).
constexpr int64_t kMoeScratchBytes = int64_t(8) << 20;

// Device address of the scratch array on device `dev` (the current device),
// looked up once per device.
hipError_t moe_scratch(int dev, void **ptr);

}  // namespace agq
