// Argument block and kernel lookup of the quantized GEMM kernels (qmm_mfma.hip).
#pragma once

#include <stdint.h>

#include "qmv_kernels.hpp"

namespace agq {

// Tile shape: a block of 4 waves computes 32*kQmmTM activation rows by
// 32*kQmmTN weight rows; global loads run kQmmDepth 64-column groups ahead.
constexpr int kQmmTM = 2;
constexpr int kQmmTN = 4;
constexpr int kQmmDepth = 4;

// Passed by value as the single kernel argument.
struct QmmArgs {
    const uint16_t *x;    // activation rows, bf16 [M or R, K]
    const uint32_t *w;    // packed codes [planes, N, K*bits/32]
    const uint16_t *s;    // bf16 scales [planes, N, K/64]
    const uint16_t *b;    // bf16 biases [planes, N, K/64]
    uint16_t *y;          // bf16 outputs [M or P, N]
    const uint32_t *lhs;  // gather: x row per pair (NULL = identity)
    const uint32_t *rhs;  // gather: expert per pair (NULL = identity)
    int64_t N;            // weight rows per plane
    int32_t M;            // activation rows (dense) or pairs P (gather)
    int32_t K;            // columns
    int32_t G;            // 64-column groups per row
    int32_t rowbytes;     // bytes of codes per weight row
    uint32_t xbytes;      // bytes of x (the range of its buffer descriptor)
    int32_t R_x;          // gather: rows of x
    int32_t E;            // gather: expert planes
    int32_t pad_;
};

struct QmmKernel {
    const void *sym = nullptr;
    int bm = 0, bn = 0;  // tile rows of x and of W
    int lds = 0;         // dynamic LDS bytes of the tile buffers
};

QmmKernel qmm_kernel_for(int bits, bool gather);

}  // namespace agq
