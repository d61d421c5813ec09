// Kernel argument block and kernel lookup shared by the launcher and the kernels.
#pragma once

#include <stdint.h>

namespace agq {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Passed by value as the single kernel argument.
struct ProductArgs {
    const uint16_t *x;    // activation rows, bf16 [rows, K]
    const u32x4 *w;       // packed codes in 16-byte chunks, [planes, N, C]
    const uint16_t *s;    // bf16 scales [planes, N, G]
    const uint16_t *b;    // bf16 biases [planes, N, G]
    uint16_t *y;          // bf16 outputs [M or P, N]
    const uint32_t *lhs;  // gather: x row per pair (NULL = identity)
    const uint32_t *rhs;  // gather: expert per pair (NULL = identity)
    int64_t N;            // weight rows per plane
    int64_t RPG;          // weight rows per row group
    int32_t K;            // columns
    int32_t C;            // 16-byte chunks per weight row
    int32_t G;            // 64-column groups per weight row
    int32_t M;            // activation rows (dense) or pairs P (gather)
    int32_t R_x;          // gather: rows of x
    int32_t E;            // gather: expert planes
    int32_t S;            // waves per row group (K split)
    int32_t GPB;          // row groups per block
    int32_t gshift;       // log2 of 16-byte chunks per scale group (group sizes 32, 64, 128)
    int32_t pad_;
};

// Argument block of the fused batch-1 projection: the product's arguments
// (one activation row) plus the norm weights, the norm's epsilon and 1/K, and
// the residual rows (each used only by the variants that have that stage).
struct FusedArgs {
    ProductArgs p;
    const uint16_t *gamma;  // bf16 [K]
    const uint16_t *res;    // bf16 [N]
    float eps;
    float inv_k;
    int32_t pad_[2];
};

// Argument block of the NVFP4 product (qmv_nvfp4.hip): 1-4 activation rows,
// E2M1 codes in 16-byte chunks of 32, one E4M3 byte per 16 columns.
struct Nvfp4Args {
    const uint16_t *x;  // activation rows, bf16 [M, K]
    const u32x4 *w;     // codes [N, C] chunks
    const uint8_t *s;   // E4M3 scales [N, K/16]
    uint16_t *y;        // bf16 outputs [M, N]
    int64_t N;          // weight rows
    int64_t RPG;        // weight rows per row group
    int32_t K;          // columns
    int32_t C;          // 16-byte chunks per row (K/32)
    int32_t S;          // waves per row group (K split)
    int32_t GPB;        // row groups per block
    float ts;           // tensor scale
    int32_t pad_[3];
};

// Argument block of the matrix-core kernels (4-bit codes, K a multiple of
// 512): bands of 16*T weight rows, S waves per block splitting K into slices
// of SPW 128-column segments, each block walking BPG bands round-robin.
struct MfmaArgs {
    const uint16_t *x;    // activation rows, bf16 [rows, K]
    const uint32_t *w;    // packed codes [planes, N, K/8]
    const uint16_t *s;    // bf16 scales [planes, N, K/64]
    const uint16_t *b;    // bf16 biases [planes, N, K/64]
    uint16_t *y;          // bf16 outputs [M or P, N]
    const uint32_t *lhs;  // gather: x row per pair (NULL = identity)
    const uint32_t *rhs;  // gather: expert per pair (NULL = identity)
    int64_t N;            // weight rows per plane
    int32_t K;            // columns
    int32_t G;            // 64-column groups per weight row
    int32_t M;            // activation rows (dense) or pairs P (gather)
    int32_t R_x;          // gather: rows of x
    int32_t E;            // gather: expert planes
    int32_t S;            // waves per block (K split)
    int32_t SPW;          // 128-column segments per wave (a multiple of 4)
    int32_t BPG;          // bands each block walks
    int32_t pad_[2];
};

// Kernel symbol for (bits, activation rows per pass, chunks per lane, weight
// rows per iteration, load ring stages, K segments per row group of a block's
// LDS copy of x (0: none)), or NULL.
const void *product_kernel(int bits, int mw, int cpt, int R, int NB, int x_lds, bool gather);
const void *dequant_kernel_sym(int bits);
// Group quantizer kernel for 2-, 3-, 4-, 5-, 6- or 8-bit codes from fp32 or bf16 weights (NULL otherwise).
const void *quantize_kernel_for(int bits, bool bf16_in);
// Matrix-core kernel with bands of 16*tiles rows (tiles 1 or 2). Dense
// products choose the activation load form by their rows per pass: one
// rotated load per segment up to 4 rows, staged through LDS up to 8, four
// loads for passes of 9-16 rows (launched with one grid row per pass of 16).
// The gather chooses its form per pass.
const void *mfma_kernel(int tiles, bool gather, int rows);
// Fused batch-1 projection kernel for (bits, chunks per lane, rows per
// iteration, ring stages, K segments of the block's LDS copy of x (0: none),
// epilogue: 0 residual, 1 SwiGLU, 2 GeGLU, 3 none; RMS norm prologue), or NULL.
const void *fused_kernel(int bits, int cpt, int R, int NB, int xs, int epi, bool norm);
// NVFP4 product kernel for (activation rows 1-4, chunks per lane, rows per iteration, ring stages), or NULL.
const void *nvfp4_kernel_for(int mw, int cpt, int R, int NB);

// Bit-stream widths (2, 3, 5 and 6 bits, group size 64; qmv_stream.hip).
struct StreamArgs {
    const uint16_t *x;  // activation rows, bf16 [M, K]
    const uint32_t *w;  // codes [N, K*bits/32], the row's low-first bit stream
    const uint16_t *s;  // bf16 scales [N, K/64]
    const uint16_t *b;  // bf16 biases [N, K/64]
    uint16_t *y;        // bf16 outputs [M, N]
    int64_t N;
    int32_t K;          // a multiple of 64
    int32_t M;          // activation rows, 1 .. 8
    // The expert gather (grid row y = expert plane; M holds the pair count P):
    // x [R_x, K], planes w [E, N, K*bits/32], s and b [E, N, K/64], y [P, N];
    // NULL index arrays are the identity.
    const uint32_t *lhs;
    const uint32_t *rhs;
    int32_t R_x;
    int32_t E;
    float ts;  // NVFP4: the tensor scale (s then holds E4M3 bytes [N, K/16])
    int32_t pad_;
};
constexpr int kStreamRowsPerBlock = 16;  // 4 waves of 4 weight rows
// The matvec kernel for `bits` and M activation rows (NULL outside 2, 3, 5, 6 and
// 1..8, and 4 bits at M = 1).
const void *stream_kernel(int bits, int M);
constexpr int kMaxGatherPairs = 4096;
// The K-split form (8 rows per block, two waves per row set alternating
// chunks of K) for `bits` (2, 3, 5, 6) and M <= 2; NULL otherwise.
const void *stream_split_kernel(int bits, int M);
// The NVFP4 batch-1 product on the bit-stream kernel (K a multiple of 64).
const void *stream_nvfp4_kernel();
// The expert gather kernel for `bits` taking up to `mw` pairs of a plane per
// pass (grid: row blocks x planes; NULL outside 2, 3, 5, 6 and 1..8).
const void *stream_gather_kernel(int bits, int mw);
// The codes widened to the 8-bit layout, one thread per 32 codes (grid: units / 256
// blocks of 256 threads, units = rows * K / 32).
const void *stream_to_u8_kernel(int bits);
// Dequantize kernel of the bit-stream widths: one thread per 32 codes (`bits` words).
const void *stream_dequant_kernel(int bits);

}  // namespace agq
