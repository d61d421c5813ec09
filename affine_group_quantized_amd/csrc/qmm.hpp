// Argument block and kernel lookup of the quantized GEMM kernels (qmm_mfma.hip).
#pragma once

#include <stdint.h>

#include "qmv_kernels.hpp"

namespace agq {

// Tile shapes: a block of 4 waves computes 32*TM activation rows by 32*TN
// weight rows; global loads run DEPTH 64-column groups ahead. Two shapes:
//  - 64 x 64 tiles, loads 4 groups ahead, each group's results folded a group
//    later (latency over occupancy);
//  - 128 x 64 tiles, loads 2 groups ahead (occupancy: 2 waves per SIMD).
// The large tile wherever it leaves at least kQmmLargeBlocksPerCu blocks per
// compute unit, and the activation rows (dense M, or pairs per expert plane)
// exceed the small tile's threshold. Measured (4-bit, us): 4096x4096 at M =
// 256 / 512 / 1024: small 43.0 / 56.4 / 112, large 59.8 / 66.8 / 76.8;
// 4096x14336 at M = 256 / 512 / 1024: small 153 / 204 / 419, large 218 / 218 /
// 266; 28672x4096 at M = 256 / 512: small 245 / 455, large 164 / 323; the
// Mixtral-shaped prefill gather (1024 pairs): small 588, large 426.
constexpr int kQmmSmallM = 128;
constexpr int kQmmSmallPairs = 64;
constexpr int kQmmLargeBlocksPerCu = 2;
// Split-weight tiles (256 x 128, qmm_hl_kernel) from this many rows, where
// their grid gives at least 3/4 of the compute units a block (a partial round
// costs a full one) (4-bit, us: 4096x4096 at M = 2048: 157 -> 107; 28672x4096
// at M = 256 / 512 / 2048: 166 / 326 / 1221 -> 110 / 218 / 796; 4096x14336 at
// M = 2048: 554 -> 341). Tiles of 128 rows lost at M = 256 (28672x4096: 166 ->
// 174) and on the Mixtral prefill gather.
constexpr int kQmmHlMinRows = 256;
// Dense products of more rows than this take the split-weight tiles (256-row
// tiles, partly empty) wherever their grid, alone or split along K, fills the
// device: against the matvec passes and the corrected tiles (4-bit, us):
// 4096x14336 at M = 64 / 128 / 255: 63.6 / 121 / 154 -> 52.9 / 59.9 / 70.9;
// 28672x4096 at M = 96 / 128: 130 / 155 -> 99.3 / 105; 4096x4096 at M = 64 /
// 96: 21.0 / 37.4 against 24.8 / 28.8 (so not from 64 rows).
constexpr int kQmmHlSplitMinRows = 64;
// Dense products of more rows than this, up to kQmmHlSplitMinRows, take
// 64-row split-weight tiles where their grid (alone or split along K) fills
// the device, instead of 3-4 matvec passes; up to kQmmHlSmallNarrowRows rows
// (three passes) only where K splits at least kQmmHlSmallMinSplits ways, i.e.
// few weight rows (4-bit, us, passes -> tiles: 4096x14336 at M = 48 / 64:
// 64.8 / 63.6 -> 41.0 / 42.0; 6144x4096: 30.5 / 30.4 -> 22.3 / 23.6;
// 14336x4096 (2 splits) at M = 48 / 64: 38.6 / 49.0 -> 42.3 / 43.7; 28672x4096
// (no split) 73.2 / 81.3 -> 75.2 / 75.2; at M = 24 / 32 the passes win).
constexpr int kQmmHlSmallMinRows = 32;
constexpr int kQmmHlSmallNarrowRows = 48;
constexpr int kQmmHlSmallMinSplits = 4;
constexpr int kQmmPassRows = 128;  // 4-bit products of up to this many rows run on the matvec kernel in passes of 16

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
    float ts;             // NVFP4: the tensor scale applied to each result (unused by the affine kernels)
    float *part;          // K split: fp32 partial products [splits, M, N] (NULL: results go to y)
    int32_t gps;          // K split: 64-column groups per split (blockIdx.z = split)
    int32_t pad_;
};

struct QmmKernel {
    const void *sym = nullptr;
    int bm = 0, bn = 0;  // tile rows of x and of W
    int lds = 0;         // dynamic LDS bytes of the tile buffers
    int threads = 256;   // block size
    int splits = 1;      // K splits (grid.z); above 1 the partials go to a workspace and qmm_reduce_kernel sums them
    int gps = 0;         // 64-column groups per split
    bool split_weight = false;  // the split-weight tiles (qmm_hl_kernel, gather_qmm_hl_kernel)
};

// K splits of the split-weight tiles: where a grid of them leaves compute
// units idle, blockIdx.z takes a run of at least kQmmSplitMinGroups groups and
// the splits' fp32 partials meet in a workspace.
constexpr int kQmmSplitMinGroups = 4;

// The kernel for `rows` activation rows (dense M, or the gather's pairs per
// expert plane) against N weight rows of K columns in `planes` planes on
// `cus` compute units; K splits only where split_ok (dense, with a workspace).
QmmKernel qmm_kernel_for(int bits, bool gather, int64_t rows, int64_t N, int64_t K, int64_t planes, int cus,
                         bool split_ok);
// The NVFP4 GEMM (E2M1 codes, E4M3 scales per 16 columns) for M > 4 activation rows.
QmmKernel qmm_nvfp4_kernel_for(int64_t M, int64_t N, int64_t K, int cus, bool split_ok);
// Workspace bytes of a kernel choice: splits * M * N fp32 partials (0 without a split).
inline int64_t qmm_split_bytes(const QmmKernel &k, int64_t M, int64_t N) {
    return k.splits > 1 ? (int64_t)k.splits * M * N * 4 : 0;
}
// y = bf16(ts * sum over splits of the partials), splits summed in order.
const void *qmm_reduce_kernel();
// Tile geometry shared by both shapes (the host checks use it before any HIP call).
constexpr int kQmmTileN = 64;
constexpr int kQmmTileMinM = 64;
constexpr int kQmmHlTileN = 128;  // weight rows of the large tiles (the widest tile)

}  // namespace agq
