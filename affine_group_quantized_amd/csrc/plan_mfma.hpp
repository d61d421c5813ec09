// Launch planning for the matrix-core kernels (qmv_mfma.hip). Pure host code
// with no HIP calls, shared by the launcher and by agq_plan_product().
#pragma once

#include <stdint.h>

#include "agq.h"
#include "plan.hpp"

namespace agq {

#ifndef AGQ_MFMA_MIN_ROWS
// Activation rows from which dense 4-bit products use the matrix cores (0:
// never). Below it the VALU form is as fast or faster: 14336x4096 at M = 2 /
// 3 / 4 / 5 / 8 takes 9.6 / 11.0 / 12.2 / 14.9 / 19.2 us on the VALU and
// 11.4 / 11.6-11.8 / 11.9 / 12.6-13.0 / 13.3 us on the matrix cores (at
// M <= 4 with the compact activation load); 4096x14336 at M = 2 / 3 / 4,
// 10.4 / 12.4 / 13.0 against 12.1-12.3 / 12.35 / 12.7 us.
#define AGQ_MFMA_MIN_ROWS 4
#endif
#ifndef AGQ_MFMA_TILES
#define AGQ_MFMA_TILES 0  // 16-row tiles per band: 1, 2, or 0 to choose from the shape
#endif
constexpr int kMfmaMinRows = AGQ_MFMA_MIN_ROWS;
#ifndef AGQ_MFMA_RING
#define AGQ_MFMA_RING 4  // 128-column segments in flight per wave: 4 or 8 (scales load in blocks of 4)
#endif
constexpr int kMfmaRing = AGQ_MFMA_RING;
#ifndef AGQ_MFMA_MAX_S
#define AGQ_MFMA_MAX_S 4  // smaller blocks pack two or more per compute unit (8: 10-35% slower)
#endif
#ifndef AGQ_MFMA_X_LDS_MAX
// Largest activation block copied to LDS (bytes); 0: never. Off: without the
// copy the kernels load codes in whole lines (line loads need LDS of their
// own), and that measured faster (14336x4096 at M = 8: 13.6 against 14.3 us).
#define AGQ_MFMA_X_LDS_MAX 0
#endif
constexpr int kMfmaXLdsMax = AGQ_MFMA_X_LDS_MAX;
constexpr int kMfmaXPer = 16;  // 16-byte words of x each thread copies
constexpr int kMfmaMaxS = AGQ_MFMA_MAX_S;  // most waves splitting K
#ifndef AGQ_MFMA_GATHER_MAX_S
#define AGQ_MFMA_GATHER_MAX_S 2  // the gather's planes give parallelism enough (W1 / W2: 69.9 / 63.8 -> 67.7 / 61.7 us)
#endif
constexpr int kMfmaGatherMaxS = AGQ_MFMA_GATHER_MAX_S < AGQ_MFMA_MAX_S ? AGQ_MFMA_GATHER_MAX_S : AGQ_MFMA_MAX_S;

struct MfmaPlan {
    int x_lds_bytes = 0;  // LDS copy of x; 0: waves load their operands from global memory
    int pass_rows = 16;   // gather: pairs per pass (the copy's rows when there is one)
    int lds_bytes = 0;    // dynamic LDS per block: the copy of x, and the gather's pair lists
    int T = 0;          // 16-row tiles per band
    int S = 0;          // waves per block, splitting K
    int SPW = 0;        // 128-column segments per wave
    int BPG = 0;        // bands per block
    int64_t bands = 0;  // bands per plane
    int64_t groups = 0; // blocks per plane
    int threads = 0;
    int64_t resident = 0;
};

// Whether a product runs on the matrix cores: 4-bit codes, K a multiple of
// 512 (whole blocks of 8 groups, 16-byte aligned scale rows), and several
// activation rows, or the gather (whose passes take up to 16 pairs). Byte
// offsets into x are 32-bit: the activation block must stay below 2 GiB.
inline bool mfma_eligible(int64_t M, int64_t K, int bits, int64_t experts, int64_t x_rows) {
    if (kMfmaMinRows <= 0 || bits != 4 || K % (128 * kMfmaRing) != 0) return false;
    if (x_rows * K * 2 + K * 2 >= (int64_t(1) << 31)) return false;
    return experts > 0 || M >= kMfmaMinRows;
}

// K split: the most waves (at most 4, or 2 for the gather) that divide the
// row's 4-segment blocks evenly; bands of two tiles unless that leaves fewer
// than one band-wave per SIMD of the device.
inline void mfma_shape(int64_t N, int64_t K, int64_t experts, MfmaPlan *p) {
    const int nseg = (int)(K / 128), blocks4 = nseg / kMfmaRing;  // whole rings per row
    int S = 1;
    for (int s = experts > 0 ? kMfmaGatherMaxS : kMfmaMaxS; s >= 1; --s)
        if (blocks4 % s == 0) {
            S = s;
            break;
        }
    p->S = S;
    p->SPW = nseg / S;
    p->threads = 64 * S;
    int T = AGQ_MFMA_TILES;
    if (T != 1 && T != 2) {
        const int64_t planes = experts > 0 ? experts : 1;
        T = ((N + 31) / 32) * S * planes >= 1024 ? 2 : 1;
    }
    p->T = T;
    p->bands = (N + 16 * T - 1) / (16 * T);
}

// LDS copy of the activation rows when the block's threads can stage it
// (kMfmaXPer words each) and it fits kMfmaXLdsMax. Dense: all M rows. Gather
// (off by default): passes of as many pairs as the copy holds, up to 16, when
// that is at least kMfmaGatherMinPass (fewer would stream planes with more
// pairs several times). On the Mixtral-shaped W1 the 64 KB copy halves the
// resident blocks: 94.3 us against 80.6 us with operands from L2.
#ifndef AGQ_MFMA_GATHER_X_LDS
#define AGQ_MFMA_GATHER_X_LDS 0
#endif
constexpr int kMfmaGatherMinPass = AGQ_MFMA_GATHER_X_LDS ? 8 : 17;
inline bool mfma_x_fits(int64_t rows, int64_t K, int threads) {
    const int64_t bytes = rows * K * 2;
    return bytes <= kMfmaXLdsMax && (bytes / 16 + threads - 1) / threads <= kMfmaXPer;
}
inline void mfma_x_lds(int64_t M, int64_t K, int64_t experts, int64_t pairs, MfmaPlan *p) {
    if (experts == 0) {
        p->x_lds_bytes = mfma_x_fits(M, K, p->threads) ? (int)(M * K * 2 + 16) : 0;
        p->lds_bytes = p->x_lds_bytes;
        return;
    }
    int rows = 16;
    while (rows > 0 && !mfma_x_fits(rows, K, p->threads)) --rows;
    p->pass_rows = rows >= kMfmaGatherMinPass ? rows : 16;
    p->x_lds_bytes = rows >= kMfmaGatherMinPass ? (int)(rows * K * 2 + 16) : 0;
    p->lds_bytes = p->x_lds_bytes + (int)((pairs * 2 + 15) / 16 * 16 + pairs * 4);
}

// Blocks per plane: every block resident at once (the gather oversubscribes,
// as its planes carry different numbers of pairs), each walking BPG bands.
inline void mfma_grid(int64_t resident_waves, int64_t experts, MfmaPlan *p) {
    p->resident = resident_waves;
    int64_t budget = resident_waves * (experts > 0 ? kGatherOversub : 1) / p->S / (experts > 0 ? experts : 1);
    if (budget < 1) budget = 1;
    const int64_t bpg = (p->bands + budget - 1) / budget;
    p->BPG = (int)bpg;
    p->groups = (p->bands + bpg - 1) / bpg;
}

}  // namespace agq
