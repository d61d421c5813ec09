// Launch planning for the matrix-core kernels (qmv_mfma.hip). Pure host code
// with no HIP calls, shared by the launcher and by agq_plan_product().
#pragma once

#include <stdint.h>

#include "agq.h"
#include "plan.hpp"

namespace agq {

// Activation rows from which dense 4-bit products use the matrix cores.
// Below it the VALU form is as fast or faster: 14336x4096 at M = 2 / 3 / 4 /
// 5 / 8 takes 9.6 / 11.0 / 12.2 / 14.9 / 19.2 us on the VALU and 11.4 /
// 11.6-11.8 / 11.9 / 12.6-13.0 / 13.3 us on the matrix cores (at M <= 4 with
// the compact activation load); 4096x14336 at M = 2 / 3 / 4, 10.4 / 12.4 /
// 13.0 against 12.1-12.3 / 12.35 / 12.7 us.
constexpr int kMfmaMinRows = 4;
constexpr int kMfmaRing = 4;   // 128-column segments in flight per wave (scales load in blocks of 4)
constexpr int kMfmaMaxS = 4;   // most waves splitting K (8: 10-35% slower; smaller blocks pack two or more per CU)
// The gather's planes give parallelism enough: at most 2 waves per block
// (W1 / W2: 69.9 / 63.8 -> 67.7 / 61.7 us).
constexpr int kMfmaGatherMaxS = 2;

struct MfmaPlan {
    int pass_rows = 16;   // gather: pairs per pass
    int lds_bytes = 0;    // dynamic LDS per block: the gather's pair lists
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
    if (bits != 4 || K % (128 * kMfmaRing) != 0) return false;
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
    const int64_t planes = experts > 0 ? experts : 1;
    p->T = ((N + 31) / 32) * S * planes >= 1024 ? 2 : 1;
    p->bands = (N + 16 * p->T - 1) / (16 * p->T);
}

// Dynamic LDS of the gather kernel: the pair list (uint16, padded to 16
// bytes) and the pairs' x rows (uint32).
inline void mfma_lds(int64_t experts, int64_t pairs, MfmaPlan *p) {
    p->lds_bytes = experts > 0 ? (int)((pairs * 2 + 15) / 16 * 16 + pairs * 4) : 0;
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
