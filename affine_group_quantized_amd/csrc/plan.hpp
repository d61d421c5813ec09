// Launch planning for the product kernels. Pure host code with no HIP calls,
// shared by the launcher and by agq_plan_product().
#pragma once

#include <stdint.h>

#include "agq.h"

namespace agq {

constexpr int kMaxWavesPerGroup = 8;   // kernels are built with __launch_bounds__(512)
// 16-byte chunks per lane within a wave's K segment: at most 7 (8 chunks per
// lane plus two row buffers no longer fit in 256 VGPRs). Longer rows split K
// over more waves rather than holding more chunks per lane, as long as 8 waves
// cover the row: 4 chunks keep 3 waves per SIMD resident (4096x14336 at batch
// 1: 8.6 us with 2 waves of 4 chunks against 9.5 us with one wave of 7).
constexpr int kMaxCpt = 7;
constexpr int kPrefCpt = 4;
constexpr int kXRegBudget = 8;         // CPT * MW <= 8: staged activations use <= 128 VGPRs
// Preferred budget for several activation rows: one chunk per lane at M >= 2,
// splitting K over more waves (each holding less x, so more of them stay
// resident), as long as 8 waves cover the row; kXRegBudget past that.
// 14336x4096 at M = 2 / 4: 9.2 / 12.3 us against 9.8 / 13.1 us with 2 chunks.
constexpr int kXRegWide = 2;
constexpr int kMaxPairs = 4096;        // gather: pair list kept in LDS as uint16
// 16-byte weight loads in flight per lane, counting every stage of the load
// ring, and the ring depth. Short walks use the shallow plan (more, lighter
// waves finish sooner); walks of at least kDeepRows rows per row group use the
// deep one.
constexpr int kLoadsShallow = 4;
constexpr int kLoadsDeep = 8;
constexpr int kStagesShallow = 2;
constexpr int kStagesDeep = 2;
constexpr int kDeepRows = 16;
// Several activation rows per pass (MW > 1: the wide and gather forms): x
// takes 16*MW*CPT VGPRs per lane, residency is low, and each wave needs more
// rows in flight. One plan for short and long walks.
constexpr int kLoadsWide = 4;
constexpr int kStagesWide = 2;
// Ring depth of the wide form when one wave covers a whole row (S == 1): such
// waves hold fewer activation registers than the K-split shapes of the same
// instantiation, and room for more rows in flight.
constexpr int kStagesWide1 = 4;
// Pairs per pass of the VALU gather. Planes with more pairs take several
// passes, each reading the plane again; fewer pairs per pass keep x in fewer
// VGPRs and more waves resident. On the Mixtral-shaped workload (2 to 8 pairs
// per plane) passes of 8 win: 86.5 + 96.2 us for W1 + W2 against 88.1 + 99.8
// us with passes of 4.
constexpr int kGatherMW = 8;
constexpr int kGatherXReg = 8;         // gather: CPT * MW <= this (16 VGPRs of staged activations per unit)
constexpr int kGatherOversub = 4;      // gather grid: resident groups x this

constexpr int floor_pow2(int v) { return v >= 16 ? 16 : v >= 8 ? 8 : v >= 4 ? 4 : v >= 2 ? 2 : 1; }

// Weight rows per wave iteration: aim for `loads` outstanding 16-byte loads
// per lane over the `stages` buffers of the load ring; keep R*MW accumulators
// at or below 16 (register pressure of the wide and gather forms).
constexpr int rows_per_iter(int cpt, int mw, int loads, int stages) {
    return floor_pow2(loads / stages / cpt) < floor_pow2(16 / mw) ? floor_pow2(loads / stages / cpt)
                                                                  : floor_pow2(16 / mw);
}
// Whether the deeper whole-row ring fits the register file: roughly 6 VGPRs
// per chunk and stage for codes, scales and biases, and 16 per chunk and
// activation row for x (4 chunks at 2 rows and 4 stages spill).
constexpr bool wide1_fits(int cpt, int mw) { return cpt * (6 * kStagesWide1 + 16 * mw) <= 200; }
constexpr int plan_stages(int mw, bool deep, bool whole_row = false, int cpt = 1) {
    return mw > 1 ? (whole_row && wide1_fits(cpt, mw) ? kStagesWide1 : kStagesWide) : deep ? kStagesDeep : kStagesShallow;
}
constexpr int plan_rows(int cpt, int mw, bool deep, bool whole_row = false) {
    return mw > 1  ? rows_per_iter(cpt, mw, kLoadsWide, plan_stages(mw, deep, whole_row, cpt))
           : deep ? rows_per_iter(cpt, mw, kLoadsDeep, kStagesDeep)
                  : rows_per_iter(cpt, mw, kLoadsShallow, kStagesShallow);
}

// Row groups per block: 4 single-wave groups, or 4 two-wave groups (one LDS
// copy of x for 8 waves); one group for S >= 3.
constexpr int kGpbS1 = 4;
constexpr int kGpbS2 = 4;
// Largest activation block staged in LDS (bytes; 20 and 40 KB caps measured
// slower: down 7.9 -> 8.9 us).
constexpr int kXLdsMax = 81920;
constexpr int kXLdsPerChunk = 68;

struct Plan {
    int bits = 0, C = 0, cpt = 0, mw = 0, R = 0, NB = 0, S = 0, GPB = 0, threads = 0;
    int x_lds_bytes = 0;  // dynamic LDS for x; 0 = waves stage x straight from global memory
    int64_t RPG = 0, TG = 0, blocks = 0;
    int64_t resident = 0;  // waves of this kernel the device holds at once (grid sizing input)
};

// Kernel shape: chunks per lane, K split, rows per iteration, block size.
// Returns AGQ_ENOTSUP when K is too large for the register-resident activation
// scheme at this M. Arguments are assumed valid otherwise (bits in {4,8},
// K % 64 == 0, N >= 1, 1 <= M <= 8). `experts` is 0 for the dense products and
// the number of expert planes for the gather.
inline agq_status plan_shape(int64_t M, int64_t K, int bits, int64_t experts, Plan *p, bool deep = false) {
    const bool gather = experts > 0;
    Plan q;
    q.bits = bits;
    q.C = (int)(K * bits / 128);
    q.mw = gather ? kGatherMW : (int)M;
    int cptmax = (gather ? kGatherXReg : kXRegBudget) / q.mw;
    if (cptmax < 1) cptmax = 1;
    if (cptmax > kMaxCpt) cptmax = kMaxCpt;
    // The preferred cap, unless only a larger one keeps S within a block.
    int pref = gather ? cptmax : q.mw > 1 ? kXRegWide / q.mw : kPrefCpt;
    if (pref < 1) pref = 1;
    if (cptmax > pref && (q.C + 64 * pref - 1) / (64 * pref) <= kMaxWavesPerGroup) cptmax = pref;
    int need = (q.C + 63) / 64;
    if (need <= cptmax) {
        q.cpt = need;
        q.S = 1;
    } else {
        q.S = (q.C + 64 * cptmax - 1) / (64 * cptmax);
        if (q.S > kMaxWavesPerGroup) return AGQ_ENOTSUP;
        q.cpt = (q.C + 64 * q.S - 1) / (64 * q.S);
    }
    const bool whole_row = !gather && q.S == 1;
    q.R = plan_rows(q.cpt, q.mw, deep, whole_row);
    q.NB = plan_stages(q.mw, deep, whole_row, q.cpt);
    q.GPB = q.S == 1 ? kGpbS1 : (q.S == 2 ? kGpbS2 : 1);
    q.threads = 64 * q.S * q.GPB;
    // One LDS copy of x, in staging form, can serve a whole block of
    // single-wave row groups, or of row groups of two K segments.
    // Without it every row group reads x from global memory, which for several
    // activation rows costs more L2 traffic than the weights themselves.
    // Long walks (the deep plan) amortize each wave's own staging of x over
    // many rows, and skip the block barrier the LDS copy needs.
    // LDS bytes of the copy: per activation row and covered chunk, sixteen
    // 32-bit staged values and the chunk's sum of x (4-bit and 8-bit alike).
    const int64_t xbytes = (int64_t)q.mw * 64 * q.cpt * q.S * kXLdsPerChunk;
    // (At least 256 threads per segment: the fill's per-thread share is sized
    // for 256*S threads.)
    const bool shared = (q.S == 1 || q.S == 2) && q.GPB >= 4;
    // (The gather's passes are short walks whatever the plane's length.)
    q.x_lds_bytes = ((gather || !deep) && shared && xbytes <= kXLdsMax) ? (int)xbytes : 0;
    *p = q;
    return AGQ_OK;
}

// Row tiling: one row group per resident wave set, so the whole grid is
// resident at once (no second, partly empty round of waves), except for the
// gather (below). `resident_waves`
// is the number of waves of this kernel the device holds at once (compute
// units times waves per unit at the kernel's occupancy). For the gather, the
// grid repeats per expert plane and the budget is shared among the planes.
inline void plan_grid(int64_t N, int64_t resident_waves, int64_t experts, Plan *q) {
    q->resident = resident_waves;
    // The gather's planes carry different numbers of pairs, so its grid is
    // oversubscribed: blocks of lightly loaded planes finish early and the
    // hardware hands their compute units the blocks still waiting.
    int64_t tg_target = resident_waves * (experts > 0 ? kGatherOversub : 1) / q->S / (experts > 0 ? experts : 1);
    if (tg_target < 1) tg_target = 1;
    // Iterations per group: a multiple of the load ring depth.
    const int64_t step = q->NB;
    int64_t iters = (N + tg_target * q->R - 1) / (tg_target * q->R);
    iters = ((iters + step - 1) / step) * step;
    // The fewest groups that cover N rows in `iters` iterations of R rows.
    q->TG = (N + iters * q->R - 1) / (iters * q->R);
    q->RPG = iters * q->R;
    q->blocks = (q->TG + q->GPB - 1) / q->GPB;
    q->TG = q->blocks * q->GPB;  // every launched group walks rows (groups past N store nothing)
}

// Whether a walk is long enough for the deep load depth.
inline bool wants_deep(int64_t N, int64_t resident_waves, int S, int64_t experts) {
    int64_t groups = resident_waves / S / (experts > 0 ? experts : 1);
    if (groups < 1) groups = 1;
    return N >= (int64_t)kDeepRows * groups;
}

// The fused batch-1 projection uses the one-row plan, except that the deep
// plan also shares the block's LDS copy of x where the shallow one would (the
// norm is applied while the block fills it, with far fewer registers than
// normalizing per wave). A gated epilogue pairs gate row 2j with up row 2j + 1:
// in one iteration when it reads two or more rows, else in consecutive
// iterations of a walk over row pairs (the ring holds both). Plans of more
// than 4 chunks per lane (rows longer than 8 waves of 4) are not instantiated.
constexpr int kFusedMaxCpt = 4;

inline agq_status plan_fused_shape(int64_t K, int bits, Plan *p, bool deep = false) {
    Plan q;
    agq_status st = plan_shape(1, K, bits, 0, &q, deep);
    if (st != AGQ_OK) return st;
    if (q.cpt > kFusedMaxCpt) return AGQ_ENOTSUP;
    if (deep) {
        Plan sh;
        plan_shape(1, K, bits, 0, &sh, false);
        q.x_lds_bytes = sh.x_lds_bytes;  // same S and chunks per lane as the deep plan
    }
    *p = q;
    return AGQ_OK;
}

inline agq_status make_plan(int64_t M, int64_t N, int64_t K, int bits, int64_t resident_waves, int64_t experts,
                            Plan *p) {
    Plan q;
    agq_status st = plan_shape(M, K, bits, experts, &q);
    if (st != AGQ_OK) return st;
    if (wants_deep(N, resident_waves, q.S, experts)) plan_shape(M, K, bits, experts, &q, true);
    plan_grid(N, resident_waves, experts, &q);
    *p = q;
    return AGQ_OK;
}

}  // namespace agq
