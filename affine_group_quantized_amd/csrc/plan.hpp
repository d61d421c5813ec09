// Launch planning for the product kernels. Pure host code with no HIP calls,
// shared by the launcher and by agq_plan_product().
#pragma once

#include <stdint.h>

#include "agq.h"

namespace agq {

constexpr int kMaxWavesPerGroup = 8;   // kernels are built with __launch_bounds__(512)
constexpr int kMaxCpt = 8;             // 16-byte chunks per lane in one wave's K segment
constexpr int kXRegBudget = 8;         // CPT * MW <= 8: staged activations use <= 128 VGPRs
constexpr int kMaxPairs = 4096;        // gather: pair list kept in LDS as uint16
constexpr int kWavesPerCuTarget = 8;

constexpr int floor_pow2(int v) { return v >= 8 ? 8 : v >= 4 ? 4 : v >= 2 ? 2 : 1; }

// Weight rows in flight per wave iteration. Aim for ~8 outstanding 16-byte
// loads per lane; keep R*MW accumulators at or below 32.
constexpr int rows_per_iter(int cpt, int mw) {
    return floor_pow2(8 / cpt) < floor_pow2(32 / mw) ? floor_pow2(8 / cpt) : floor_pow2(32 / mw);
}

struct Plan {
    int bits = 0, C = 0, cpt = 0, mw = 0, R = 0, S = 0, GPB = 0, threads = 0;
    int64_t RPG = 0, TG = 0, blocks = 0;
};

// Returns AGQ_OK and fills `p`, or AGQ_ENOTSUP when K is too large for the
// register-resident activation scheme at this M. Arguments are assumed valid
// otherwise (bits in {4,8}, K % 64 == 0, N >= 1, 1 <= M <= 8). `experts` is 0
// for the dense products and the number of expert planes for the gather, whose
// grid repeats the row tiling once per plane.
inline agq_status make_plan(int64_t M, int64_t N, int64_t K, int bits, int num_cus, int64_t experts, Plan *p) {
    const bool gather = experts > 0;
    Plan q;
    q.bits = bits;
    q.C = (int)(K * bits / 128);
    q.mw = gather ? 8 : (int)M;
    int cptmax = kXRegBudget / q.mw;
    if (cptmax > kMaxCpt) cptmax = kMaxCpt;
    int need = (q.C + 63) / 64;
    if (need <= cptmax) {
        q.cpt = need;
        q.S = 1;
    } else {
        q.S = (q.C + 64 * cptmax - 1) / (64 * cptmax);
        if (q.S > kMaxWavesPerGroup) return AGQ_ENOTSUP;
        q.cpt = (q.C + 64 * q.S - 1) / (64 * q.S);
    }
    q.R = rows_per_iter(q.cpt, q.mw);
    q.GPB = q.S == 1 ? 4 : (q.S == 2 ? 2 : 1);
    q.threads = 64 * q.S * q.GPB;
    int64_t waves = (int64_t)(num_cus > 0 ? num_cus : 256) * kWavesPerCuTarget;
    int64_t tg_target = waves / q.S / (gather ? experts : 1);
    if (tg_target < 1) tg_target = 1;
    int64_t rpg = (N + tg_target - 1) / tg_target;
    rpg = ((rpg + q.R - 1) / q.R) * q.R;
    if (rpg < q.R) rpg = q.R;
    q.RPG = rpg;
    q.TG = (N + rpg - 1) / rpg;
    q.blocks = (q.TG + q.GPB - 1) / q.GPB;
    *p = q;
    return AGQ_OK;
}

}  // namespace agq
