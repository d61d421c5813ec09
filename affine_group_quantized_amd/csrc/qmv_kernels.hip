// Affine group-quantized matrix-vector kernels for gfx950.
//
// Operands are the triple of "MLX CUDA Cleanup Plan", Target Architecture §1:
// BF16 activations, U32-packed 4/8-bit affine codes, and BF16 scale and bias
// per 64-column group (Refactor Plan, Phase 3). Output row n of activation
// row m is
//     y[m,n] = sum_g ( s[n,g] * sum_{k in g} x[m,k]*q[n,k] + b[n,g] * sum_{k in g} x[m,k] )
// which is sum_k x[m,k] * (s*q + b) regrouped per 64-column group. The
// per-group activation sums do not depend on n, so they are computed once.
//
// Work decomposition. A weight row is C 16-byte chunks. A 4-bit chunk holds 32
// codes, an 8-bit chunk 16: one scale group of 64 columns is 2 or 4 chunks
// (group sizes 32 and 128 halve or double that; a chunk never spans groups).
//  - Waves split K into segments of 64*CPT chunks. Lane l of a wave owns
//    chunks seg + 64*j + l (j < CPT), so each load instruction of the wave
//    reads 1 KB of contiguous memory.
//  - A lane's columns are the same for every weight row. Its slice of the
//    activations is therefore loaded once and kept in VGPRs for the whole
//    kernel: as bfloat16 pairs (4-bit) or fp32 (8-bit).
//  - S waves, each owning one K segment, form a row group that visits RPG
//    weight rows, R rows per iteration; row groups take R-row slices
//    round-robin. Each wave streams its rows through a ring of NB register
//    buffers, refilled NB iterations ahead.
//  - Where a block's row groups share columns, the block copies x into LDS
//    once, already in staging form, and the waves read their slices there.
//  - The R*MW lane partials of an iteration are reduced together: cross-half
//    swaps (v_permlane32_swap, v_permlane16_swap) fold pairs of them into one
//    register, then DPP finishes each 16-lane row, about 2.5 VALU ops per
//    value. With S > 1 the waves' sums are combined through LDS in a fixed
//    order, so results are bitwise deterministic.
//
// 4-bit inner loop. Each packed word gives four bfloat16 pairs (128 + q)
// with one AND, one shift-AND and four byte permutes. v_dot2c_f32_bf16
// multiplies them by activation pairs staged in the matching column order.
// The accumulator starts at -128 * sum(x) of the chunk, which cancels the
// offset. That is 0.875 integer ops plus 0.5 dot ops per weight.
//
// 8-bit inner loop: v_cvt_f32_ubyte{0..3} and fp32 FMA, two ops per weight.
//
// Weights, scales and biases are read with non-temporal loads, since each
// byte is used exactly once per call.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "plan.hpp"
#include "qmv_device.hpp"
#include "qmv_kernels.hpp"
#include "qmv_core.hpp"

namespace agq {

template <int BITS, int CPT, int MW, int R, int NB, int XS>
__global__ __launch_bounds__(512) void qmv_kernel(ProductArgs a) {
    __shared__ float red[kRedFloats];
    const int wave = wave_id();
    const int64_t rg = (int64_t)blockIdx.x * a.GPB + wave / a.S;
    const RowWalk walk = row_walk<R>(a, rg, (int64_t)gridDim.x * a.GPB);
    // A wave without rows may leave only when it meets no block barrier: with
    // S == 1 and x read from global memory. (Otherwise it walks rows past the
    // end, which read nothing and store nothing.)
    if (a.S == 1 && XS == 0 && walk.first >= walk.end) return;
    const int iters = (int)(a.RPG / R);  // RPG is a multiple of NB*R
    const Plane pl{a.w, a.s, a.b, a.C, a.G};
    product_rows<BITS, CPT, MW, R, NB, XS>(a, pl, DenseRows{a.x, a.K}, DenseOut{a.y, a.N}, walk, iters, red);
}

// Output rows of a gather pass: its m-th pair p = plist[m] writes y[p, :].
struct GatherOut {
    static constexpr bool kGlu = false;
    static constexpr bool kInit = false;
    uint16_t *y;
    int64_t N;
    const uint16_t *plist;
    __device__ __forceinline__ void put(int m, int64_t n, float v) const {
        y[(int64_t)plist[m] * N + n] = f32_to_bf16(v);
    }
};

// Rows per iteration of a gather pass with ME pairs: fewer rows in flight for the
// widest passes (register pressure). Any R partitions the same rows exactly once.
constexpr int gather_rows(int me, int r) { return me > 4 ? 1 : r; }

template <int BITS, int CPT, int ME, int R, int NB, int XS>
__device__ __forceinline__ void gather_pass(const ProductArgs &a, const Plane &pl, const uint16_t *plist,
                                            const uint32_t *xlist, int base, int64_t rg, int64_t groups, float *red) {
    constexpr int RR = gather_rows(ME, R);
    const RowWalk walk = row_walk<RR>(a, rg, groups);
    // RPG is a multiple of NB*R, so RPG / RR is a multiple of NB.
    product_rows<BITS, CPT, ME, RR, NB, XS>(a, pl, GatherRows{a.x, a.K, xlist + base},
                                            GatherOut{a.y, a.N, plist + base}, walk, (int)(a.RPG / RR), red);
    // The next pass refills the block's LDS copy of x. (With S > 1 the block
    // has already met at the end of product_rows.)
    if (XS > 0 && a.S == 1) __syncthreads();
}

// Compact (ascending) the pairs p < P that satisfy `pred` into list[]; wave 0 only.
template <typename Pred>
__device__ __forceinline__ int compact_pairs(int P, uint16_t *list, Pred pred) {
    const int lane = threadIdx.x & 63;
    int count = 0;
    for (int base = 0; base < P; base += 64) {
        const int p = base + lane;
        const bool take = p < P && pred(p);
        const uint64_t mask = __ballot(take);
        if (take) list[count + __popcll(mask & ((1ull << lane) - 1ull))] = (uint16_t)p;
        count += __popcll(mask);
    }
    return count;
}

// blockIdx.y = expert plane e; blockIdx.x = row tile. Pairs routed to e are
// grouped in LDS, so each used plane streams from memory once per pass of up
// to kGatherMW pairs. A block whose expert has no pairs exits before reading weights.
template <int BITS, int CPT, int R, int NB, int XS>
__global__ __launch_bounds__(512) void gather_qmv_kernel(ProductArgs a) {
    __shared__ float red[kRedFloats];
    __shared__ uint16_t plist[kMaxPairs];
    __shared__ uint32_t xlist[kMaxPairs];  // x row of each listed pair
    __shared__ int pcount;
    const int lane = threadIdx.x & 63;
    const int wave = wave_id();
    const uint32_t e = blockIdx.y;
    const int64_t rg = (int64_t)blockIdx.x * a.GPB + wave / a.S;
    const int64_t groups = (int64_t)gridDim.x * a.GPB;
    const RowWalk walk = row_walk<R>(a, rg, groups);
    const uint32_t *lhs = a.lhs, *rhs = a.rhs;
    const uint32_t nx = (uint32_t)a.R_x, ne = (uint32_t)a.E;

    if (e == 0) {
        // Pairs with an out-of-range index get NaN rows (written by the e == 0 blocks).
        if (wave == 0) {
            const int c = compact_pairs(a.M, plist, [&](int p) {
                const uint32_t xr = lhs ? lhs[p] : (uint32_t)p;
                const uint32_t ex = rhs ? rhs[p] : (uint32_t)p;
                return xr >= nx || ex >= ne;
            });
            if (lane == 0) pcount = c;
        }
        __syncthreads();
        const int nbad = pcount;
        const int wig = wave % a.S;
        const int iters = (int)(a.RPG / R);
        for (int i = 0; i < nbad; ++i) {
            uint16_t *yr = a.y + (int64_t)plist[i] * a.N;
            for (int it = 0; it < iters; ++it)
                for (int r = wig * 64 + lane; r < R; r += 64 * a.S) {
                    const int64_t n = walk.at(it) + r;
                    if (n < walk.end) yr[n] = 0x7FC0u;
                }
        }
        __syncthreads();
    }
    if (wave == 0) {
        const int c = compact_pairs(a.M, plist, [&](int p) {
            const uint32_t xr = lhs ? lhs[p] : (uint32_t)p;
            const uint32_t ex = rhs ? rhs[p] : (uint32_t)p;
            return ex == e && xr < nx;
        });
        // (LDS accesses of one wave complete in order: plist is written above.)
        for (int i = lane; i < c; i += 64) {
            const int p = plist[i];
            xlist[i] = lhs ? lhs[p] : (uint32_t)p;
        }
        if (lane == 0) pcount = c;
    }
    __syncthreads();
    const int count = pcount;
    if (count == 0) return;
    // Waves without rows leave only where they meet no block barrier. Passes
    // walk R or one row per iteration (gather_rows); a group has no rows in
    // any pass when it has none one row at a time.
    const RowWalk walk1 = row_walk<1>(a, rg, groups);
    if (a.S == 1 && XS == 0 && walk1.first >= walk1.end) return;
    const Plane pl{a.w + (int64_t)e * a.N * a.C, a.s + (int64_t)e * a.N * a.G, a.b + (int64_t)e * a.N * a.G, a.C, a.G};
    for (int base = 0; base < count; base += kGatherMW) {
        const int me = count - base < kGatherMW ? count - base : kGatherMW;
        switch (me) {
            case 1: gather_pass<BITS, CPT, 1, R, NB, XS>(a, pl, plist, xlist, base, rg, groups, red); break;
            case 2: gather_pass<BITS, CPT, 2, R, NB, XS>(a, pl, plist, xlist, base, rg, groups, red); break;
            case 3: gather_pass<BITS, CPT, 3, R, NB, XS>(a, pl, plist, xlist, base, rg, groups, red); break;
            case 4: gather_pass<BITS, CPT, 4, R, NB, XS>(a, pl, plist, xlist, base, rg, groups, red); break;
            default:
                if constexpr (kGatherMW > 4) {
                    switch (me) {
                        case 5: gather_pass<BITS, CPT, 5, R, NB, XS>(a, pl, plist, xlist, base, rg, groups, red); break;
                        case 6: gather_pass<BITS, CPT, 6, R, NB, XS>(a, pl, plist, xlist, base, rg, groups, red); break;
                        case 7: gather_pass<BITS, CPT, 7, R, NB, XS>(a, pl, plist, xlist, base, rg, groups, red); break;
                        default: gather_pass<BITS, CPT, 8, R, NB, XS>(a, pl, plist, xlist, base, rg, groups, red); break;
                    }
                }
                break;
        }
    }
}

// out[row, k] = fma(s, q, b): one rounding of the exact affine value.
template <int BITS>
__global__ __launch_bounds__(256) void dequant_kernel(const uint32_t *__restrict__ w, const uint16_t *__restrict__ s,
                                                      const uint16_t *__restrict__ b, float *__restrict__ out,
                                                      int64_t words, int64_t words_per_row, int64_t K, int64_t gs) {
    constexpr int PER = 32 / BITS;
    constexpr uint32_t MASK = (1u << BITS) - 1u;
    const int64_t groups = K / gs;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < words;
         i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t row = i / words_per_row;
        const int64_t k0 = (i - row * words_per_row) * PER;
        const int64_t g = row * groups + k0 / gs;  // a word's codes share one group (gs >= 32 >= PER)
        const float sf = bf16_lo(s[g]);
        const float bf = bf16_lo(b[g]);
        const uint32_t word = w[i];
        float v[PER];
#pragma unroll
        for (int j = 0; j < PER; ++j) v[j] = fmaf(sf, (float)((word >> (BITS * j)) & MASK), bf);
        float4 *o = reinterpret_cast<float4 *>(out + row * K + k0);
#pragma unroll
        for (int j = 0; j < PER / 4; ++j) o[j] = make_float4(v[4 * j], v[4 * j + 1], v[4 * j + 2], v[4 * j + 3]);
    }
}

// ---------------------------------------------------------------------------
// Kernel selection.

template <int BITS, int MW, int CPT, int R, int NB>
static const void *qmv_sym_xl(int xs) {
    switch (xs) {
        case 0: return reinterpret_cast<const void *>(&qmv_kernel<BITS, CPT, MW, R, NB, 0>);
        case 1: return reinterpret_cast<const void *>(&qmv_kernel<BITS, CPT, MW, R, NB, 1>);
        case 2: return reinterpret_cast<const void *>(&qmv_kernel<BITS, CPT, MW, R, NB, 2>);
    }
    return nullptr;
}

// The shallow and the deep plan of each (MW, CPT), and for several activation
// rows the plan of waves that cover a whole row (which never split K, so no
// more than one LDS segment). The deep plan reads x per wave (no LDS copy).
template <int BITS, int MW, int CPT>
static const void *qmv_sym(int R, int NB, int xl) {
    constexpr int RS = plan_rows(CPT, MW, false), RD = plan_rows(CPT, MW, true);
    constexpr int NS = plan_stages(MW, false), ND = plan_stages(MW, true);
    constexpr int RW = plan_rows(CPT, MW, false, true), NW = plan_stages(MW, false, true, CPT);
    if (R == RS && NB == NS) return qmv_sym_xl<BITS, MW, CPT, RS, NS>(xl);
    if constexpr (RD != RS || ND != NS) {
        if (R == RD && NB == ND && xl == 0) return reinterpret_cast<const void *>(&qmv_kernel<BITS, CPT, MW, RD, ND, 0>);
    }
    if constexpr (MW > 1 && (RW != RS || NW != NS)) {
        if (R == RW && NB == NW && xl <= 1)
            return xl ? reinterpret_cast<const void *>(&qmv_kernel<BITS, CPT, MW, RW, NW, 1>)
                      : reinterpret_cast<const void *>(&qmv_kernel<BITS, CPT, MW, RW, NW, 0>);
    }
    return nullptr;
}

template <int BITS, int MW>
static const void *qmv_by_cpt(int cpt, int R, int NB, int xl) {
    if constexpr (kXRegBudget / MW >= 8) {
        switch (cpt) {
            case 1: return qmv_sym<BITS, MW, 1>(R, NB, xl);
            case 2: return qmv_sym<BITS, MW, 2>(R, NB, xl);
            case 3: return qmv_sym<BITS, MW, 3>(R, NB, xl);
            case 4: return qmv_sym<BITS, MW, 4>(R, NB, xl);
            case 5:
                if constexpr (kMaxCpt >= 5) return qmv_sym<BITS, MW, 5>(R, NB, xl);
                break;
            case 6:
                if constexpr (kMaxCpt >= 6) return qmv_sym<BITS, MW, 6>(R, NB, xl);
                break;
            case 7:
                if constexpr (kMaxCpt >= 7) return qmv_sym<BITS, MW, 7>(R, NB, xl);
                break;
            case 8:
                if constexpr (kMaxCpt >= 8) return qmv_sym<BITS, MW, 8>(R, NB, xl);
                break;
        }
    } else if constexpr (kXRegBudget / MW >= 4) {
        switch (cpt) {
            case 1: return qmv_sym<BITS, MW, 1>(R, NB, xl);
            case 2: return qmv_sym<BITS, MW, 2>(R, NB, xl);
            case 3: return qmv_sym<BITS, MW, 3>(R, NB, xl);
            case 4: return qmv_sym<BITS, MW, 4>(R, NB, xl);
        }
    } else if constexpr (kXRegBudget / MW >= 2) {
        switch (cpt) {
            case 1: return qmv_sym<BITS, MW, 1>(R, NB, xl);
            case 2: return qmv_sym<BITS, MW, 2>(R, NB, xl);
        }
    } else {
        if (cpt == 1) return qmv_sym<BITS, MW, 1>(R, NB, xl);
    }
    return nullptr;
}

template <int BITS>
static const void *qmv_by_mw(int mw, int cpt, int R, int NB, int xl) {
    switch (mw) {
        case 1: return qmv_by_cpt<BITS, 1>(cpt, R, NB, xl);
        case 2: return qmv_by_cpt<BITS, 2>(cpt, R, NB, xl);
        case 3: return qmv_by_cpt<BITS, 3>(cpt, R, NB, xl);
        case 4: return qmv_by_cpt<BITS, 4>(cpt, R, NB, xl);
        case 5: return qmv_by_cpt<BITS, 5>(cpt, R, NB, xl);
        case 6: return qmv_by_cpt<BITS, 6>(cpt, R, NB, xl);
        case 7: return qmv_by_cpt<BITS, 7>(cpt, R, NB, xl);
        case 8: return qmv_by_cpt<BITS, 8>(cpt, R, NB, xl);
    }
    return nullptr;
}

template <int BITS, int CPT>
static const void *gather_sym_cpt(int R, int NB, int xs) {
    constexpr int RG = plan_rows(CPT, kGatherMW, false), NG = plan_stages(kGatherMW, false);  // one plan for every walk
    if (R != RG || NB != NG) return nullptr;
    switch (xs) {
        case 0: return reinterpret_cast<const void *>(&gather_qmv_kernel<BITS, CPT, RG, NG, 0>);
        case 1: return reinterpret_cast<const void *>(&gather_qmv_kernel<BITS, CPT, RG, NG, 1>);
        case 2: return reinterpret_cast<const void *>(&gather_qmv_kernel<BITS, CPT, RG, NG, 2>);
    }
    return nullptr;
}

template <int BITS>
static const void *gather_sym(int cpt, int R, int NB, int xs) {
    switch (cpt) {
        case 1: return gather_sym_cpt<BITS, 1>(R, NB, xs);
        case 2:
            if constexpr (kGatherXReg / kGatherMW >= 2) return gather_sym_cpt<BITS, 2>(R, NB, xs);
            break;
    }
    return nullptr;
}

const void *product_kernel(int bits, int mw, int cpt, int R, int NB, int x_lds, bool gather) {
    if (gather) {
        if (mw != kGatherMW) return nullptr;
        return bits == 4 ? gather_sym<4>(cpt, R, NB, x_lds) : gather_sym<8>(cpt, R, NB, x_lds);
    }
    return bits == 4 ? qmv_by_mw<4>(mw, cpt, R, NB, x_lds) : qmv_by_mw<8>(mw, cpt, R, NB, x_lds);
}

const void *dequant_kernel_sym(int bits) {
    return bits == 4 ? reinterpret_cast<const void *>(&dequant_kernel<4>)
                     : reinterpret_cast<const void *>(&dequant_kernel<8>);
}

}  // namespace agq
