// Fused batch-1 projection for gfx950: the decode layer's neighbouring stages
// that "MLX CUDA Cleanup Plan", Phase 5, moves onto the device, folded into the
// affine group-quantized matrix-vector product of one activation row:
//  - RMS norm prologue: x_n = bf16(x * rs * gamma) is applied to the raw
//    activation words as they are staged, rs = 1 / sqrt(sum(x^2) / K + eps)
//    from wave sums of squares added in a fixed order. No normalized copy of
//    x is written to memory.
//  - epilogue with a residual: y[n] = v[n] + residual[n]; the residual rows are
//    loaded with the weight rows and start the accumulators, so the row loop
//    never waits on a load issued after the ring's weight loads.
//  - epilogues 1 and 2 (SwiGLU, GeGLU with the tanh form of gelu): projections
//    that share x (gate and up) are concatenated with their rows interleaved,
//    y[j] = act(v[2j]) * v[2j + 1]; both rows of a pair are reduced in the same
//    iteration and meet in one lane.
// The product itself is the VALU core of the batch-1 matvec kernels. Where
// the plan shares one LDS copy of x among a block's waves (one or two K
// segments per row group), the norm is applied to the raw words of that copy
// as the block fills it (a block sum of squares at one more barrier);
// otherwise (rows split over three or more waves) each wave normalizes the
// slice it stages. The norm and each epilogue are separate instantiations, so
// a kernel does no work for a stage it does not have.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "plan.hpp"
#include "qmv_core.hpp"
#include "qmv_device.hpp"
#include "qmv_kernels.hpp"

namespace agq {

// The activation row, with the norm's weights, epsilon, 1/K and the LDS slots
// of the block's sum of squares.
template <bool NORM>
struct NormRows {
    static constexpr bool kNorm = NORM;
    const uint16_t *x;
    int64_t K;
    const uint16_t *gamma;
    float eps, inv_k;
    float *part;  // LDS, one float per wave of the block
    __device__ __forceinline__ const uint16_t *operator()(int) const { return x; }
    template <int XS>
    static constexpr int fill_threads() { return 256; }
};

// Epilogues: kEpiResidual adds residual[n]; kEpiSwiGLU / kEpiGeGLU gate
// interleaved row pairs; kEpiNone stores v[n].
constexpr int kEpiResidual = 0, kEpiSwiGLU = 1, kEpiGeGLU = 2, kEpiNone = 3;

// silu(g) = g / (1 + e^-g); gelu(g) = g/2 (1 + tanh(sqrt(2/pi) (g + 0.044715 g^3))).
template <int EPI>
__device__ __forceinline__ float glu_act(float g) {
    if constexpr (EPI == kEpiSwiGLU) {
        return g / (1.f + __expf(-g));
    } else {
        return 0.5f * g * (1.f + tanhf(0.7978845608028654f * (g + 0.044715f * g * g * g)));
    }
}

template <int EPI>
struct FusedOut {
    static constexpr bool kGlu = EPI == kEpiSwiGLU || EPI == kEpiGeGLU;
    static constexpr bool kInit = EPI == kEpiResidual;  // residual rows start the accumulators
    uint16_t *y;
    const uint16_t *init;  // residual rows
    __device__ __forceinline__ void put(int, int64_t n, float v) const { y[n] = f32_to_bf16(v); }
    __device__ __forceinline__ void glu(int64_t j, float g, float u) const { y[j] = f32_to_bf16(glu_act<EPI>(g) * u); }
};

template <int BITS, int CPT, int R, int NB, int XS, int EPI, bool NORM>
__global__ __launch_bounds__(512) void qmv_fused_kernel(FusedArgs f) {
    __shared__ float red[kRedFloats];
    __shared__ float part[kBlockWaves];
    const ProductArgs &a = f.p;
    const int wave = wave_id();
    const int64_t rg = (int64_t)blockIdx.x * a.GPB + wave / a.S;
    const int64_t groups = (int64_t)gridDim.x * a.GPB;
    const int iters = (int)(a.RPG / R);  // RPG is a multiple of NB*R
    const Plane pl{a.w, a.s, a.b, a.C, a.G};
    const NormRows<NORM> rows{a.x, a.K, f.gamma, f.eps, f.inv_k, part};
    const FusedOut<EPI> out{a.y, f.res};
    if constexpr (FusedOut<EPI>::kGlu && R == 1) {
        // One row per iteration: gate and up rows of a pair in consecutive
        // iterations (iters is even: a multiple of NB = 2).
        static_assert(NB % 2 == 0, "pairs of iterations");
        const PairWalk walk{rg, groups, a.N};
        // Waves without rows leave only when they meet no block barrier (S == 1,
        // x staged by each wave).
        if (a.S == 1 && XS == 0 && walk.at(0) >= walk.end) return;
        product_rows<BITS, CPT, 1, R, NB, XS>(a, pl, rows, out, walk, iters, red);
    } else {
        const RowWalk walk = row_walk<R>(a, rg, groups);
        if (a.S == 1 && XS == 0 && walk.first >= walk.end) return;
        product_rows<BITS, CPT, 1, R, NB, XS>(a, pl, rows, out, walk, iters, red);
    }
}

// Plain-row epilogues (residual, none) at the plain row count; gated ones at theirs.
template <int BITS, int CPT, int R, int NB, int XS, bool GLU>
static const void *fused_variant(int epi, bool norm) {
#define AGQ_FUSED(E, N) reinterpret_cast<const void *>(&qmv_fused_kernel<BITS, CPT, R, NB, XS, E, N>)
    if constexpr (GLU) {
        switch (epi) {
            case kEpiSwiGLU: return norm ? AGQ_FUSED(kEpiSwiGLU, true) : AGQ_FUSED(kEpiSwiGLU, false);
            case kEpiGeGLU: return norm ? AGQ_FUSED(kEpiGeGLU, true) : AGQ_FUSED(kEpiGeGLU, false);
        }
    } else {
        switch (epi) {
            case kEpiResidual: return norm ? AGQ_FUSED(kEpiResidual, true) : AGQ_FUSED(kEpiResidual, false);
            case kEpiNone: return norm ? AGQ_FUSED(kEpiNone, true) : nullptr;  // (no stage: the plain product)
        }
    }
#undef AGQ_FUSED
    return nullptr;
}

template <int BITS, int CPT, int R, bool GLU>
static const void *fused_xs(int xs, int epi, bool norm) {
    constexpr int NB = plan_stages(1, false);
    switch (xs) {
        case 1: return fused_variant<BITS, CPT, R, NB, 1, GLU>(epi, norm);
        case 2: return fused_variant<BITS, CPT, R, NB, 2, GLU>(epi, norm);
        case 0:
            if constexpr (CPT >= 3) return fused_variant<BITS, CPT, R, NB, 0, GLU>(epi, norm);
            break;
    }
    return nullptr;
}

// The reachable plans of a chunk count: the shallow and the deep rows per
// iteration, each with the block's LDS copy over one or two K segments, and
// for rows split over three or more waves (3 or 4 chunks per lane) without it.
template <int BITS, int CPT>
static const void *fused_sym(int R, int NB, int xs, int epi, bool norm) {
    static_assert(plan_stages(1, false) == plan_stages(1, true), "one ring depth for the batch-1 plans");
    if (NB != plan_stages(1, false)) return nullptr;
    constexpr int RS = plan_rows(CPT, 1, false), RD = plan_rows(CPT, 1, true);
    if (epi == kEpiSwiGLU || epi == kEpiGeGLU) {
        if (R == RS) return fused_xs<BITS, CPT, RS, true>(xs, epi, norm);
        if constexpr (RD != RS) {
            if (R == RD) return fused_xs<BITS, CPT, RD, true>(xs, epi, norm);
        }
    } else {
        if (R == RS) return fused_xs<BITS, CPT, RS, false>(xs, epi, norm);
        if constexpr (RD != RS) {
            if (R == RD) return fused_xs<BITS, CPT, RD, false>(xs, epi, norm);
        }
    }
    return nullptr;
}

template <int BITS>
static const void *fused_by_cpt(int cpt, int R, int NB, int xs, int epi, bool norm) {
    static_assert(kFusedMaxCpt == 4, "instantiations below cover chunks per lane 1..4");
    switch (cpt) {
        case 1: return fused_sym<BITS, 1>(R, NB, xs, epi, norm);
        case 2: return fused_sym<BITS, 2>(R, NB, xs, epi, norm);
        case 3: return fused_sym<BITS, 3>(R, NB, xs, epi, norm);
        case 4: return fused_sym<BITS, 4>(R, NB, xs, epi, norm);
    }
    return nullptr;
}

const void *fused_kernel(int bits, int cpt, int R, int NB, int xs, int epi, bool norm) {
    return bits == 4   ? fused_by_cpt<4>(cpt, R, NB, xs, epi, norm)
           : bits == 8 ? fused_by_cpt<8>(cpt, R, NB, xs, epi, norm)
                       : nullptr;
}

}  // namespace agq
