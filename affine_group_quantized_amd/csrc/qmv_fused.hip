// Fused batch-1 projection for gfx950: the decode layer's neighbouring stages
// that "MLX CUDA Cleanup Plan", Phase 5, moves onto the device, folded into the
// affine group-quantized matrix-vector product of one activation row:
//  - RMS norm prologue: x_n = bf16(x * rs * gamma) is applied to the raw
//    activation words as they are staged, rs = 1 / sqrt(sum(x^2) / K + eps)
//    from wave sums of squares added in a fixed order. No normalized copy of
//    x is written to memory.
//  - epilogue 0: y[n] = v[n] (+ residual[n]); the residual rows are loaded with
//    the weight rows and start the accumulators, so the row loop never waits on
//    a load issued after the ring's weight loads.
//  - epilogues 1 and 2 (SwiGLU, GeGLU with the tanh form of gelu): projections
//    that share x (gate and up) are concatenated with their rows interleaved,
//    y[j] = act(v[2j]) * v[2j + 1]; both rows of a pair are reduced in the same
//    iteration and meet in one lane.
// The product itself is the VALU core of the batch-1 matvec kernels. Where
// the plan shares one LDS copy of x among a block's waves, the norm is applied
// to the raw words of that copy as the block fills it (a block sum of squares
// at one more barrier); otherwise each wave normalizes the slice it stages.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "plan.hpp"
#include "qmv_core.hpp"
#include "qmv_device.hpp"
#include "qmv_kernels.hpp"

namespace agq {

// The activation row, with the norm's weights, epsilon and the LDS slots of
// the K-split sum of squares.
struct NormRows {
    static constexpr bool kNorm = true;
    const uint16_t *x;
    int64_t K;
    const uint16_t *gamma;  // NULL: no norm
    float eps;
    float *part;            // LDS, one float per wave of the block
    __device__ __forceinline__ const uint16_t *operator()(int) const { return x; }
    template <int XS>
    static constexpr int fill_threads() { return 256; }
};

// silu(g) = g / (1 + e^-g); gelu(g) = g/2 (1 + tanh(sqrt(2/pi) (g + 0.044715 g^3))).
template <int ACT>
__device__ __forceinline__ float glu_act(float g) {
    if constexpr (ACT == 1) {
        return g / (1.f + __expf(-g));
    } else {
        return 0.5f * g * (1.f + tanhf(0.7978845608028654f * (g + 0.044715f * g * g * g)));
    }
}

template <int ACT>
struct FusedOut {
    static constexpr bool kGlu = ACT != 0;
    static constexpr bool kInit = ACT == 0;  // residual rows start the accumulators
    uint16_t *y;
    const uint16_t *init;  // residual rows or NULL
    __device__ __forceinline__ void put(int, int64_t n, float v) const { y[n] = f32_to_bf16(v); }
    __device__ __forceinline__ void glu(int64_t j, float g, float u) const { y[j] = f32_to_bf16(glu_act<ACT>(g) * u); }
};

template <int BITS, int CPT, int R, int NB, int XS, int ACT>
__global__ __launch_bounds__(512) void qmv_fused_kernel(FusedArgs f) {
    __shared__ float red[kRedFloats];
    __shared__ float part[kBlockWaves];
    const ProductArgs &a = f.p;
    const int wave = wave_id();
    const int64_t rg = (int64_t)blockIdx.x * a.GPB + wave / a.S;
    const RowWalk walk = row_walk<R>(a, rg, (int64_t)gridDim.x * a.GPB);
    // Waves without rows leave only when they meet no block barrier (S == 1, x
    // staged by each wave).
    if (a.S == 1 && XS == 0 && walk.first >= walk.end) return;
    const int iters = (int)(a.RPG / R);  // RPG is a multiple of NB*R
    const Plane pl{a.w, a.s, a.b, a.C, a.G};
    product_rows<BITS, CPT, 1, R, NB, XS>(a, pl, NormRows{a.x, a.K, f.gamma, f.eps, part},
                                         FusedOut<ACT>{a.y, f.res}, walk, iters, red);
}

// The shallow plan (x staged by each wave, or through the block's LDS copy
// of one or two K segments) and the deep plan (x staged by each wave).
template <int BITS, int CPT, int ACT>
static const void *fused_sym(int R, int NB, int xs) {
    constexpr bool glu = ACT != 0;
    constexpr int RS = fused_rows(CPT, false, glu), RD = fused_rows(CPT, true, glu);
    constexpr int NS = plan_stages(1, false), ND = plan_stages(1, true);
    if (R == RS && NB == NS) {
        switch (xs) {
            case 0: return reinterpret_cast<const void *>(&qmv_fused_kernel<BITS, CPT, RS, NS, 0, ACT>);
            case 1: return reinterpret_cast<const void *>(&qmv_fused_kernel<BITS, CPT, RS, NS, 1, ACT>);
            case 2: return reinterpret_cast<const void *>(&qmv_fused_kernel<BITS, CPT, RS, NS, 2, ACT>);
        }
        return nullptr;
    }
    if constexpr (RD != RS || ND != NS) {
        if (R == RD && NB == ND && xs == 0)
            return reinterpret_cast<const void *>(&qmv_fused_kernel<BITS, CPT, RD, ND, 0, ACT>);
    }
    return nullptr;
}

template <int BITS, int ACT>
static const void *fused_by_cpt(int cpt, int R, int NB, int xs) {
    static_assert(kFusedMaxCpt == 4, "instantiations below cover chunks per lane 1..4");
    switch (cpt) {
        case 1: return fused_sym<BITS, 1, ACT>(R, NB, xs);
        case 2: return fused_sym<BITS, 2, ACT>(R, NB, xs);
        case 3: return fused_sym<BITS, 3, ACT>(R, NB, xs);
        case 4: return fused_sym<BITS, 4, ACT>(R, NB, xs);
    }
    return nullptr;
}

template <int BITS>
static const void *fused_by_act(int act, int cpt, int R, int NB, int xs) {
    switch (act) {
        case 0: return fused_by_cpt<BITS, 0>(cpt, R, NB, xs);
        case 1: return fused_by_cpt<BITS, 1>(cpt, R, NB, xs);
        case 2: return fused_by_cpt<BITS, 2>(cpt, R, NB, xs);
    }
    return nullptr;
}

const void *fused_kernel(int bits, int cpt, int R, int NB, int xs, int act) {
    return bits == 4 ? fused_by_act<4>(act, cpt, R, NB, xs) : bits == 8 ? fused_by_act<8>(act, cpt, R, NB, xs) : nullptr;
}

}  // namespace agq
