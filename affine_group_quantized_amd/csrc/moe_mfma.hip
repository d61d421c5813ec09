// Fused decode MoE layer on the gfx950 matrix cores: the fused decode-MoE
// kernel of "epic: CUDA (MLX backend) prefill and decode acceleration
// program" (Code-audit findings, +55% on qwen3-30b-a3b; Phase 2, #626). For T
// tokens with k experts each (pair p = t*k + j, expert e = experts[p], router
// weight r[p]):
//
//   moe_gate_up_kernel: h_p = silu(W_gate[e] x_t) * (W_up[e] x_t)
//   moe_down_kernel:    o_p = r[p] * (W_down[e] h_p)          (fp32, per pair)
//   moe_combine_kernel: y_t = sum_j o_{t*k + j}                (slot order)
//
// The first two are the expert gather: blocks of (band group, expert plane),
// each used plane streamed once for all of its pairs. In the first, each
// band's two tiles are 16 rows of the gate plane and the same 16 rows of the
// up plane, so both values of a unit meet in one lane and the SwiGLU epilogue
// runs there. h is kept at about fp32 precision without an fp32 operand path:
// it is written as two bfloat16 rows per pair, hi = bf16(h) and lo =
// bf16(h - hi), and the down projection multiplies both (one more activation
// row each), so rounding h for the matrix cores costs about 2^-17 of it
// instead of 2^-9. The down projection's epilogue adds the two rows and
// applies the router weight; the combine sums each token's k slots in slot
// order, so results are bitwise deterministic without atomics. (One kernel
// per output band walking every expert in turn, combining in LDS, took 98 us
// for the Mixtral-shaped down projection against 64 us for the gather: its
// 256 blocks restart their load pipeline at every expert.)
// A token with an expert id out of range gets a NaN output row.

#include <mutex>

#include "mfma_core.hpp"
#include "moe.hpp"

namespace agq {
using namespace mfma;

// Scratch of agq_moe_decode_noalloc, for callers that cannot allocate: one
// array per device, alive until the process ends. Every call on a device
// shares it and it keeps the last call's contents (nothing in it has to start
// at zero: the first launch writes every h row the second reads). Calls that
// overlap in time on one device race on it.
static __device__ __align__(256) uint8_t scratch[kMoeScratchBytes];

namespace {
constexpr int kScratchDevices = 64;
void *g_scratch_ptr[kScratchDevices] = {};
std::mutex g_scratch_mu;
}  // namespace

hipError_t moe_scratch(int dev, void **ptr) {
    if (dev < 0 || dev >= kScratchDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        // The host-side name of the array is a stand-in, not a device address:
        // ask the runtime where this device's copy lives.
        void *p = nullptr;
        hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return hipSuccess;
}

namespace {

// Dense-product argument view for the shared pass code (K split, segments per
// wave, bands per block, the K of the rows streamed).
__device__ __forceinline__ MfmaArgs pass_args(int K, int S, int SPW, int BPG) {
    MfmaArgs a{};
    a.K = K;
    a.G = K / 64;
    a.S = S;
    a.SPW = SPW;
    a.BPG = BPG;
    return a;
}

// SwiGLU epilogue of a dual band: tile 0 holds the gate and tile 1 the up
// projection of unit n = band*16 + nl for pass row m = 4*g + r.
struct SwigluOut {
    uint16_t *h;            // [2P, F] bf16: row 2p = hi, row 2p + 1 = lo
    int64_t F;
    const uint16_t *plist;  // the pass's pairs
    template <int T>
    __device__ __forceinline__ void put(const f32x4 (&acc)[T], int64_t band, int g, int nl, int mrows,
                                        int64_t N) const {
        static_assert(T == 2, "dual bands: gate and up");
        const int64_t n = band * 16 + nl;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int m = 4 * g + r;
            if (m < mrows && n < N) {
                const float gate = acc[0][r], up = acc[1][r];
                const float v = gate / (1.f + __expf(-gate)) * up;
                const uint16_t hi = f32_to_bf16(v);
                const uint16_t lo = f32_to_bf16(v - bf16_lo(hi));
                const int64_t p = plist[m];
                h[(2 * p) * F + n] = hi;
                h[(2 * p + 1) * F + n] = lo;
            }
        }
    }
};

// Router-weighted fp32 rows of a finished down-projection band. Pass rows
// come in (hi, lo) couples, so lane (g, nl) holds both rows of the pass's
// pairs 2g and 2g + 1 (r = 0, 1 and 2, 3).
struct WeightedOut {
    float *o;               // [P, H] fp32
    int64_t H;
    const uint16_t *plist;  // the pass's pairs
    const float *weights;   // router weight per pair
    template <int T>
    __device__ __forceinline__ void put(const f32x4 (&acc)[T], int64_t band, int g, int nl, int mrows,
                                        int64_t N) const {
#pragma unroll
        for (int t = 0; t < T; ++t) {
            const int64_t n = band * (16 * T) + 16 * t + nl;
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                const int pp = 2 * g + q;  // pass pair
                if (2 * pp < mrows && n < N) {
                    const int p = plist[pp];
                    o[(int64_t)p * H + n] = weights[p] * (acc[t][2 * q] + acc[t][2 * q + 1]);
                }
            }
        }
    }
};

// The pairs p < P routed to plane e, ascending, into list (wave 0 of the block).
__device__ __forceinline__ int pairs_of(const uint32_t *experts, int P, uint32_t e, uint16_t *list) {
    const int lane = threadIdx.x & 63;
    int count = 0;
    for (int base = 0; base < P; base += 64) {
        const int p = base + lane;
        const bool take = p < P && experts[p] == e;
        const uint64_t mask = __ballot(take);
        if (take) list[count + __popcll(mask & ((1ull << lane) - 1ull))] = (uint16_t)p;
        count += __popcll(mask);
    }
    return count;
}

}  // namespace

// blockIdx.y = expert e, blockIdx.x = band group. The pairs routed to e (in
// increasing p) are listed in LDS and taken 16 per pass; each pass streams the
// gate and up planes' bands once.
__global__ __launch_bounds__(512) void moe_gate_up_kernel(MoeArgs a) {
    __shared__ float red[Red<2>::FLOATS];
    __shared__ u32x4 wt[kMfmaGatherMaxS * (2 * 128 + 256)];
    __shared__ int pcount;
    extern __shared__ u32x4 moe_dyn[];
    uint16_t *plist = reinterpret_cast<uint16_t *>(moe_dyn);
    uint32_t *xlist = reinterpret_cast<uint32_t *>(moe_dyn + (a.P * 2 + 15) / 16);
    const int lane = threadIdx.x & 63;
    const int wig = wave_id();
    const uint32_t e = blockIdx.y;
    if (wig == 0) {
        const int count = pairs_of(a.experts, a.P, e, plist);
        for (int i = lane; i < count; i += 64) xlist[i] = (uint32_t)(plist[i] / a.k);
        if (lane == 0) pcount = count;
    }
    __syncthreads();
    const int count = pcount;
    if (count == 0) return;
    const int64_t plane = (int64_t)e * a.F;
    const uint32_t rowbytes = (uint32_t)(a.H / 2);
    Band bd{reinterpret_cast<const uint8_t *>(a.wg) + plane * rowbytes, a.sg + plane * (a.H / 64),
            a.bg + plane * (a.H / 64), a.F, rowbytes, (int32_t)(a.H / 64)};
    bd.w2 = reinterpret_cast<const uint8_t *>(a.wu) + plane * rowbytes;
    bd.s2 = a.su + plane * (a.H / 64);
    bd.b2 = a.bu + plane * (a.H / 64);
    const uint32_t xbytes = (uint32_t)a.T * (uint32_t)a.H * 2u;
    const __amdgpu_buffer_rsrc_t xr = range_of(a.x, xbytes);
    const MfmaArgs pa = pass_args((int)a.H, a.S1, a.SPW1, a.BPG1);
    for (int base = 0; base < count; base += 16) {
        const int me = count - base < 16 ? count - base : 16;
        with_xq(me, [&](auto xq) {
            constexpr int XQ = decltype(xq)::value;
            const Lanes ln = lane_consts<XQ>(pa, [&](uint32_t r) {
                return (int)r < me ? xlist[base + r] * (uint32_t)a.H * 2u : xbytes;
            });
            mfma_pass<2, XQ, SwigluOut, true>(pa, bd, ln, xr, me, SwigluOut{a.h, a.F, plist + base}, blockIdx.x,
                                              gridDim.x, red, wt);
        });
    }
}

// blockIdx.y = expert e, blockIdx.x = band group (bands of 16*T rows of H).
// The pairs routed to e are listed in LDS and taken 8 per pass, each as its
// (hi, lo) rows of h: 16 activation rows per pass.
template <int T>
__global__ __launch_bounds__(512) void moe_down_kernel(MoeArgs a) {
    __shared__ float red[Red<T>::FLOATS];
    __shared__ u32x4 wt[kMfmaGatherMaxS * (T * 128 + 256)];
    __shared__ int pcount;
    extern __shared__ u32x4 moe_dyn[];
    uint16_t *plist = reinterpret_cast<uint16_t *>(moe_dyn);
    const int lane = threadIdx.x & 63;
    const int wig = wave_id();
    const uint32_t e = blockIdx.y;
    if (wig == 0) {
        const int count = pairs_of(a.experts, a.P, e, plist);
        if (lane == 0) pcount = count;
    }
    __syncthreads();
    const int count = pcount;
    if (count == 0) return;
    const int64_t plane = (int64_t)e * a.H;
    const uint32_t rowbytes = (uint32_t)(a.F / 2);
    const Band bd{reinterpret_cast<const uint8_t *>(a.wd) + plane * rowbytes, a.sd + plane * (a.F / 64),
                  a.bd + plane * (a.F / 64), a.H, rowbytes, (int32_t)(a.F / 64)};
    const uint32_t xbytes = (uint32_t)(2 * a.P) * (uint32_t)a.F * 2u;  // h: two rows per pair
    const __amdgpu_buffer_rsrc_t xr = range_of(a.h, xbytes);
    const MfmaArgs pa = pass_args((int)a.F, a.S2, a.SPW2, a.BPG2);
    for (int base = 0; base < count; base += 8) {
        const int me = count - base < 8 ? count - base : 8;
        const int rows = 2 * me;
        with_xq(rows, [&](auto xq) {
            constexpr int XQ = decltype(xq)::value;
            const Lanes ln = lane_consts<XQ>(pa, [&](uint32_t r) {
                return (int)r < rows ? (2u * plist[base + (r >> 1)] + (r & 1u)) * (uint32_t)a.F * 2u : xbytes;
            });
            mfma_pass<T, XQ, WeightedOut>(pa, bd, ln, xr, rows, WeightedOut{a.o, a.H, plist + base, a.weights},
                                          blockIdx.x, gridDim.x, red, wt);
        });
    }
}

// y[t, n] = bf16(sum_j o[t*k + j, n]) in increasing j; NaN where one of the
// token's expert ids is out of range.
__global__ __launch_bounds__(256) void moe_combine_kernel(MoeArgs a) {
    const int64_t total = (int64_t)a.T * a.H;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t t = i / a.H, n = i - t * a.H;
        float v = 0.f;
        bool bad = false;
        for (int j = 0; j < a.k; ++j) {
            const int64_t p = t * a.k + j;
            bad |= a.experts[p] >= (uint32_t)a.E;
            v += a.o[p * a.H + n];
        }
        a.y[i] = bad ? (uint16_t)0x7FC0u : f32_to_bf16(v);
    }
}

const void *moe_kernel(int stage, int tiles) {
    if (stage == 0) return reinterpret_cast<const void *>(&moe_gate_up_kernel);
    if (stage == 2) return reinterpret_cast<const void *>(&moe_combine_kernel);
    return tiles == 1 ? reinterpret_cast<const void *>(&moe_down_kernel<1>)
                      : reinterpret_cast<const void *>(&moe_down_kernel<2>);
}

}  // namespace agq
