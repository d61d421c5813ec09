// Fused decode MoE layer on the gfx950 matrix cores: the fused decode-MoE
// kernel of "epic: CUDA (MLX backend) prefill and decode acceleration
// program" (Code-audit findings, +55% on qwen3-30b-a3b; Phase 2, #626), here in
// two launches. For T tokens with k experts each (pair p = t*k + j, expert
// e = experts[p], router weight r[p]):
//
//   launch 1 (moe_gate_up_kernel): h_p = silu(W_gate[e] x_t) * (W_up[e] x_t)
//   launch 2 (moe_down_kernel):    y_t = sum_j r[p] * (W_down[e] h_p)
//
// Launch 1 is the expert gather with dual bands: each band's two tiles are 16
// rows of the gate plane and the same 16 rows of the up plane, so both values
// of a unit meet in one lane and the SwiGLU epilogue runs there. h is kept at
// about fp32 precision without an fp32 operand path: it is written as two
// bfloat16 rows per pair, hi = bf16(h) and lo = bf16(h - hi), and the down
// projection multiplies both (one more activation row each), so rounding h for
// the matrix cores costs about 2^-17 of it instead of 2^-9.
//
// Launch 2 gives each block one 16-row band of the output (H rows) and walks
// every expert that some pair uses, in increasing order, streaming that
// plane's band once for all of its pairs. The router-weighted sum over a
// token's k experts accumulates in LDS in that fixed order (no atomics), so
// results are bitwise deterministic; the block writes its band of y once.
// A pair whose expert id is out of range makes its token's output row NaN.

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

// Router-weighted accumulation of a finished down-projection band into the
// block's LDS rows. Pass rows come in (hi, lo) couples, so lane (g, nl)
// holds both rows of the pass's pairs 2g and 2g + 1 (r = 0, 1 and 2, 3).
struct CombineOut {
    float *ylds;            // [tokens, 16*T]
    const uint16_t *plist;  // the pass's pairs
    const float *weights;   // router weight per pair
    int k;
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
                    const float v = acc[t][2 * q] + acc[t][2 * q + 1];
                    float &dst = ylds[(p / k) * (16 * T) + 16 * t + nl];
                    dst = fmaf(weights[p], v, dst);
                }
            }
        }
    }
};

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
        int count = 0;
        for (int base = 0; base < a.P; base += 64) {
            const int p = base + lane;
            const bool take = p < a.P && a.experts[p] == e;
            const uint64_t mask = __ballot(take);
            if (take) plist[count + __popcll(mask & ((1ull << lane) - 1ull))] = (uint16_t)p;
            count += __popcll(mask);
        }
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

// blockIdx.x = output band (16*T rows of H). Every expert some pair uses, in
// increasing order, then the band's rows of y.
template <int T>
__global__ __launch_bounds__(512) void moe_down_kernel(MoeArgs a) {
    __shared__ float red[Red<T, kMoeMaxS>::FLOATS];
    __shared__ u32x4 wt[kMoeMaxS * (T * 128 + 256)];
    extern __shared__ u32x4 moe_dyn[];
    // Dynamic LDS: pair list sorted by expert (P uint16, padded), per-expert
    // counts and offsets (E + 1 ints each), a NaN flag per token, then the
    // token rows of the band (T_tokens x 16*T floats).
    uint16_t *plist = reinterpret_cast<uint16_t *>(moe_dyn);
    int *cnt = reinterpret_cast<int *>(moe_dyn + (a.P * 2 + 15) / 16);
    int *off = cnt + a.E + 1;
    int *bad = off + a.E + 1;
    float *ylds = reinterpret_cast<float *>(bad + ((a.T + 3) / 4) * 4);
    const int lane = threadIdx.x & 63;
    const int wig = wave_id();
    const int S = (int)(blockDim.x >> 6);
    const uint32_t ne = (uint32_t)a.E;

    for (int i = (int)threadIdx.x; i < a.T; i += (int)blockDim.x) bad[i] = 0;
    for (int i = (int)threadIdx.x; i < a.T * 16 * T; i += (int)blockDim.x) ylds[i] = 0.f;
    __syncthreads();
    // Counts per expert (wave w takes experts w, w + S, ...), out-of-range ids.
    for (int e = wig; e < a.E; e += S) {
        int c = 0;
        for (int base = 0; base < a.P; base += 64) {
            const int p = base + lane;
            c += __popcll(__ballot(p < a.P && a.experts[p] == (uint32_t)e));
        }
        if (lane == 0) cnt[e] = c;
    }
    for (int p = (int)threadIdx.x; p < a.P; p += (int)blockDim.x)
        if (a.experts[p] >= ne) bad[p / a.k] = 1;
    __syncthreads();
    if (threadIdx.x == 0) {
        int s = 0;
        for (int e = 0; e < a.E; ++e) {
            off[e] = s;
            s += cnt[e];
        }
        off[a.E] = s;
    }
    __syncthreads();
    // Each expert's pairs in increasing p.
    for (int e = wig; e < a.E; e += S) {
        int c = off[e];
        for (int base = 0; base < a.P; base += 64) {
            const int p = base + lane;
            const bool take = p < a.P && a.experts[p] == (uint32_t)e;
            const uint64_t mask = __ballot(take);
            if (take) plist[c + __popcll(mask & ((1ull << lane) - 1ull))] = (uint16_t)p;
            c += __popcll(mask);
        }
    }
    __syncthreads();

    const uint32_t rowbytes = (uint32_t)(a.F / 2);
    const uint32_t xbytes = (uint32_t)(2 * a.P) * (uint32_t)a.F * 2u;  // h: two rows per pair
    const __amdgpu_buffer_rsrc_t xr = range_of(a.h, xbytes);
    const MfmaArgs pa = pass_args((int)a.F, S, a.SPW2, 1);
    for (int e = 0; e < a.E; ++e) {
        const int count = off[e + 1] - off[e];
        if (count == 0) continue;  // uniform
        const int64_t plane = (int64_t)e * a.H;
        const Band bd{reinterpret_cast<const uint8_t *>(a.wd) + plane * rowbytes, a.sd + plane * (a.F / 64),
                      a.bd + plane * (a.F / 64), a.H, rowbytes, (int32_t)(a.F / 64)};
        const uint16_t *list = plist + off[e];
        for (int base = 0; base < count; base += 8) {
            const int me = count - base < 8 ? count - base : 8;
            const int rows = 2 * me;  // (hi, lo) rows of h per pair
            with_xq(rows, [&](auto xq) {
                constexpr int XQ = decltype(xq)::value;
                const Lanes ln = lane_consts<XQ>(pa, [&](uint32_t r) {
                    return (int)r < rows ? (2u * list[base + (r >> 1)] + (r & 1u)) * (uint32_t)a.F * 2u : xbytes;
                });
                mfma_pass<T, XQ, CombineOut, false, kMoeMaxS>(pa, bd, ln, xr, rows,
                                                              CombineOut{ylds, list + base, a.weights, a.k},
                                                              blockIdx.x, gridDim.x, red, wt);
            });
            __syncthreads();  // (S == 1 passes end without one) the next pass reuses the LDS buffers
        }
    }
    __syncthreads();
    const int64_t n0 = (int64_t)blockIdx.x * 16 * T;
    for (int i = (int)threadIdx.x; i < a.T * 16 * T; i += (int)blockDim.x) {
        const int t = i / (16 * T), c = i % (16 * T);
        if (n0 + c < a.H) a.y[(int64_t)t * a.H + n0 + c] = bad[t] ? (uint16_t)0x7FC0u : f32_to_bf16(ylds[i]);
    }
}

const void *moe_kernel(bool down) {
    return down ? reinterpret_cast<const void *>(&moe_down_kernel<1>)
                : reinterpret_cast<const void *>(&moe_gate_up_kernel);
}

}  // namespace agq
