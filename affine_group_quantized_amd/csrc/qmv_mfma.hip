// Small-batch affine group-quantized products on the gfx950 matrix cores:
// the dense kernel (several activation rows, or passes of 16) and the
// expert-gathered kernel. The operand layout, tiling and load forms are
// described in mfma_core.hpp.

#include "mfma_core.hpp"

namespace agq {
using namespace mfma;

// XQ: the activation load form, 4 for M <= 4, 2 (staged) for M = 5..8, and 1
// for passes of up to 16 rows. blockIdx.y = pass: activation rows
// [16*pass, 16*pass + 16) of M (one pass for M <= 16). The passes of a launch
// walk the same bands at about the same time, so a band's codes read from HBM
// once serve the later passes from L2.
template <int T, int XQ>
__global__ __launch_bounds__(512) void qmv_mfma_kernel(MfmaArgs a) {
    __shared__ float red[Red<T>::FLOATS];
    // line loads, and the staged activations
    __shared__ u32x4 wt[kMfmaMaxS * (T * 128 + (XQ == 2 ? 256 : 0))];
    const int m0 = (int)blockIdx.y * 16;
    const int mrows = a.M - m0 < 16 ? a.M - m0 : 16;
    const uint32_t xbytes = (uint32_t)mrows * (uint32_t)a.K * 2u;
    const Band bd{reinterpret_cast<const uint8_t *>(a.w), a.s, a.b, a.N, (uint32_t)(a.K / 2), a.G};
    // Lanes of rows >= mrows start at the descriptor's end and read zeros.
    const Lanes ln = lane_consts<XQ>(a, [&](uint32_t r) { return r * (uint32_t)a.K * 2u; });
    mfma_pass<T, XQ>(a, bd, ln, range_of(a.x + (int64_t)m0 * a.K, xbytes), mrows,
                     RowsOut(a.y + (int64_t)m0 * a.N, a.N), blockIdx.x, gridDim.x, red, wt);
}

// blockIdx.y = expert plane e. The pairs routed to e are listed in LDS and
// taken 16 per pass, so each used plane streams once per pass; blocks of
// planes without pairs exit before reading weights. Blocks of plane 0 also
// write NaN rows for pairs whose indices are out of range. Dynamic LDS: the
// pair list (P uint16, padded to 16 bytes) and their x rows (P uint32).
template <int T>
__global__ __launch_bounds__(512) void gather_mfma_kernel(MfmaArgs a) {
    __shared__ float red[Red<T>::FLOATS];
    // line loads and the staged activations; the planner gives the gather at
    // most kMfmaGatherMaxS waves per block
    __shared__ u32x4 wt[kMfmaGatherMaxS * (T * 128 + 256)];
    __shared__ int pcount;
    uint16_t *plist = reinterpret_cast<uint16_t *>(g_mfma_dyn);
    uint32_t *xlist = reinterpret_cast<uint32_t *>(g_mfma_dyn + ((uint32_t)a.M * 2u + 15u) / 16u);
    const int lane = threadIdx.x & 63;
    const int wig = wave_id();
    const uint32_t e = blockIdx.y;
    const int64_t rg = blockIdx.x, groups = gridDim.x;
    const uint32_t *lhs = a.lhs, *rhs = a.rhs;
    const uint32_t nx = (uint32_t)a.R_x, ne = (uint32_t)a.E;
    const int P = a.M;

    auto compact = [&](auto pred) {
        int count = 0;
        for (int base = 0; base < P; base += 64) {
            const int p = base + lane;
            const bool take = p < P && pred(p);
            const uint64_t mask = __ballot(take);
            if (take) plist[count + __popcll(mask & ((1ull << lane) - 1ull))] = (uint16_t)p;
            count += __popcll(mask);
        }
        return count;
    };

    if (e == 0) {
        if (wig == 0) {
            const int c = compact([&](int p) {
                const uint32_t xr = lhs ? lhs[p] : (uint32_t)p;
                const uint32_t ex = rhs ? rhs[p] : (uint32_t)p;
                return xr >= nx || ex >= ne;
            });
            if (lane == 0) pcount = c;
        }
        __syncthreads();
        const int nbad = pcount;
        for (int i = 0; i < nbad; ++i) {
            uint16_t *yr = a.y + (int64_t)plist[i] * a.N;
            for (int bi = 0; bi < a.BPG; ++bi) {
                const int64_t row0 = (rg + (int64_t)bi * groups) * (16 * T);
                for (int r = (int)threadIdx.x; r < 16 * T; r += (int)blockDim.x)
                    if (row0 + r < a.N) yr[row0 + r] = 0x7FC0u;
            }
        }
        __syncthreads();
    }
    if (wig == 0) {
        const int c = compact([&](int p) {
            const uint32_t xr = lhs ? lhs[p] : (uint32_t)p;
            const uint32_t ex = rhs ? rhs[p] : (uint32_t)p;
            return ex == e && xr < nx;
        });
        for (int i = lane; i < c; i += 64) {
            const int p = plist[i];
            xlist[i] = lhs ? lhs[p] : (uint32_t)p;
        }
        if (lane == 0) pcount = c;
    }
    __syncthreads();
    const int count = pcount;
    if (count == 0) return;
    const uint32_t xbytes = (uint32_t)a.R_x * (uint32_t)a.K * 2u;
    const __amdgpu_buffer_rsrc_t xr = range_of(a.x, xbytes);
    const int64_t plane = (int64_t)e * a.N;
    const Band bd{reinterpret_cast<const uint8_t *>(a.w) + plane * (a.K / 2), a.s + plane * a.G, a.b + plane * a.G,
                  a.N, (uint32_t)(a.K / 2), a.G};
    for (int base = 0; base < count; base += 16) {
        const int me = count - base < 16 ? count - base : 16;
        with_xq(me, [&](auto xq) {
            constexpr int XQ = decltype(xq)::value;
            const Lanes ln = lane_consts<XQ>(a, [&](uint32_t r) {
                return (int)r < me ? xlist[base + r] * (uint32_t)a.K * 2u : xbytes;
            });
            mfma_pass<T, XQ>(a, bd, ln, xr, me, PairsOut(a.y, a.N, plist + base), rg, groups, red, wt);
        });
    }
}

const void *mfma_kernel(int tiles, bool gather, int rows) {
    if (gather) return tiles == 1 ? reinterpret_cast<const void *>(&gather_mfma_kernel<1>)
                                   : reinterpret_cast<const void *>(&gather_mfma_kernel<2>);
    if (rows <= 4) return tiles == 1 ? reinterpret_cast<const void *>(&qmv_mfma_kernel<1, 4>)
                                     : reinterpret_cast<const void *>(&qmv_mfma_kernel<2, 4>);
    if (rows <= 8) return tiles == 1 ? reinterpret_cast<const void *>(&qmv_mfma_kernel<1, 2>)
                                     : reinterpret_cast<const void *>(&qmv_mfma_kernel<2, 2>);
    return tiles == 1 ? reinterpret_cast<const void *>(&qmv_mfma_kernel<1, 1>)
                      : reinterpret_cast<const void *>(&qmv_mfma_kernel<2, 1>);
}

}  // namespace agq
