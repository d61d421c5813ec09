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
// codes (half a group); an 8-bit chunk holds 16 codes (a quarter of a group).
//  - Waves split K into segments of 64*CPT chunks. Lane l of a wave owns
//    chunks seg + 64*j + l (j < CPT), so each load instruction of the wave
//    reads 1 KB of contiguous memory.
//  - A lane's columns are the same for every weight row. Its slice of the
//    activations is therefore loaded once and kept in VGPRs for the whole
//    kernel: as bfloat16 pairs (4-bit) or fp32 (8-bit).
//  - S waves, each owning one K segment, form a row group that walks a
//    contiguous range of RPG weight rows, R rows per iteration. All loads of
//    an iteration (R*CPT 16-byte chunks per lane) are issued before any use.
//  - Lane partial sums are reduced with DPP inside the wave. With S > 1 they
//    are then combined through LDS in a fixed order, so results are bitwise
//    deterministic.
//
// 4-bit inner loop. Each packed word gives four bfloat16 pairs (128 + q)
// through nibble_pair(). v_dot2c_f32_bf16 multiplies them by activation pairs
// staged in the same (i, i+4) column order. The accumulator starts at
// -128 * sum(x) of the chunk, which cancels the offset. That is 0.875 integer
// ops plus 0.5 dot ops per weight.
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

namespace agq {

constexpr int kRedSlots = kMaxWavesPerGroup * 64;  // per buffer: GPB*S*R*MW <= 8 waves * 64 values

template <int BITS>
struct Fmt {
    static constexpr int EPC = 128 / BITS;  // codes per 16-byte chunk
    static constexpr int CPG = 64 / EPC;    // chunks per 64-column group
};

// Stage one lane's activation slice for chunk `c` of activation row `xr`.
// 4-bit: 16 bfloat16 pairs in (i, i+4) order per packed word. 8-bit: 16 fp32.
template <int BITS>
__device__ __forceinline__ void stage_x(const uint16_t *__restrict__ xr, int c, bool valid, uint32_t (&xv)[16],
                                        float &xs) {
    if constexpr (BITS == 4) {
        u32x4 d[4] = {};
        if (valid) {
            const u32x4 *p = reinterpret_cast<const u32x4 *>(xr + (int64_t)c * 32);
#pragma unroll
            for (int t = 0; t < 4; ++t) d[t] = p[t];
        }
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            xv[4 * t + 0] = (d[t].x & 0xFFFFu) | (d[t].z << 16);
            xv[4 * t + 1] = (d[t].x >> 16) | (d[t].z & 0xFFFF0000u);
            xv[4 * t + 2] = (d[t].y & 0xFFFFu) | (d[t].w << 16);
            xv[4 * t + 3] = (d[t].y >> 16) | (d[t].w & 0xFFFF0000u);
        }
        float s = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) s = dot2_bf16(xv[i], 0x3F803F80u, s);
        xs = s;
    } else {
        u32x4 d[2] = {};
        if (valid) {
            const u32x4 *p = reinterpret_cast<const u32x4 *>(xr + (int64_t)c * 16);
            d[0] = p[0];
            d[1] = p[1];
        }
        float s = 0.f;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            uint32_t dw[4] = {d[t].x, d[t].y, d[t].z, d[t].w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float lo = bf16_lo(dw[i]), hi = bf16_hi(dw[i]);
                xv[8 * t + 2 * i] = __float_as_uint(lo);
                xv[8 * t + 2 * i + 1] = __float_as_uint(hi);
                s += lo;
                s += hi;
            }
        }
        xs = s;
    }
}

// Partial dot product of one chunk with one staged activation slice.
template <int BITS>
__device__ __forceinline__ float chunk_dot(const u32x4 &wv, const uint32_t (&xv)[16], float xs) {
    if constexpr (BITS == 4) {
        float d = -128.f * xs;
        const uint32_t w[4] = {wv.x, wv.y, wv.z, wv.w};
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            d = dot2_bf16(nibble_pair<0>(w[t]), xv[4 * t + 0], d);
            d = dot2_bf16(nibble_pair<1>(w[t]), xv[4 * t + 1], d);
            d = dot2_bf16(nibble_pair<2>(w[t]), xv[4 * t + 2], d);
            d = dot2_bf16(nibble_pair<3>(w[t]), xv[4 * t + 3], d);
        }
        return d;
    } else {
        float d = 0.f;
        const uint32_t w[4] = {wv.x, wv.y, wv.z, wv.w};
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            d = fmaf(__uint_as_float(xv[4 * t + 0]), (float)(w[t] & 0xFFu), d);
            d = fmaf(__uint_as_float(xv[4 * t + 1]), (float)((w[t] >> 8) & 0xFFu), d);
            d = fmaf(__uint_as_float(xv[4 * t + 2]), (float)((w[t] >> 16) & 0xFFu), d);
            d = fmaf(__uint_as_float(xv[4 * t + 3]), (float)(w[t] >> 24), d);
        }
        return d;
    }
}

// Shared core: MW activation rows (xrow[m]) against weight rows [row0, row1) of
// one plane; outputs to yrow[m][n]. `iters` must be equal for every row group of
// the block when S > 1 (block-wide barriers).
template <int BITS, int CPT, int MW, int R>
__device__ __forceinline__ void product_rows(const ProductArgs &a, const u32x4 *__restrict__ wp,
                                             const uint16_t *__restrict__ sp, const uint16_t *__restrict__ bp,
                                             const uint16_t *const *xrow, uint16_t *const *yrow,
                                             int64_t row0, int64_t row1, int iters, float *red) {
    using F = Fmt<BITS>;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int S = a.S;
    const int wig = wave % S;
    const int grp = wave / S;

    int chunk[CPT];
    bool cv[CPT];
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
        chunk[j] = (wig * CPT + j) * 64 + lane;
        cv[j] = chunk[j] < a.C;
    }

    uint32_t xv[MW][CPT][16];
    float xs[MW][CPT];
#pragma unroll
    for (int m = 0; m < MW; ++m)
#pragma unroll
        for (int j = 0; j < CPT; ++j) stage_x<BITS>(xrow[m], chunk[j], cv[j], xv[m][j], xs[m][j]);

    const int64_t C = a.C, G = a.G;
    for (int it = 0; it < iters; ++it) {
        const int64_t rb = row0 + (int64_t)it * R;
        u32x4 wv[R][CPT];
        uint32_t sv[R][CPT], bv[R][CPT];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const bool rv = rb + r < row1;
#pragma unroll
            for (int j = 0; j < CPT; ++j) {
                wv[r][j] = u32x4{0u, 0u, 0u, 0u};
                sv[r][j] = 0u;
                bv[r][j] = 0u;
                if (rv && cv[j]) {
                    const int64_t row = rb + r;
                    wv[r][j] = __builtin_nontemporal_load(wp + row * C + chunk[j]);
                    const int64_t gi = row * G + chunk[j] / F::CPG;
                    sv[r][j] = __builtin_nontemporal_load(sp + gi);
                    bv[r][j] = __builtin_nontemporal_load(bp + gi);
                }
            }
        }
        float acc[R][MW];
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int m = 0; m < MW; ++m) acc[r][m] = 0.f;
#pragma unroll
        for (int r = 0; r < R; ++r) {
#pragma unroll
            for (int j = 0; j < CPT; ++j) {
                const float sf = bf16_lo(sv[r][j]);
                const float bf = bf16_lo(bv[r][j]);
#pragma unroll
                for (int m = 0; m < MW; ++m) {
                    const float d = chunk_dot<BITS>(wv[r][j], xv[m][j], xs[m][j]);
                    acc[r][m] = fmaf(sf, d, acc[r][m]);
                    acc[r][m] = fmaf(bf, xs[m][j], acc[r][m]);
                }
            }
        }
        if (S == 1) {
#pragma unroll
            for (int r = 0; r < R; ++r)
#pragma unroll
                for (int m = 0; m < MW; ++m) {
                    const float t = wave_sum(acc[r][m]);
                    if (lane == 0 && rb + r < row1) yrow[m][rb + r] = f32_to_bf16(t);
                }
        } else {
            float *buf = red + (it & 1) * kRedSlots;
#pragma unroll
            for (int r = 0; r < R; ++r)
#pragma unroll
                for (int m = 0; m < MW; ++m) {
                    const float t = wave_sum(acc[r][m]);
                    if (lane == 0) buf[(grp * S + wig) * (R * MW) + r * MW + m] = t;
                }
            __syncthreads();
            if (wig == 0 && lane < R * MW) {
                const int r = lane / MW, m = lane % MW;
                float t = 0.f;
                for (int s = 0; s < S; ++s) t += buf[(grp * S + s) * (R * MW) + lane];
                if (rb + r < row1) {
#pragma unroll
                    for (int mm = 0; mm < MW; ++mm)
                        if (mm == m) yrow[mm][rb + r] = f32_to_bf16(t);
                }
            }
        }
    }
    if (S > 1) __syncthreads();  // the LDS buffers are reused by the caller's next pass
}

template <int BITS, int CPT, int MW, int R>
__global__ __launch_bounds__(512) void qmv_kernel(ProductArgs a) {
    __shared__ float red[2 * kRedSlots];
    const int wave = threadIdx.x >> 6;
    const int64_t rg = (int64_t)blockIdx.x * a.GPB + wave / a.S;
    const int64_t row0 = rg * a.RPG;
    int64_t row1 = row0 + a.RPG;
    if (row1 > a.N) row1 = a.N;
    if (a.S == 1 && row0 >= row1) return;  // no barriers on the S == 1 path
    const int iters = (int)((a.RPG + R - 1) / R);
    const uint16_t *xrow[MW];
    uint16_t *yrow[MW];
#pragma unroll
    for (int m = 0; m < MW; ++m) {
        xrow[m] = a.x + (int64_t)m * a.K;
        yrow[m] = a.y + (int64_t)m * a.N;
    }
    product_rows<BITS, CPT, MW, R>(a, a.w, a.s, a.b, xrow, yrow, row0, row1, iters, red);
}

template <int BITS, int ME, int R>
__device__ __forceinline__ void gather_pass(const ProductArgs &a, const u32x4 *wp, const uint16_t *sp,
                                            const uint16_t *bp, const uint16_t *plist, int base, int64_t row0,
                                            int64_t row1, int iters, float *red) {
    const uint16_t *xrow[ME];
    uint16_t *yrow[ME];
#pragma unroll
    for (int m = 0; m < ME; ++m) {
        const int p = plist[base + m];
        const int64_t xr = a.lhs ? (int64_t)a.lhs[p] : (int64_t)p;
        xrow[m] = a.x + xr * a.K;
        yrow[m] = a.y + (int64_t)p * a.N;
    }
    product_rows<BITS, 1, ME, R>(a, wp, sp, bp, xrow, yrow, row0, row1, iters, red);
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
// to 8 pairs. A block whose expert has no pairs exits before reading weights.
template <int BITS, int R>
__global__ __launch_bounds__(512) void gather_qmv_kernel(ProductArgs a) {
    __shared__ float red[2 * kRedSlots];
    __shared__ uint16_t plist[kMaxPairs];
    __shared__ int pcount;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const uint32_t e = blockIdx.y;
    const int64_t rg = (int64_t)blockIdx.x * a.GPB + wave / a.S;
    const int64_t row0 = rg * a.RPG;
    int64_t row1 = row0 + a.RPG;
    if (row1 > a.N) row1 = a.N;
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
        for (int i = 0; i < nbad; ++i) {
            uint16_t *yr = a.y + (int64_t)plist[i] * a.N;
            for (int64_t n = row0 + wig * 64 + lane; n < row1; n += 64 * a.S) yr[n] = 0x7FC0u;
        }
        __syncthreads();
    }
    if (wave == 0) {
        const int c = compact_pairs(a.M, plist, [&](int p) {
            const uint32_t xr = lhs ? lhs[p] : (uint32_t)p;
            const uint32_t ex = rhs ? rhs[p] : (uint32_t)p;
            return ex == e && xr < nx;
        });
        if (lane == 0) pcount = c;
    }
    __syncthreads();
    const int count = pcount;
    if (count == 0) return;
    if (a.S == 1 && row0 >= row1) return;
    const int iters = (int)((a.RPG + R - 1) / R);
    const u32x4 *wp = a.w + (int64_t)e * a.N * a.C;
    const uint16_t *sp = a.s + (int64_t)e * a.N * a.G;
    const uint16_t *bp = a.b + (int64_t)e * a.N * a.G;
    for (int base = 0; base < count; base += 8) {
        const int me = count - base < 8 ? count - base : 8;
        switch (me) {
            case 1: gather_pass<BITS, 1, R>(a, wp, sp, bp, plist, base, row0, row1, iters, red); break;
            case 2: gather_pass<BITS, 2, R>(a, wp, sp, bp, plist, base, row0, row1, iters, red); break;
            case 3: gather_pass<BITS, 3, R>(a, wp, sp, bp, plist, base, row0, row1, iters, red); break;
            case 4: gather_pass<BITS, 4, R>(a, wp, sp, bp, plist, base, row0, row1, iters, red); break;
            case 5: gather_pass<BITS, 5, R>(a, wp, sp, bp, plist, base, row0, row1, iters, red); break;
            case 6: gather_pass<BITS, 6, R>(a, wp, sp, bp, plist, base, row0, row1, iters, red); break;
            case 7: gather_pass<BITS, 7, R>(a, wp, sp, bp, plist, base, row0, row1, iters, red); break;
            default: gather_pass<BITS, 8, R>(a, wp, sp, bp, plist, base, row0, row1, iters, red); break;
        }
    }
}

// out[row, k] = fma(s, q, b): one rounding of the exact affine value.
template <int BITS>
__global__ __launch_bounds__(256) void dequant_kernel(const uint32_t *__restrict__ w, const uint16_t *__restrict__ s,
                                                      const uint16_t *__restrict__ b, float *__restrict__ out,
                                                      int64_t words, int64_t words_per_row, int64_t K) {
    constexpr int PER = 32 / BITS;
    constexpr uint32_t MASK = (1u << BITS) - 1u;
    const int64_t groups = K / 64;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < words;
         i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t row = i / words_per_row;
        const int64_t k0 = (i - row * words_per_row) * PER;
        const int64_t g = row * groups + k0 / 64;
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

template <int BITS, int MW, int CPT>
static const void *qmv_sym() {
    return reinterpret_cast<const void *>(&qmv_kernel<BITS, CPT, MW, rows_per_iter(CPT, MW)>);
}

template <int BITS, int MW>
static const void *qmv_by_cpt(int cpt) {
    if constexpr (kXRegBudget / MW >= 8) {
        switch (cpt) {
            case 1: return qmv_sym<BITS, MW, 1>();
            case 2: return qmv_sym<BITS, MW, 2>();
            case 3: return qmv_sym<BITS, MW, 3>();
            case 4: return qmv_sym<BITS, MW, 4>();
            case 5: return qmv_sym<BITS, MW, 5>();
            case 6: return qmv_sym<BITS, MW, 6>();
            case 7: return qmv_sym<BITS, MW, 7>();
            case 8: return qmv_sym<BITS, MW, 8>();
        }
    } else if constexpr (kXRegBudget / MW >= 4) {
        switch (cpt) {
            case 1: return qmv_sym<BITS, MW, 1>();
            case 2: return qmv_sym<BITS, MW, 2>();
            case 3: return qmv_sym<BITS, MW, 3>();
            case 4: return qmv_sym<BITS, MW, 4>();
        }
    } else if constexpr (kXRegBudget / MW >= 2) {
        switch (cpt) {
            case 1: return qmv_sym<BITS, MW, 1>();
            case 2: return qmv_sym<BITS, MW, 2>();
        }
    } else {
        if (cpt == 1) return qmv_sym<BITS, MW, 1>();
    }
    return nullptr;
}

template <int BITS>
static const void *qmv_by_mw(int mw, int cpt) {
    switch (mw) {
        case 1: return qmv_by_cpt<BITS, 1>(cpt);
        case 2: return qmv_by_cpt<BITS, 2>(cpt);
        case 3: return qmv_by_cpt<BITS, 3>(cpt);
        case 4: return qmv_by_cpt<BITS, 4>(cpt);
        case 5: return qmv_by_cpt<BITS, 5>(cpt);
        case 6: return qmv_by_cpt<BITS, 6>(cpt);
        case 7: return qmv_by_cpt<BITS, 7>(cpt);
        case 8: return qmv_by_cpt<BITS, 8>(cpt);
    }
    return nullptr;
}

const void *product_kernel(int bits, int mw, int cpt, bool gather) {
    if (gather) {
        if (cpt != 1) return nullptr;
        return bits == 4 ? reinterpret_cast<const void *>(&gather_qmv_kernel<4, rows_per_iter(1, 8)>)
                         : reinterpret_cast<const void *>(&gather_qmv_kernel<8, rows_per_iter(1, 8)>);
    }
    return bits == 4 ? qmv_by_mw<4>(mw, cpt) : qmv_by_mw<8>(mw, cpt);
}

const void *dequant_kernel_sym(int bits) {
    return bits == 4 ? reinterpret_cast<const void *>(&dequant_kernel<4>)
                     : reinterpret_cast<const void *>(&dequant_kernel<8>);
}

}  // namespace agq
