// Shared core of the VALU product kernels (dense, wide, gather and the fused
// batch-1 projection): activation staging, weight-row loads, per-lane dot
// products, wave reductions and the row walk. The algorithm is described at
// the top of qmv_kernels.hip.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "plan.hpp"
#include "qmv_device.hpp"
#include "qmv_kernels.hpp"

namespace agq {

// Dynamic LDS of the product kernels: the block's copy of x (XFill).
extern __shared__ u32x4 g_xlds[];

// Third descriptor word of a raw buffer (gfx9 family: 32-bit data format,
// no swizzle, stride 0) and the non-temporal cache policy of its loads.
constexpr int kRsrcWord3 = 0x00020000;
constexpr int kLoadNT = 2;

// Descriptor over `bytes` bytes at `base`. Loads at offsets >= bytes return
// zero without touching memory, so a descriptor of 0 bytes turns every load
// through it into a zero fill.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t byte_range(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, (int)bytes, kRsrcWord3);
}

// Activation staging. A lane's slice of one activation row for one chunk is
// sixteen 32-bit registers:
//  - 4-bit codes: 32 bf16 values as 16 bfloat16 pairs, in the order of the
//    code pairs a packed word unpacks to: for each 16-byte word of x
//    (x0..x7), the pairs (x0,x4), (x1,x5), (x2,x6), (x3,x7);
//  - 8-bit codes: 16 values widened to fp32;
// plus the chunk's sum of x: in one running sum when a wave stages from
// global memory, per 16-byte word and then pairwise in the block's LDS copy.
// (The two orders can differ only in the last bit of that sum.)

// Stage form of one 16-byte word of x (8 bf16) for 4-bit codes: four pairs.
__device__ __forceinline__ void pairs_of_word(const u32x4 &q, uint32_t (&o)[4]) {
    o[0] = byte_perm(q.z, q.x, 0x05040100u);  // (x0, x4)
    o[1] = byte_perm(q.z, q.x, 0x07060302u);  // (x1, x5)
    o[2] = byte_perm(q.w, q.y, 0x05040100u);  // (x2, x6)
    o[3] = byte_perm(q.w, q.y, 0x07060302u);  // (x3, x7)
}

// Sum of the 8 bf16 values of a 16-byte word, given as any four pairs of it.
__device__ __forceinline__ float word_sum(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
    constexpr uint32_t kOnes = 0x3F803F80u;  // bfloat16 pair (1, 1)
    return dot2_bf16(d, kOnes, dot2_bf16(c, kOnes, dot2_bf16(b, kOnes, dot2_bf16(a, kOnes, 0.f))));
}

// Stage one chunk from its raw words (4 x 16 B for 4-bit codes, 2 x 16 B for
// 8-bit) read from global memory. `keep` is all ones, or zero for a lane past
// the end of the row.
template <int BITS>
__device__ __forceinline__ void stage_from_words(const u32x4 *d, uint32_t keep, uint32_t (&xv)[16], float &xs) {
    // (Masks and shifts rather than byte permutes, and one running sum: measured
    // faster here than the permute-and-pairwise form the LDS fill uses.)
    constexpr uint32_t kOnes = 0x3F803F80u;  // bfloat16 pair (1, 1)
    float s = 0.f;
    if constexpr (BITS == 4) {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const u32x4 q = d[t] & keep;
            xv[4 * t + 0] = (q.x & 0xFFFFu) | (q.z << 16);         // (x0, x4)
            xv[4 * t + 1] = (q.x >> 16) | (q.z & 0xFFFF0000u);     // (x1, x5)
            xv[4 * t + 2] = (q.y & 0xFFFFu) | (q.w << 16);         // (x2, x6)
            xv[4 * t + 3] = (q.y >> 16) | (q.w & 0xFFFF0000u);     // (x3, x7)
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) s = dot2_bf16(xv[i], kOnes, s);
    } else {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const u32x4 q = d[t] & keep;
            const uint32_t dw[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                xv[8 * t + 2 * i] = __float_as_uint(bf16_lo(dw[i]));
                xv[8 * t + 2 * i + 1] = __float_as_uint(bf16_hi(dw[i]));
                s = dot2_bf16(dw[i], kOnes, s);
            }
        }
    }
    xs = s;
}

// Raw activation words of chunk `c` (in range) of activation row `xr`, from
// global memory: 4 x 16 B (4-bit codes) or 2 x 16 B (8-bit codes).
template <int BITS>
__device__ __forceinline__ void fetch_x_chunk(const uint16_t *__restrict__ xr, int c, u32x4 (&d)[BITS == 4 ? 4 : 2]) {
    constexpr int W = BITS == 4 ? 4 : 2;
    const u32x4 *p = reinterpret_cast<const u32x4 *>(xr) + (int64_t)c * W;
#pragma unroll
    for (int t = 0; t < W; ++t) d[t] = p[t];
}

// The block's LDS copy of x [MW, K], already in staging form. Activation row
// m, chunk c < CP (CP = 64*CPT*XS, the chunks the block's lanes cover; zero
// past the row) is four 16-byte words at word (m*CP + c)*4; its sum of x is
// float (m*CP + c) after the MW*CP*4 words.
// FT: the fewest threads a block filling the copy has (the registers each
// thread holds between fetch_x and store_x are sized for it).
template <int BITS, int MW, int CPT, int XS, int FT = 256>
struct XFill {
    static constexpr int RAW = BITS == 4 ? 4 : 2;      // raw 16-byte words of x per chunk
    static constexpr int CP = 64 * CPT * XS;           // chunks per activation row in LDS
    static constexpr int WORDS = MW * CP * RAW;        // raw words of the padded copy
    static constexpr int PER = (WORDS + FT - 1) / FT;  // per thread
    static constexpr int BYTES = MW * CP * 68;         // LDS bytes
};

__device__ __forceinline__ float *x_lds_sums(int words) { return reinterpret_cast<float *>(g_xlds + words); }

// Block-cooperative copy of the activation rows rows(0..MW) (each 16-byte
// aligned) into LDS, in two halves. fetch_x issues the global loads into
// registers: thread t takes raw words t, t + blockDim, ... of the padded copy.
// store_x converts them to staging form, adds each chunk's word sums across
// the neighbouring lanes that hold them, and ends with a barrier that every
// wave of the block must reach. Weight loads issued between the two stay in
// flight: loads retire in order, so waiting for the x registers does not wait
// for anything issued later.
template <int BITS, int MW, int CPT, int XS, int FT, typename Rows>
__device__ __forceinline__ void fetch_x(const Rows &rows, int C, u32x4 (&xr)[XFill<BITS, MW, CPT, XS, FT>::PER]) {
    using F = XFill<BITS, MW, CPT, XS, FT>;
    const int per = (F::WORDS + (int)blockDim.x - 1) / (int)blockDim.x;  // block-uniform, <= PER
#pragma unroll
    for (int k = 0; k < F::PER; ++k) {
        if (k < per) {  // uniform branch
            const int i = (int)threadIdx.x + k * (int)blockDim.x;
            const int m = i / (F::CP * F::RAW), c = (i / F::RAW) % F::CP, t = i % F::RAW;
            const bool ok = i < F::WORDS && c < C;
            // Words past a row or past the copy read word 0 of row 0 and are zeroed in store_x.
            const u32x4 *src = reinterpret_cast<const u32x4 *>(rows(ok ? m : 0));
            xr[k] = src[ok ? c * F::RAW + t : 0];
        }
    }
}

template <int BITS, int MW, int CPT, int XS, int FT>
__device__ __forceinline__ void store_x(int C, const u32x4 (&xr)[XFill<BITS, MW, CPT, XS, FT>::PER]) {
    using F = XFill<BITS, MW, CPT, XS, FT>;
    float *sums = x_lds_sums(MW * F::CP * 4);
    const int per = (F::WORDS + (int)blockDim.x - 1) / (int)blockDim.x;
#pragma unroll
    for (int k = 0; k < F::PER; ++k) {
        if (k < per) {  // uniform branch: every lane runs the DPP below
            const int i = (int)threadIdx.x + k * (int)blockDim.x;
            const int chunk = i / F::RAW, c = chunk % F::CP, t = i % F::RAW;
            const bool in = i < F::WORDS;
            const u32x4 q = in && c < C ? xr[k] : u32x4{0u, 0u, 0u, 0u};
            float p;
            if constexpr (BITS == 4) {
                uint32_t o[4];
                pairs_of_word(q, o);
                if (in) g_xlds[chunk * 4 + t] = u32x4{o[0], o[1], o[2], o[3]};
                p = word_sum(o[0], o[1], o[2], o[3]);
                // The chunk's four words are in four neighbouring lanes (t = lane % 4):
                // (p0 + p1) + (p2 + p3) in every lane of the quad.
                p += dpp_f32<0xB1>(p);  // quad_perm [1,0,3,2]
                p += dpp_f32<0x4E>(p);  // quad_perm [2,3,0,1]
            } else {
                if (in) {
                    g_xlds[chunk * 4 + 2 * t] = u32x4{__float_as_uint(bf16_lo(q.x)), __float_as_uint(bf16_hi(q.x)),
                                                      __float_as_uint(bf16_lo(q.y)), __float_as_uint(bf16_hi(q.y))};
                    g_xlds[chunk * 4 + 2 * t + 1] = u32x4{__float_as_uint(bf16_lo(q.z)), __float_as_uint(bf16_hi(q.z)),
                                                          __float_as_uint(bf16_lo(q.w)), __float_as_uint(bf16_hi(q.w))};
                }
                p = word_sum(q.x, q.y, q.z, q.w);
                p += dpp_f32<0xB1>(p);  // the chunk's two words: lanes 2j, 2j+1
            }
            if (in && t == 0) sums[chunk] = p;
        }
    }
    __syncthreads();
}

// The norm weights matching the raw words fetch_x loads (zeros where it loads
// padding).
template <int BITS, int MW, int CPT, int XS, int FT>
__device__ __forceinline__ void fetch_gamma(const uint16_t *gamma, int K, int C,
                                            u32x4 (&gr)[XFill<BITS, MW, CPT, XS, FT>::PER]) {
    using F = XFill<BITS, MW, CPT, XS, FT>;
    const __amdgpu_buffer_rsrc_t rs = byte_range(gamma, (uint32_t)K * 2u);
    const int per = (F::WORDS + (int)blockDim.x - 1) / (int)blockDim.x;
#pragma unroll
    for (int k = 0; k < F::PER; ++k) {
        if (k < per) {  // uniform branch
            const int i = (int)threadIdx.x + k * (int)blockDim.x;
            const int c = (i / F::RAW) % F::CP, t = i % F::RAW;
            const bool ok = i < F::WORDS && c < C;
            gr[k] = __builtin_amdgcn_raw_buffer_load_b128(rs, ok ? (uint32_t)(c * F::RAW + t) * 16u : (uint32_t)K * 2u,
                                                          0, 0);
        }
    }
}

// RMS norm applied to the raw words of the block's fill (one activation row,
// each word of the row held by exactly one thread of the block): the block's
// sum of squares (wave sums, then the waves' sums in order through LDS `part`,
// at one block barrier), then x_n = bf16(x * rs * gamma) word by word.
template <int BITS, int MW, int CPT, int XS, int FT>
__device__ __forceinline__ void rms_norm_fill(int C, float inv_k, float eps, float *part,
                                              u32x4 (&xr)[XFill<BITS, MW, CPT, XS, FT>::PER],
                                              const u32x4 (&gr)[XFill<BITS, MW, CPT, XS, FT>::PER]) {
    using F = XFill<BITS, MW, CPT, XS, FT>;
    static_assert(MW == 1, "the block's fill normalizes one activation row");
    const int per = (F::WORDS + (int)blockDim.x - 1) / (int)blockDim.x;
    float ss = 0.f;
#pragma unroll
    for (int k = 0; k < F::PER; ++k) {
        if (k < per) {
            const int i = (int)threadIdx.x + k * (int)blockDim.x;
            const int c = (i / F::RAW) % F::CP;
            const u32x4 q = i < F::WORDS && c < C ? xr[k] : u32x4{0u, 0u, 0u, 0u};
            ss = dot2_bf16(q.x, q.x, ss);  // bf16 squares are exact in fp32
            ss = dot2_bf16(q.y, q.y, ss);
            ss = dot2_bf16(q.z, q.z, ss);
            ss = dot2_bf16(q.w, q.w, ss);
        }
    }
    const float pv[1] = {ss};
    float sum[1];
    wave_sums<1>(pv, sum);  // the total sits in lane 0
    if ((threadIdx.x & 63) == 0) part[wave_id()] = sum[0];
    __syncthreads();
    float tot = 0.f;
    const int waves = (int)blockDim.x >> 6;
    for (int w = 0; w < waves; ++w) tot += part[w];
    const float rs = __builtin_amdgcn_rsqf(tot * inv_k + eps);
#pragma unroll
    for (int k = 0; k < F::PER; ++k) {
        if (k < per) {
            const u32x4 q = xr[k], g = gr[k];
            xr[k] = u32x4{norm_pair(q.x, g.x, rs), norm_pair(q.y, g.y, rs), norm_pair(q.z, g.z, rs),
                          norm_pair(q.w, g.w, rs)};
        }
    }
}

// Stage chunk c (< CP) of activation row m from the block's LDS copy.
template <int BITS, int MW, int CPT, int XS>
__device__ __forceinline__ void stage_x_lds(int m, int c, uint32_t (&xv)[16], float &xs) {
    using F = XFill<BITS, MW, CPT, XS>;
    const int chunk = m * F::CP + c;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const u32x4 d = g_xlds[chunk * 4 + t];
        xv[4 * t + 0] = d.x;
        xv[4 * t + 1] = d.y;
        xv[4 * t + 2] = d.z;
        xv[4 * t + 3] = d.w;
    }
    xs = x_lds_sums(MW * F::CP * 4)[chunk];
}

// Partial dot product of one chunk with one staged activation slice.
// 4-bit: the accumulator starts at -128 * sum(x) (nxs), cancelling the 128 offset
// of the bfloat16 code pairs.
template <int BITS>
__device__ __forceinline__ float chunk_dot(const u32x4 &wv, const uint32_t (&xv)[16], float nxs) {
    const uint32_t w[4] = {wv.x, wv.y, wv.z, wv.w};
    if constexpr (BITS == 4) {
        float d = nxs;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const uint32_t lo = w[t] & 0x0F0F0F0Fu;
            const uint32_t hi = (w[t] >> 4) & 0x0F0F0F0Fu;
            d = dot2_bf16(byte_perm(kMagic43, lo, kSelEven), xv[4 * t + 0], d);
            d = dot2_bf16(byte_perm(kMagic43, hi, kSelEven), xv[4 * t + 1], d);
            d = dot2_bf16(byte_perm(kMagic43, lo, kSelOdd), xv[4 * t + 2], d);
            d = dot2_bf16(byte_perm(kMagic43, hi, kSelOdd), xv[4 * t + 3], d);
        }
        return d;
    } else {
        float d = 0.f;
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

// One iteration's worth of packed codes, scales and biases for R weight rows,
// and (INIT) one bf16 initial value per row: the accumulator of that row starts
// there (the fused projection's residual).
template <int CPT, int R, bool INIT = false>
struct RowBuf {
    u32x4 w[R][CPT];
    uint16_t s[R][CPT];  // 16-bit on purpose: a 32-bit copy would be zero-extended at the
    uint16_t b[R][CPT];  // loop entry, forcing a wait for these loads before the next ones
    uint32_t e[INIT ? R : 1];  // bf16 in the low half (scalar registers)
};

// The bf16 at p, read through the scalar data cache (p is wave-uniform): the
// aligned dword holding it, then its half. The dword never crosses a page
// boundary, so it reads nothing outside the page that holds p.
typedef const __attribute__((address_space(4))) uint32_t scalar_u32;
__device__ __forceinline__ uint32_t scalar_bf16(const uint16_t *p) {
    const uintptr_t a = reinterpret_cast<uintptr_t>(p);
    const uint32_t w = *reinterpret_cast<scalar_u32 *>(a & ~(uintptr_t)3);
    return (a & 2) ? (w >> 16) : (w & 0xFFFFu);
}

// The rows, scales and biases of one weight plane, with their row pitches.
struct Plane {
    const u32x4 *w;
    const uint16_t *s, *b;
    int64_t C, G;  // 16-byte chunks and 64-column groups per row
};

// Issue every load of rows [rb, rb + R) at once, through one buffer
// descriptor per row and array. A row at or past `end` gets an empty
// descriptor (its loads return zero and read nothing); chunks past the row end
// fall outside the row's descriptor and read zero too. No load is conditional,
// so the compiler's load-wait counts stay exact. Lane offsets are 32-bit byte
// offsets; row bases are scalar.
template <int CPT, int R, bool INIT = false>
__device__ __forceinline__ void load_rows(RowBuf<CPT, R, INIT> &buf, const Plane &pl, int64_t rb, int64_t end,
                                          const uint32_t (&woff)[CPT], const uint32_t (&goff)[CPT],
                                          const uint16_t *init = nullptr) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const bool in = rb + r < end;
        const int64_t row = in ? rb + r : 0;
        const __amdgpu_buffer_rsrc_t wr = byte_range(pl.w + row * pl.C, in ? (uint32_t)pl.C * 16u : 0u);
#pragma unroll
        for (int j = 0; j < CPT; ++j) buf.w[r][j] = __builtin_amdgcn_raw_buffer_load_b128(wr, woff[j], 0, kLoadNT);
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const bool in = rb + r < end;
        const int64_t row = in ? rb + r : 0;
        const __amdgpu_buffer_rsrc_t sr = byte_range(pl.s + row * pl.G, in ? (uint32_t)pl.G * 2u : 0u);
        const __amdgpu_buffer_rsrc_t br = byte_range(pl.b + row * pl.G, in ? (uint32_t)pl.G * 2u : 0u);
#pragma unroll
        for (int j = 0; j < CPT; ++j) {
            buf.s[r][j] = __builtin_amdgcn_raw_buffer_load_b16(sr, goff[j], 0, kLoadNT);
            buf.b[r][j] = __builtin_amdgcn_raw_buffer_load_b16(br, goff[j], 0, kLoadNT);
        }
    }
    if constexpr (INIT) {
        // One scalar load per row (no vector-memory instruction); rows past
        // the walk read row 0 and drop it.
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const bool in = rb + r < end;
            const uint32_t v = scalar_bf16(init + (in ? rb + r : 0));
            buf.e[r] = in ? v : 0u;
        }
    }
}

// Partial sums of one lane for R rows and MW activation rows.
template <int BITS, int CPT, int MW, int R, bool INIT>
__device__ __forceinline__ void compute_rows(const RowBuf<CPT, R, INIT> &buf, const uint32_t (&xv)[MW][CPT][16],
                                             const float (&xs)[MW][CPT], const float (&nxs)[MW][CPT],
                                             float (&acc)[R][MW]) {
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int m = 0; m < MW; ++m) acc[r][m] = 0.f;
#pragma unroll
    for (int r = 0; r < R; ++r) {
#pragma unroll
        for (int j = 0; j < CPT; ++j) {
            const float sf = bf16_lo((uint32_t)buf.s[r][j]);
            const float bf = bf16_lo((uint32_t)buf.b[r][j]);
#pragma unroll
            for (int m = 0; m < MW; ++m) {
                const float d = chunk_dot<BITS>(buf.w[r][j], xv[m][j], nxs[m][j]);
                acc[r][m] = fmaf(sf, d, acc[r][m]);
                acc[r][m] = fmaf(bf, xs[m][j], acc[r][m]);
            }
        }
    }
}

// Activation row m of a dense product: x[m, :]. (fill_threads: the fill
// registers of the LDS copy are sized for 256-thread blocks whatever the
// segment count, which measured faster for two segments than sizing them for
// the 512 threads such blocks have.)
struct DenseRows {
    static constexpr bool kNorm = false;
    const uint16_t *x;
    int64_t K;
    __device__ __forceinline__ const uint16_t *operator()(int m) const { return x + (int64_t)m * K; }
    template <int XS>
    static constexpr int fill_threads() { return 256; }
};

// Activation row m of a gather pass: x[xlist[m], :], with the pass's x rows
// listed in LDS.
struct GatherRows {
    static constexpr bool kNorm = false;
    const uint16_t *x;
    int64_t K;
    const uint32_t *xlist;
    __device__ __forceinline__ const uint16_t *operator()(int m) const { return x + (int64_t)xlist[m] * K; }
    // 256 threads per segment: sized for 256 threads, a two-segment copy of
    // eight rows spills the gather's registers.
    template <int XS>
    static constexpr int fill_threads() { return 256 * XS; }
};

// Output rows of the dense products: activation row m writes y[m, :].
// (kGlu: the rows pair up in a gated epilogue; kInit: rows start from initial
// values loaded with the weights.)
struct DenseOut {
    static constexpr bool kGlu = false;
    static constexpr bool kInit = false;
    uint16_t *y;
    int64_t N;
    __device__ __forceinline__ void put(int m, int64_t n, float v) const { y[(int64_t)m * N + n] = f32_to_bf16(v); }
};

// The weight rows a row group visits: iteration `it` covers rows
// [at(it), at(it) + R), dropping rows >= end. Row groups take R-row slices
// round-robin, so at any moment the whole grid reads one compact band of the
// matrix. Iterations past the walk land on rows >= end.
struct RowWalk {
    int64_t first;   // first row of iteration 0
    int64_t stride;  // rows between consecutive iterations
    int64_t end;     // rows >= end are neither read nor stored
    __device__ __forceinline__ int64_t at(int it) const { return first + (int64_t)it * stride; }
};

template <int R>
__device__ __forceinline__ RowWalk row_walk(const ProductArgs &a, int64_t rg, int64_t groups) {
    return RowWalk{rg * R, groups * R, a.N};
}

// A walk over row pairs (2p, 2p + 1), one row per iteration: iterations 2i
// and 2i + 1 read the two rows of pair first + i * stride. Gated epilogues use
// it to meet a gate row and its up row in consecutive iterations.
struct PairWalk {
    int64_t first;   // first pair
    int64_t stride;  // pairs between consecutive iteration pairs
    int64_t end;     // rows >= end are neither read nor stored
    __device__ __forceinline__ int64_t at(int it) const {
        return 2 * (first + (int64_t)(it >> 1) * stride) + (it & 1);
    }
};

// Reduce the lane partials of iteration `it` to row results and store them.
// All R*MW values are reduced together (wave_sums); value i = r*MW + m leaves
// in row rho = lane/16 of register i/4, and the first lane of that row owns it.
//  - S == 1: that lane stores it.
//  - S > 1: it goes to the wave's LDS slot for the iteration. Every F
//    iterations (and after the last) the block meets at one barrier and the
//    first wave of each row group adds the S waves' slots in a fixed order and
//    stores the rows. Two slot regions alternate, so one barrier per flush
//    suffices: a region is written again only after the next barrier, which
//    the combining wave reaches after its reads.
template <int MW, int R>
struct Flush {
    static constexpr int V = R * MW;
    static constexpr int F = 64 / V;  // iterations per flush: F*V <= 64 values, one per lane
};
constexpr int kSlotFloats = 64;  // per wave and region
constexpr int kBlockWaves = 8;   // __launch_bounds__(512)

// Gated epilogues with one row per iteration (a PairWalk, S == 1) hold the
// gate row's sum in `pend` until the up row's iteration.
template <int MW, int R, typename Out, typename Walk>
__device__ __forceinline__ void finish_rows(float (&acc)[R][MW], const Out &out, const Walk &walk, int it,
                                            int iters, int S, int wig, int grp, int lane, float *red,
                                            float &pend) {
    constexpr int V = Flush<MW, R>::V;
    float v[V], t[sum_regs(V)];
#pragma unroll
    for (int i = 0; i < V; ++i) v[i] = acc[i / MW][i % MW];
    wave_sums<V>(v, t);
    const int rho = lane >> 4;
    const bool leader = (lane & 15) == 0;
    if (S == 1) {
        const int64_t rb = walk.at(it);
#pragma unroll
        for (int j = 0; j < sum_regs(V); ++j) {
            const int i = 4 * j + sum_slot(rho);
            const int r = i / MW, m = i % MW;
            if constexpr (Out::kGlu && R == 1) {
                // A PairWalk: even iterations reduce a gate row, odd ones its up row.
                if (it & 1) {
                    if (leader && rho == 0 && rb < walk.end) out.glu(rb >> 1, pend, t[j]);
                } else {
                    pend = t[j];
                }
            } else if constexpr (Out::kGlu) {
                // One activation row, R even: the gate rows (i even) sit in lane rows
                // 0 and 1, their up rows (i + 1) in lane rows 2 and 3 of the same register.
                const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(t[j]), __float_as_uint(t[j]),
                                                                 false, false);
                const float up = __uint_as_float(sw[1]);  // lanes < 32: t[j] of lane + 32
                if (leader && rho < 2 && i < V && rb + r < walk.end) out.glu((rb + r) >> 1, t[j], up);
            } else {
                if (leader && i < V && rb + r < walk.end) out.put(m, rb + r, t[j]);
            }
        }
        return;
    }
    constexpr int F = Flush<MW, R>::F;
    const int slot = it % F;
    float *region = red + ((it / F) & 1) * (kBlockWaves * kSlotFloats);
#pragma unroll
    for (int j = 0; j < sum_regs(V); ++j) {
        const int i = 4 * j + sum_slot(rho);
        if (leader && i < V) region[(grp * S + wig) * kSlotFloats + slot * V + i] = t[j];
    }
    if (slot == F - 1 || it == iters - 1) {  // uniform over the block (equal iteration counts)
        __syncthreads();
        if constexpr (Out::kGlu) {
            // One activation row: lane 2u holds a gate row, lane 2u + 1 its up row (R
            // even, or a PairWalk with one row per iteration: flushes start at even
            // iterations).
            // (Every lane of the wave sums, so the neighbour exchange sees active lanes;
            // lanes past the flushed values read slots they do not store.)
            if (wig == 0) {
                float tot = 0.f;
                for (int s = 0; s < S; ++s) tot += region[(grp * S + s) * kSlotFloats + lane];
                const float up = dpp_f32<0xB1>(tot);  // lane ^ 1
                const int64_t row = walk.at(it - slot + lane / V) + lane % V;
                if (lane < (slot + 1) * V && (lane & 1) == 0 && row < walk.end) out.glu(row >> 1, tot, up);
            }
        } else if (wig == 0 && lane < (slot + 1) * V) {
            float tot = 0.f;
            for (int s = 0; s < S; ++s) tot += region[(grp * S + s) * kSlotFloats + lane];
            const int i = lane % V, r = i / MW, m = i % MW;
            const int64_t row = walk.at(it - slot + lane / V) + r;
            if (row < walk.end) out.put(m, row, tot);
        }
    }
}

// Initial values of the rows (Out::kInit), or NULL.
template <typename Out>
__device__ __forceinline__ const uint16_t *init_values(const Out &out) {
    if constexpr (Out::kInit)
        return out.init;
    else
        return nullptr;
}

// Add the rows' initial values to the partials of one lane of the row group
// (activation row 0), so that the wave and K-split sums carry them once.
template <int CPT, int R, bool INIT, int MW>
__device__ __forceinline__ void add_init(const RowBuf<CPT, R, INIT> &buf, float (&acc)[R][MW], bool owner) {
    if constexpr (INIT) {
#pragma unroll
        for (int r = 0; r < R; ++r) acc[r][0] += owner ? bf16_lo(buf.e[r]) : 0.f;
    }
}

// RMS norm of one activation row, applied to the raw bf16 words a wave has
// loaded: x_n = bf16(x * rs * gamma) with rs = 1 / sqrt(sum(x^2) / K + eps)
// (v_rsq_f32 of the mean square plus eps, the mean as a product with 1/K).
// The sum of squares (lanes past the row end add nothing) is a wave sum; with
// S > 1 the S waves of the row group add their sums through LDS, in order, at
// one block barrier (every wave of the block calls this).
template <int CPT, int XC, typename Rows>
__device__ __forceinline__ void rms_norm_words(const Rows &xrows, u32x4 (&xw)[CPT][XC],
                                               const u32x4 (&gw)[CPT][XC], const bool (&cv)[CPT], int S, int wig,
                                               int grp, int lane) {
    float ss = 0.f;
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
        const uint32_t keep = cv[j] ? 0xFFFFFFFFu : 0u;
#pragma unroll
        for (int t = 0; t < XC; ++t) {
            const u32x4 q = xw[j][t] & keep;
            ss = dot2_bf16(q.x, q.x, ss);  // bf16 squares are exact in fp32
            ss = dot2_bf16(q.y, q.y, ss);
            ss = dot2_bf16(q.z, q.z, ss);
            ss = dot2_bf16(q.w, q.w, ss);
        }
    }
    const float part[1] = {ss};
    float sum[1];
    wave_sums<1>(part, sum);  // the total sits in lane 0
    float tot = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(sum[0]), 0));
    if (S > 1) {
        if (lane == 0) xrows.part[grp * S + wig] = tot;
        __syncthreads();
        tot = 0.f;
        for (int s = 0; s < S; ++s) tot += xrows.part[grp * S + s];
    }
    const float rs = __builtin_amdgcn_rsqf(tot * xrows.inv_k + xrows.eps);
#pragma unroll
    for (int j = 0; j < CPT; ++j)
#pragma unroll
        for (int t = 0; t < XC; ++t) {
            const u32x4 q = xw[j][t], g = gw[j][t];
            xw[j][t] = u32x4{norm_pair(q.x, g.x, rs), norm_pair(q.y, g.y, rs), norm_pair(q.z, g.z, rs),
                             norm_pair(q.w, g.w, rs)};
        }
}

// Shared core: MW activation rows (xrows(m), m < MW) against the weight rows
// that `walk` visits in one plane; row n of activation row m goes to
// out.put(m, n, .) (or, for a gated Out, each gate/up row pair to out.glu).
// `iters` (a multiple of NB) must be equal for every row group of the block
// when S > 1 or XS > 0 (block-wide barriers), or when Rows normalizes x with
// S > 1 (one more block barrier).
//
// The row loop streams through a ring of NB register buffers: each buffer is
// refilled with the rows NB iterations ahead as soon as it has been consumed.
// Rows past the walk read nothing (empty descriptors).
template <int BITS, int CPT, int MW, int R, int NB, int XS, typename Rows, typename Out, typename Walk>
__device__ __forceinline__ void product_rows(const ProductArgs &a, const Plane &pl, const Rows &xrows,
                                             const Out &out, const Walk &walk, int iters, float *red) {
    const int lane = threadIdx.x & 63;
    const int wave = wave_id();
    const int S = a.S;
    const int wig = wave % S;
    const int grp = wave / S;

    int chunk[CPT];
    bool cv[CPT];
    uint32_t woff[CPT], goff[CPT];
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
        chunk[j] = (wig * CPT + j) * 64 + lane;
        cv[j] = chunk[j] < a.C;
        woff[j] = (uint32_t)chunk[j] * 16u;
        goff[j] = (uint32_t)(chunk[j] >> a.gshift) * 2u;  // the chunk's scale group
    }

    constexpr bool INIT = Out::kInit;
    const uint16_t *init = init_values(out);
    RowBuf<CPT, R, INIT> buf[NB];
    // Order: x loads, then the first iteration's weight loads, then wait for x
    // alone (loads retire in order) and stage it while those are in flight;
    // then the loads of the other NB-1 ring stages. (Issuing every stage ahead
    // of the staging delays the first stage's data for a wave that cannot
    // start before it.)
    // XS > 0 (compile time): the block copies x into LDS in staging form and
    // every wave reads its slice from there; otherwise each wave reads and
    // stages its slice from global memory. One code path per kernel keeps the
    // compiler's load-wait placement exact. Lanes past the row end stage zeros.
    constexpr int XC = BITS == 4 ? 4 : 2;  // 16-byte words of x per chunk
    constexpr bool XL = XS > 0;
    constexpr int FT = Rows::template fill_threads<XS == 0 ? 1 : XS>();
    using XF = XFill<BITS, MW, CPT, XS == 0 ? 1 : XS, FT>;
    u32x4 xr[XL ? XF::PER : 1];
    u32x4 gr[XL && Rows::kNorm ? XF::PER : 1];
    u32x4 xraw[XL ? 1 : MW][XL ? 1 : CPT][XC];
    if constexpr (XL) {
        fetch_x<BITS, MW, CPT, XS, FT>(xrows, a.C, xr);
        if constexpr (Rows::kNorm) fetch_gamma<BITS, MW, CPT, XS, FT>(xrows.gamma, a.K, a.C, gr);
    } else {
#pragma unroll
        for (int m = 0; m < MW; ++m) {
            const uint16_t *xm = xrows(m);
#pragma unroll
            for (int j = 0; j < CPT; ++j) fetch_x_chunk<BITS>(xm, cv[j] ? chunk[j] : a.C - 1, xraw[m][j]);
        }
    }
    // The norm weights of the lane's columns (Rows::kNorm, x staged by each
    // wave): zeros past the row end.
    u32x4 graw[Rows::kNorm && !XL ? CPT : 1][XC];
    if constexpr (Rows::kNorm && !XL) {
        static_assert(MW == 1, "the RMS norm prologue stages one activation row per wave");
        const __amdgpu_buffer_rsrc_t gr = byte_range(xrows.gamma, (uint32_t)a.K * 2u);
#pragma unroll
        for (int j = 0; j < CPT; ++j)
#pragma unroll
            for (int t = 0; t < XC; ++t)
                graw[j][t] = __builtin_amdgcn_raw_buffer_load_b128(gr, (uint32_t)(chunk[j] * XC + t) * 16u, 0, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    // With the norm in the block's fill (two block barriers before the first
    // product), every stage of the ring is issued first, so the weight stream
    // runs during the prologue.
    constexpr int EARLY = Rows::kNorm && XL ? NB : 1;
#pragma unroll
    for (int p = 0; p < EARLY; ++p) load_rows<CPT, R, INIT>(buf[p], pl, walk.at(p), walk.end, woff, goff, init);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (Rows::kNorm && !XL) rms_norm_words<CPT, XC>(xrows, xraw[0], graw, cv, S, wig, grp, lane);

    uint32_t xv[MW][CPT][16];
    float xs[MW][CPT], nxs[MW][CPT];
    if constexpr (XL) {
        if constexpr (Rows::kNorm) rms_norm_fill<BITS, MW, CPT, XS, FT>(a.C, xrows.inv_k, xrows.eps, xrows.part, xr, gr);
        store_x<BITS, MW, CPT, XS, FT>(a.C, xr);  // block barrier: every wave of the block gets here
#pragma unroll
        for (int m = 0; m < MW; ++m)
#pragma unroll
            for (int j = 0; j < CPT; ++j) stage_x_lds<BITS, MW, CPT, XS>(m, chunk[j], xv[m][j], xs[m][j]);
    } else {
#pragma unroll
        for (int m = 0; m < MW; ++m)
#pragma unroll
            for (int j = 0; j < CPT; ++j) stage_from_words<BITS>(xraw[m][j], cv[j] ? 0xFFFFFFFFu : 0u, xv[m][j], xs[m][j]);
    }
#pragma unroll
    for (int m = 0; m < MW; ++m)
#pragma unroll
        for (int j = 0; j < CPT; ++j) nxs[m][j] = BITS == 4 ? -128.f * xs[m][j] : 0.f;
#pragma unroll
    for (int p = EARLY; p < NB; ++p) load_rows<CPT, R, INIT>(buf[p], pl, walk.at(p), walk.end, woff, goff, init);
    __builtin_amdgcn_sched_barrier(0);

    // Every turn of the ring but the last refills each buffer NB iterations
    // ahead once it is consumed; the last turn (iterations iters-NB .. iters-1)
    // issues no loads. (Refills past the walk would read nothing, but each
    // load instruction still costs address-unit time.)
    float acc[R][MW];
    float pend = 0.f;
    int it0 = 0;
    for (; it0 + NB < iters; it0 += NB) {
#pragma unroll
        for (int p = 0; p < NB; ++p) {
            compute_rows<BITS, CPT, MW, R>(buf[p], xv, xs, nxs, acc);
            add_init(buf[p], acc, lane == 0 && wig == 0);
            finish_rows<MW, R>(acc, out, walk, it0 + p, iters, S, wig, grp, lane, red, pend);
            load_rows<CPT, R, INIT>(buf[p], pl, walk.at(it0 + p + NB), walk.end, woff, goff, init);
            // Keep the next buffer's use below this refill.
            __builtin_amdgcn_sched_barrier(0);
        }
    }
#pragma unroll
    for (int p = 0; p < NB; ++p) {
        compute_rows<BITS, CPT, MW, R>(buf[p], xv, xs, nxs, acc);
        add_init(buf[p], acc, lane == 0 && wig == 0);
        finish_rows<MW, R>(acc, out, walk, it0 + p, iters, S, wig, grp, lane, red, pend);
    }
    if (S > 1) __syncthreads();  // the LDS slots are reused by the caller's next pass
}

// LDS slots of the K-split combine: two regions of kSlotFloats per wave.
constexpr int kRedFloats = 2 * kBlockWaves * kSlotFloats;

}  // namespace agq
