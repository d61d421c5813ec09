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

namespace agq {



// Dynamic LDS of the product kernels: the block's copy of x (XFill).
extern __shared__ u32x4 g_xlds[];


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

// One iteration's worth of packed codes, scales and biases for R weight rows.
template <int CPT, int R>
struct RowBuf {
    u32x4 w[R][CPT];
    uint16_t s[R][CPT];  // 16-bit on purpose: a 32-bit copy would be zero-extended at the
    uint16_t b[R][CPT];  // loop entry, forcing a wait for these loads before the next ones
};

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
template <int CPT, int R>
__device__ __forceinline__ void load_rows(RowBuf<CPT, R> &buf, const Plane &pl, int64_t rb, int64_t end,
                                          const uint32_t (&woff)[CPT], const uint32_t (&goff)[CPT]) {
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
}

// Partial sums of one lane for R rows and MW activation rows.
template <int BITS, int CPT, int MW, int R>
__device__ __forceinline__ void compute_rows(const RowBuf<CPT, R> &buf, const uint32_t (&xv)[MW][CPT][16],
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
    const uint16_t *x;
    int64_t K;
    __device__ __forceinline__ const uint16_t *operator()(int m) const { return x + (int64_t)m * K; }
    template <int XS>
    static constexpr int fill_threads() { return 256; }
};

// Activation row m of a gather pass: x[xlist[m], :], with the pass's x rows
// listed in LDS.
struct GatherRows {
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
struct DenseOut {
    uint16_t *y;
    int64_t N;
    __device__ __forceinline__ uint16_t *operator()(int m) const { return y + (int64_t)m * N; }
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

template <int MW, int R, typename Out>
__device__ __forceinline__ void finish_rows(float (&acc)[R][MW], const Out &out, const RowWalk &walk, int it,
                                            int iters, int S, int wig, int grp, int lane, float *red) {
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
            if (leader && i < V && rb + r < walk.end) out(m)[rb + r] = f32_to_bf16(t[j]);
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
        if (wig == 0 && lane < (slot + 1) * V) {
            float tot = 0.f;
            for (int s = 0; s < S; ++s) tot += region[(grp * S + s) * kSlotFloats + lane];
            const int i = lane % V, r = i / MW, m = i % MW;
            const int64_t row = walk.at(it - slot + lane / V) + r;
            if (row < walk.end) out(m)[row] = f32_to_bf16(tot);
        }
    }
}

// Shared core: MW activation rows (xrows(m), m < MW) against the weight rows
// that `walk` visits in one plane; row n of activation row m goes to out(m)[n].
// `iters` (a multiple of NB) must be equal for every row group of the block
// when S > 1 or XS > 0 (block-wide barriers).
//
// The row loop streams through a ring of NB register buffers: each buffer is
// refilled with the rows NB iterations ahead as soon as it has been consumed.
// Rows past the walk read nothing (empty descriptors).
template <int BITS, int CPT, int MW, int R, int NB, int XS, typename Rows, typename Out>
__device__ __forceinline__ void product_rows(const ProductArgs &a, const Plane &pl, const Rows &xrows,
                                             const Out &out, const RowWalk &walk, int iters, float *red) {
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

    RowBuf<CPT, R> buf[NB];
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
    u32x4 xraw[XL ? 1 : MW][XL ? 1 : CPT][XC];
    if constexpr (XL) {
        fetch_x<BITS, MW, CPT, XS, FT>(xrows, a.C, xr);
    } else {
#pragma unroll
        for (int m = 0; m < MW; ++m) {
            const uint16_t *xm = xrows(m);
#pragma unroll
            for (int j = 0; j < CPT; ++j) fetch_x_chunk<BITS>(xm, cv[j] ? chunk[j] : a.C - 1, xraw[m][j]);
        }
    }
    __builtin_amdgcn_sched_barrier(0);
    load_rows<CPT, R>(buf[0], pl, walk.at(0), walk.end, woff, goff);
    __builtin_amdgcn_sched_barrier(0);

    uint32_t xv[MW][CPT][16];
    float xs[MW][CPT], nxs[MW][CPT];
    if constexpr (XL) {
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
    for (int p = 1; p < NB; ++p) load_rows<CPT, R>(buf[p], pl, walk.at(p), walk.end, woff, goff);
    __builtin_amdgcn_sched_barrier(0);

    // Every turn of the ring but the last refills each buffer NB iterations
    // ahead once it is consumed; the last turn (iterations iters-NB .. iters-1)
    // issues no loads. (Refills past the walk would read nothing, but each
    // load instruction still costs address-unit time.)
    float acc[R][MW];
    int it0 = 0;
    for (; it0 + NB < iters; it0 += NB) {
#pragma unroll
        for (int p = 0; p < NB; ++p) {
            compute_rows<BITS, CPT, MW, R>(buf[p], xv, xs, nxs, acc);
            finish_rows<MW, R>(acc, out, walk, it0 + p, iters, S, wig, grp, lane, red);
            load_rows<CPT, R>(buf[p], pl, walk.at(it0 + p + NB), walk.end, woff, goff);
            // Keep the next buffer's use below this refill.
            __builtin_amdgcn_sched_barrier(0);
        }
    }
#pragma unroll
    for (int p = 0; p < NB; ++p) {
        compute_rows<BITS, CPT, MW, R>(buf[p], xv, xs, nxs, acc);
        finish_rows<MW, R>(acc, out, walk, it0 + p, iters, S, wig, grp, lane, red);
    }
    if (S > 1) __syncthreads();  // the LDS slots are reused by the caller's next pass
}

// LDS slots of the K-split combine: two regions of kSlotFloats per wave.
constexpr int kRedFloats = 2 * kBlockWaves * kSlotFloats;

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
    uint16_t *y;
    int64_t N;
    const uint16_t *plist;
    __device__ __forceinline__ uint16_t *operator()(int m) const { return y + (int64_t)plist[m] * N; }
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
