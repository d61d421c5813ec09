// Matrix-core building blocks shared by the small-batch, gather and MoE
// kernels (qmv_mfma.hip, moe_mfma.hip).
//
// Same operands and result as the VALU kernels (qmv_kernels.hip): BF16
// activations x [M, K], U32-packed 4-bit codes (low-first) [N, K/8], BF16
// scale and bias per 64-column group (operand triple of "MLX CUDA Cleanup
// Plan", Target Architecture §1), and
//     y[m,n] = sum_g s[n,g] * (sum_{k in g} x[m,k]*(128+q[n,k]) - 128*X[m,g]) + b[n,g]*X[m,g]
//            = sum_g s[n,g] * D[m,n,g] + (b[n,g] - 128*s[n,g]) * X[m,g],
// with X[m,g] the sum of x over group g. This is sum_k x*(s*q + b) regrouped.
//
// With several activation rows the VALU form issues 4*M dot products per
// packed word and becomes issue-bound (M = 8: about 60 VALU instructions per
// word). Here v_mfma_f32_16x16x32_bf16 forms D:
//  - A (16 x 32): activation rows, lane l holds row m = l % 16. Rows past the
//    pass read zero (the buffer descriptor's range), so up to 16 rows share
//    one instruction.
//  - B (32 x 16): 16 weight rows as bfloat16 (128 + q), lane l holds row
//    n = l % 16. A code q sits in the low mantissa bits of 0x4300 (128.0),
//    so one byte permute per two codes builds the operand.
//  - D (16 x 16): lane l holds D[4*(l/16) + r][l % 16], r < 4.
// In A and B alike, lane group g = l / 16 supplies 8 of the 32 columns, as
// the four bfloat16 pairs (c0,c4), (c1,c5), (c2,c6), (c3,c7) of one packed
// word (8 consecutive columns c0..c7). The activations are arranged the same
// way, so only the pairing of lanes with columns matters.
//
// Work decomposition. A tile is 16 weight rows; a band is T tiles. K splits
// into segments of 128 columns (64 bytes of codes per row, two groups),
// processed in pairs (a 128-byte window per row). Lane group g of the B
// operand needs the 16-byte quarter g of its row's segment. Line loads read
// the window in whole 128-byte lines, 8 rows per instruction, and each lane
// moves its pieces to their lanes through a per-wave LDS buffer. (Reading the
// quarters directly, 64 contiguous bytes from each of 16 rows per
// instruction, measured slower.) One v_permlane32_swap per two words
// then regroups the words so that each MFMA sees columns of a single
// 64-column group (the scale changes per group): after swapping words (0,2)
// and (1,3) between the wave halves, words 0 and 1 of every lane hold columns
// of the segment's first group and words 2 and 3 of the second. Slot (h, t)
// (h = group, t = word) of lane group g covers columns
// 64h + 32(g%2) + 8(t + 2(g/2)) .. +8 of the segment.
//
// S waves split K (each owns SPW consecutive segments) and form a block; the
// block walks bands round-robin. Per segment a wave loads the A operands of
// its activation slice (from L2, shared by the band's T tiles), the codes of
// T tiles, and every fourth segment the
// scales and biases of the next 8 groups of each tile row. Loads run 4
// segments ahead in a ring. X[m,g] comes from the same A operands against an
// all-ones B. At the end of a band the S waves' partial sums meet in LDS in a
// fixed order, so results are deterministic.

#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "plan.hpp"
#include "plan_mfma.hpp"
#include "qmv_device.hpp"
#include "qmv_kernels.hpp"

namespace agq {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

namespace mfma {

constexpr int kRing = kMfmaRing;  // segments in flight per wave
constexpr int kSB = 4;            // segments per block of scales (8 groups, 16 bytes per row)
// Codes load in whole 128-byte lines, 8 rows per load, and move to their lanes
// through a 2 KB LDS buffer per wave and tile (gather W1 / W2: 78.2 / 76.7 ->
// 73.1 / 66.0 us against 64-byte quarters of 16 rows per load; 4096x14336 at
// M = 8: 16.0 -> 14.7 us).
constexpr uint32_t kOnes = 0x3F803F80u;  // bfloat16 pair (1, 1)
constexpr int kRsrcW3 = 0x00020000;      // raw buffer, 32-bit data format
// Cache policy of the code, scale and bias loads. Codes stream through once
// in whole lines: non-temporal, which keeps the L2 for x (gather W1 / W2:
// 74.7 / 69.6 -> 70.0 / 63.8 us). Scale loads read 16 bytes of a line and
// later loads the rest, so they are cached normally (non-temporal: 2-8% slower).
constexpr int kWPolicy = 2;
constexpr int kSPolicy = 0;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t range_of(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, (int)bytes, kRsrcW3);
}

__device__ __forceinline__ f32x4 mfma(const u32x4 &a, const u32x4 &b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                   0, 0, 0);
}

// B operand slice of one packed word: (128 + q) pairs (q0,q4), (q1,q5), (q2,q6), (q3,q7).
__device__ __forceinline__ u32x4 code_pairs(uint32_t w) {
    const uint32_t lo = w & 0x0F0F0F0Fu, hi = (w >> 4) & 0x0F0F0F0Fu;
    return u32x4{byte_perm(kMagic43, lo, kSelEven), byte_perm(kMagic43, hi, kSelEven),
                 byte_perm(kMagic43, lo, kSelOdd), byte_perm(kMagic43, hi, kSelOdd)};
}

// A operand slice of 8 activations x0..x7 (one 16-byte word): (x0,x4), (x1,x5), (x2,x6), (x3,x7).
__device__ __forceinline__ u32x4 act_pairs(const u32x4 &q) {
    return u32x4{byte_perm(q.z, q.x, 0x05040100u), byte_perm(q.z, q.x, 0x07060302u),
                 byte_perm(q.w, q.y, 0x05040100u), byte_perm(q.w, q.y, 0x07060302u)};
}

// One segment's loads: 16 bytes of codes per tile, and the lane's 4 / XQ
// activation words (XQ: the activation load form, below).
template <int T, int XQ>
struct Seg {
    u32x4 x[4 / XQ];
    u32x4 w[T];
};

// Activation load forms. The A operand needs slots i = 0..3 (i = 2h + t) of
// each pass row m in lane m of every lane group, and with few rows most lanes
// of a direct load would read nothing.
//  - XQ = 1 (passes of up to 16 rows): 4 loads per lane, slots 0-3 of its row.
//  - XQ = 4 (up to 4 rows): lane m of a group loads slot m / 4 of row m % 4,
//    one load instead of 4, and rotations within the 16-lane row bring slot i
//    of row r from lane r + 4i to lane r.
//  - XQ = 2 (up to 8 rows): staged. Load k of lane m in group g reads word m
//    (columns 8m..8m+7) of segment row 4k + g, contiguous 256-byte rows. At
//    compute time the lane unpacks its two words into A operand form (half
//    the byte permutes of XQ = 1) and writes them to a 4 KB per-wave LDS
//    buffer (both segments of the pair), slot row*16 + (word ^ row), from
//    which every lane reads its 4 slots. Writes and reads are free of bank
//    conflicts, and the LDS pipe takes work off the VALU, which bounds these
//    kernels. (Rotations for 8 rows instead, two loads and 8 moves per
//    segment, measured slower than XQ = 1: 14336x4096 at M = 8, 13.3 -> 13.9 us.)
// Lanes m >= 16 / XQ then hold other slots of the same rows: their A rows, and
// the D rows they produce, are never stored.
template <int N>
__device__ __forceinline__ u32x4 row_ror(const u32x4 &v) {
    // DPP row_ror:N: lane i of each 16-lane row receives lane (i - N) mod 16.
    return u32x4{(uint32_t)__builtin_amdgcn_update_dpp(0, (int)v.x, 0x120 + N, 0xF, 0xF, true),
                 (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v.y, 0x120 + N, 0xF, 0xF, true),
                 (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v.z, 0x120 + N, 0xF, 0xF, true),
                 (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v.w, 0x120 + N, 0xF, 0xF, true)};
}

// Dynamic LDS of the gather kernel: its pair list and their x rows.
extern __shared__ u32x4 g_mfma_dyn[];

// Scales and biases of 8 groups (4 segments) per tile row: dword j holds the
// bf16 pair of segment j's two groups.
template <int T>
struct ScaleBlock {
    u32x4 s[T], b[T];
};

// Per-wave constants of a pass.
struct Lanes {
    uint32_t wlo;       // line loads: byte offset of the lane's 16 bytes in rows 0-7 of a tile's 128-byte window
    uint32_t wslot[2];  // line loads: LDS slots (16-byte units) the lane writes its rows 0-7 and 8-15 data to
    uint32_t rslot[2];  // line loads: LDS slots the lane reads segments 0 and 1 of the window from
    uint32_t soff;      // byte offset of the lane's scale row within a tile
    uint32_t xoff[4];   // byte offsets of the lane's 4 / XQ activation words (compact loads), segment 0
    uint32_t xw[2];     // staged activations (XQ 2): LDS slots the lane writes its two words to
    uint32_t xrd[4];    // staged activations: LDS slots of the lane's 4 A operand words
};

// One plane's band geometry and operand ranges. A dual band (the gate and up
// projections of a GLU) takes tile 0 from (w, s, b) and tile 1 from (w2, s2,
// b2), both at the band's 16 rows; otherwise tile t holds rows 16*t .. of the
// band's 16*T.
struct Band {
    const uint8_t *w;  // plane codes
    const uint16_t *s, *b;
    int64_t N;
    uint32_t rowbytes;  // K / 2
    int32_t G;
    const uint8_t *w2 = nullptr;  // dual bands: tile 1
    const uint16_t *s2 = nullptr, *b2 = nullptr;
};

// Codes of one segment per tile. Units of a segment pair take turns: the
// even unit reads rows 0-7 and the odd one rows 8-15 of the pair's 128-byte
// window (8 whole lines per instruction), and compute_pair moves the bytes to
// their lanes through LDS.
template <int T, bool SCALES, int XQ, bool DUAL = false>
__device__ __forceinline__ void load_seg(Seg<T, XQ> &u, ScaleBlock<T> &sb, const Band &bd, const Lanes &ln,
                                         __amdgpu_buffer_rsrc_t xr, int64_t band, int seg) {
#pragma unroll
    for (int t = 0; t < T; ++t) {
        const int64_t row0 = DUAL ? band * 16 : band * (16 * T) + 16 * t;
        const uint8_t *wp = DUAL && t == 1 ? bd.w2 : bd.w;
        const uint16_t *sp = DUAL && t == 1 ? bd.s2 : bd.s;
        const uint16_t *bp = DUAL && t == 1 ? bd.b2 : bd.b;
        const int64_t left = bd.N - row0;
        const uint32_t rows = left <= 0 ? 0u : left >= 16 ? 16u : (uint32_t)left;
        const int64_t r0 = left <= 0 ? 0 : row0;
        u.w[t] = __builtin_amdgcn_raw_buffer_load_b128(range_of(wp + r0 * bd.rowbytes, rows * bd.rowbytes),
                                                       ln.wlo + ((uint32_t)seg & 1u) * 8u * bd.rowbytes,
                                                       (seg >> 1) * 128, kWPolicy);
        if constexpr (SCALES) {
            const uint32_t sbytes = rows * (uint32_t)bd.G * 2u;
            sb.s[t] = __builtin_amdgcn_raw_buffer_load_b128(range_of(sp + r0 * bd.G, sbytes), ln.soff, seg * 4,
                                                            kSPolicy);
            sb.b[t] = __builtin_amdgcn_raw_buffer_load_b128(range_of(bp + r0 * bd.G, sbytes), ln.soff, seg * 4,
                                                            kSPolicy);
        }
    }
#pragma unroll
    for (int i = 0; i < 4 / XQ; ++i) u.x[i] = __builtin_amdgcn_raw_buffer_load_b128(xr, ln.xoff[i], seg * 256, 0);
}

// Fold one segment into the band's accumulators. sd/bd: the bf16 scale and
// bias pairs of the segment's two groups for the lane's row of each tile.
template <int T, int XQ>
__device__ __forceinline__ void compute_seg(const u32x4 *ux, const u32x4 (&w)[T], const uint32_t (&sd)[T],
                                            const uint32_t (&bd)[T], f32x4 (&acc)[T], const u32x4 *ax) {
    const f32x4 z = {0.f, 0.f, 0.f, 0.f};
    const u32x4 ones = {kOnes, kOnes, kOnes, kOnes};
    u32x4 a[4];
    if constexpr (XQ == 1) {
#pragma unroll
        for (int i = 0; i < 4; ++i) a[i] = act_pairs(ux[i]);
    } else if constexpr (XQ == 2) {
#pragma unroll
        for (int i = 0; i < 4; ++i) a[i] = ax[i];
    } else {
        static_assert(XQ == 4, "activation loads: 4 full loads (XQ 1), staged (XQ 2) or compact (XQ 4)");
        a[0] = act_pairs(ux[0]);
        a[1] = row_ror<12>(a[0]);
        a[2] = row_ror<8>(a[0]);
        a[3] = row_ror<4>(a[0]);
    }
    // X[m, g] of the two groups, in the D layout.
    const f32x4 x0 = mfma(a[1], ones, mfma(a[0], ones, z));
    const f32x4 x1 = mfma(a[3], ones, mfma(a[2], ones, z));
#pragma unroll
    for (int t = 0; t < T; ++t) {
        const auto p02 = __builtin_amdgcn_permlane32_swap(w[t].x, w[t].z, false, false);
        const auto p13 = __builtin_amdgcn_permlane32_swap(w[t].y, w[t].w, false, false);
        const f32x4 d0 = mfma(a[1], code_pairs(p13[0]), mfma(a[0], code_pairs(p02[0]), z));
        const f32x4 d1 = mfma(a[3], code_pairs(p13[1]), mfma(a[2], code_pairs(p02[1]), z));
        const float s0 = bf16_lo(sd[t]), s1 = bf16_hi(sd[t]);
        const float c0 = fmaf(-128.f, s0, bf16_lo(bd[t])), c1 = fmaf(-128.f, s1, bf16_hi(bd[t]));
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            float v = acc[t][r];
            v = fmaf(s0, d0[r], v);
            v = fmaf(c0, x0[r], v);
            v = fmaf(s1, d1[r], v);
            v = fmaf(c1, x1[r], v);
            acc[t][r] = v;
        }
    }
}

// Segments p and p+1 (a 128-byte window) of every tile. The even unit holds
// rows 0-7 and the odd one rows 8-15 of the window; each lane writes both to
// the wave's LDS buffer and reads back its own row and quarter of either
// segment. Slots are XOR-swizzled so that neither the writes nor the reads
// conflict. A wave's LDS accesses complete in order, so the buffer needs no
// barrier. Once the pair's codes (and staged activations) sit in LDS, its
// registers are free: `reload` issues the loads of the ring's next turn into
// them before the arithmetic, so the refill waits for the data, not for the
// compute (4096x14336 at M = 4 / 8: 12.75 / 13.16 -> 11.82 / 12.49 us).
template <int T, int XQ, typename Reload>
__device__ __forceinline__ void compute_pair(Seg<T, XQ> &u0, Seg<T, XQ> &u1, const uint32_t (&sd0)[T],
                                             const uint32_t (&bd0)[T], const uint32_t (&sd1)[T],
                                             const uint32_t (&bd1)[T], f32x4 (&acc)[T], const Lanes &ln, u32x4 *wt,
                                             Reload &&reload) {
    u32x4 a0[XQ == 2 ? 4 : 1], a1[XQ == 2 ? 4 : 1];
    u32x4 *xs = wt + T * 128;
    if constexpr (XQ == 2) {
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            xs[ln.xw[k]] = act_pairs(u0.x[k]);
            xs[128 + ln.xw[k]] = act_pairs(u1.x[k]);
        }
    }
#pragma unroll
    for (int t = 0; t < T; ++t) {
        wt[t * 128 + ln.wslot[0]] = u0.w[t];
        wt[t * 128 + ln.wslot[1]] = u1.w[t];
    }
    // The activation words of the compact and four-load forms stay in registers.
    u32x4 x0[XQ == 2 ? 1 : 4 / XQ], x1[XQ == 2 ? 1 : 4 / XQ];
    if constexpr (XQ != 2) {
#pragma unroll
        for (int i = 0; i < 4 / XQ; ++i) {
            x0[i] = u0.x[i];
            x1[i] = u1.x[i];
        }
    }
    // The pair's buffers are free: the next loads go out before the arithmetic.
    reload();
    if constexpr (XQ == 2) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            a0[i] = xs[ln.xrd[i]];
            a1[i] = xs[128 + ln.xrd[i]];
        }
    }
    u32x4 w0[T], w1[T];
#pragma unroll
    for (int t = 0; t < T; ++t) {
        w0[t] = wt[t * 128 + ln.rslot[0]];
        w1[t] = wt[t * 128 + ln.rslot[1]];
    }
    compute_seg<T, XQ>(x0, w0, sd0, bd0, acc, a0);
    compute_seg<T, XQ>(x1, w1, sd1, bd1, acc, a1);
}

__device__ __forceinline__ uint32_t dword(const u32x4 &v, int j) {
    return j == 0 ? v.x : j == 1 ? v.y : j == 2 ? v.z : v.w;
}

// LDS partial sums of the K split: two regions (alternating bands) of
// MAXS waves x T tiles x 4 values x 64 lanes.
template <int T, int MAXS = kMfmaMaxS>
struct Red {
    static constexpr int REGION = MAXS * T * 4 * 64;
    static constexpr int FLOATS = 2 * REGION;
};

// Sum the S waves' partials of a finished band and hand them to the output:
// out.put(acc, band, g, nl, mrows, N) on the first wave, whose lane (g, nl)
// holds D[4*g + r][nl] of every tile.
template <int T, int MAXS, typename Out>
__device__ __forceinline__ void finish_band(f32x4 (&acc)[T], float *red, int S, int wig, int lane, int64_t band,
                                            int parity, int64_t N, int mrows, const Out &out) {
    const int g = lane >> 4, nl = lane & 15;
    if (S > 1) {
        float *reg = red + parity * Red<T, MAXS>::REGION;
#pragma unroll
        for (int t = 0; t < T; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r) reg[((wig * T + t) * 4 + r) * 64 + lane] = acc[t][r];
        __syncthreads();
        if (wig == 0) {
#pragma unroll
            for (int t = 0; t < T; ++t)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    float v = 0.f;
                    for (int w = 0; w < S; ++w) v += reg[((w * T + t) * 4 + r) * 64 + lane];
                    acc[t][r] = v;
                }
        }
    }
    if (wig == 0) out.template put<T>(acc, band, g, nl, mrows, N);
#pragma unroll
    for (int t = 0; t < T; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
}

// One pass: activation rows through the x descriptor `xr` (lane offsets in
// `ln`), against the plane's bands rg, rg + groups, ... (BPG of them).
// Every wave of the block walks the same number of segments, so the block
// meets at the same band boundaries.
template <int T, int XQ, typename Out, bool DUAL = false, int MAXS = kMfmaMaxS>
__device__ __forceinline__ void mfma_pass(const MfmaArgs &a, const Band &bd, const Lanes &ln,
                                          __amdgpu_buffer_rsrc_t xr, int mrows, const Out &out, int64_t rg,
                                          int64_t groups, float *red, u32x4 *wt_all) {
    const int lane = threadIdx.x & 63;
    const int wig = wave_id();
    const int S = a.S, SPW = a.SPW;
    const int seg0 = wig * SPW;
    const int turns = a.BPG * (SPW / kRing);  // turns of the ring over the walk
    const int tpb = SPW / kRing;               // turns per band
    // The wave's buffer: 2 KB per tile for line loads, then 4 KB of staged activations (XQ 2).
    u32x4 *wt = wt_all + wig * (T * 128 + (XQ == 2 ? 256 : 0));

    Seg<T, XQ> buf[kRing];
    ScaleBlock<T> next[kRing / kSB], cur;
    f32x4 acc[T];
#pragma unroll
    for (int t = 0; t < T; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    __builtin_amdgcn_sched_barrier(0);

    // Turn j covers segments seg0 + 4*(j % tpb) .. +3 of band rg + (j / tpb) * groups.
#pragma unroll
    for (int p = 0; p < kRing; ++p) {
        if (p % kSB == 0)
            load_seg<T, true, XQ, DUAL>(buf[p], next[p / kSB], bd, ln, xr, rg, seg0 + p);
        else
            load_seg<T, false, XQ, DUAL>(buf[p], next[0], bd, ln, xr, rg, seg0 + p);
    }
    __builtin_amdgcn_sched_barrier(0);

    int j = 0;
    for (; j + 1 < turns; ++j) {
        const int bi = j / tpb;
        const int64_t band = rg + (int64_t)bi * groups;
        const int jn = j + 1;
        const int64_t nband = rg + (int64_t)(jn / tpb) * groups;
        const int nseg = seg0 + kRing * (jn % tpb);
#pragma unroll
        for (int p = 0; p < kRing; p += 2) {
            if (p % kSB == 0) cur = next[p / kSB];
            uint32_t sd0[T], bd0[T], sd1[T], bd1[T];
#pragma unroll
            for (int t = 0; t < T; ++t) {
                sd0[t] = dword(cur.s[t], p % kSB);
                bd0[t] = dword(cur.b[t], p % kSB);
                sd1[t] = dword(cur.s[t], (p + 1) % kSB);
                bd1[t] = dword(cur.b[t], (p + 1) % kSB);
            }
            compute_pair<T, XQ>(buf[p], buf[p + 1], sd0, bd0, sd1, bd1, acc, ln, wt, [&] {
                if (p % kSB == 0)
                    load_seg<T, true, XQ, DUAL>(buf[p], next[p / kSB], bd, ln, xr, nband, nseg + p);
                else
                    load_seg<T, false, XQ, DUAL>(buf[p], next[0], bd, ln, xr, nband, nseg + p);
                load_seg<T, false, XQ, DUAL>(buf[p + 1], next[0], bd, ln, xr, nband, nseg + p + 1);
            });
            __builtin_amdgcn_sched_barrier(0);
        }
        if ((j + 1) % tpb == 0) finish_band<T, MAXS>(acc, red, S, wig, lane, band, bi & 1, bd.N, mrows, out);
    }
    {
        const int bi = j / tpb;
        const int64_t band = rg + (int64_t)bi * groups;
#pragma unroll
        for (int p = 0; p < kRing; p += 2) {
            if (p % kSB == 0) cur = next[p / kSB];
            uint32_t sd0[T], bd0[T], sd1[T], bd1[T];
#pragma unroll
            for (int t = 0; t < T; ++t) {
                sd0[t] = dword(cur.s[t], p % kSB);
                bd0[t] = dword(cur.b[t], p % kSB);
                sd1[t] = dword(cur.s[t], (p + 1) % kSB);
                bd1[t] = dword(cur.b[t], (p + 1) % kSB);
            }
            compute_pair<T, XQ>(buf[p], buf[p + 1], sd0, bd0, sd1, bd1, acc, ln, wt, [] {});
        }
        finish_band<T, MAXS>(acc, red, S, wig, lane, band, bi & 1, bd.N, mrows, out);
    }
    if (S > 1) __syncthreads();  // the LDS regions are reused by the next pass
}

// Lane constants shared by the dense and gather kernels; rowoff(r): byte
// offset of pass row r in x (or the descriptor's end for rows past the pass).
template <int XQ, typename RowOff>
__device__ __forceinline__ Lanes lane_consts(const MfmaArgs &a, RowOff rowoff) {
    const int lane = threadIdx.x & 63;
    const uint32_t g = (uint32_t)lane >> 4, nl = (uint32_t)lane & 15u;
    Lanes ln;
    // Line loads: the lane reads row l/8 (or 8 + l/8), bytes 16*(l%8) of a
    // 128-byte window: segment sg = (l%8)/4, quarter q = l%4. The LDS slot of
    // (row, segment, quarter) is segment*64 + quarter*16 + (row ^ 2*(segment*4 + quarter)).
    {
        const uint32_t l = (uint32_t)lane, sg = (l & 7u) >> 2, q = l & 3u, f = 2u * (sg * 4u + q);
        ln.wlo = (l >> 3) * (uint32_t)(a.K / 2) + 16u * (l & 7u);
        ln.wslot[0] = sg * 64u + q * 16u + ((l >> 3) ^ f);
        ln.wslot[1] = sg * 64u + q * 16u + ((8u + (l >> 3)) ^ f);
        ln.rslot[0] = 0u * 64u + g * 16u + (nl ^ (2u * (0u * 4u + g)));
        ln.rslot[1] = 1u * 64u + g * 16u + (nl ^ (2u * (1u * 4u + g)));
    }
    ln.soff = nl * (uint32_t)a.G * 2u;
    if constexpr (XQ == 2) {
        // Staged: load k reads word nl (columns 8*nl..+7 of the segment) of
        // row 4k + g; LDS slot of (row, word) is row*16 + (word ^ row).
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const uint32_t row = 4u * (uint32_t)k + g;
            ln.xoff[k] = rowoff(row) + 16u * nl;
            ln.xw[k] = row * 16u + (nl ^ row);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t h = (uint32_t)i >> 1, t = (uint32_t)i & 1u, row = nl & 7u;
            const uint32_t word = 8u * h + 4u * (g & 1u) + t + 2u * (g >> 1);
            ln.xrd[i] = row * 16u + (word ^ row);
        }
    } else {
        const uint32_t xrow = rowoff(nl % (16u / XQ));
#pragma unroll
        for (int j = 0; j < 4 / XQ; ++j) {
            const uint32_t i = (nl / (16u / XQ)) * (4u / XQ) + (uint32_t)j;  // slot
            const uint32_t h = i >> 1, t = i & 1u;
            const uint32_t col = 64u * h + 32u * (g & 1u) + 8u * (t + 2u * (g >> 1));
            ln.xoff[j] = xrow + 2u * col;
        }
    }
    return ln;
}

// Stores a finished band as bf16: tile t's row nl of the band is weight row
// band*16*T + 16*t + nl; D row 4*g + r is pass row m, written to row(m) of y.
template <typename Self>
struct StoreRows {
    template <int T>
    __device__ __forceinline__ void put(const f32x4 (&acc)[T], int64_t band, int g, int nl, int mrows,
                                        int64_t N) const {
        const Self &self = static_cast<const Self &>(*this);
#pragma unroll
        for (int t = 0; t < T; ++t) {
            const int64_t n = band * (16 * T) + 16 * t + nl;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = 4 * g + r;
                if (m < mrows && n < N) self(m)[n] = f32_to_bf16(acc[t][r]);
            }
        }
    }
};

struct RowsOut : StoreRows<RowsOut> {
    uint16_t *y;
    int64_t N;
    __device__ RowsOut(uint16_t *y_, int64_t n_) : y(y_), N(n_) {}
    __device__ __forceinline__ uint16_t *operator()(int m) const { return y + (int64_t)m * N; }
};

struct PairsOut : StoreRows<PairsOut> {
    uint16_t *y;
    int64_t N;
    const uint16_t *plist;
    __device__ PairsOut(uint16_t *y_, int64_t n_, const uint16_t *p_) : y(y_), N(n_), plist(p_) {}
    __device__ __forceinline__ uint16_t *operator()(int m) const { return y + (int64_t)plist[m] * N; }
};

// Calls f with the activation load form (XQ) for a gather pass of `rows`
// rows: 4 up to 4 rows, 2 up to 8, else 1. (Dense products choose on the
// host, as separate kernels: one kernel holding two forms made 14336x4096 at
// M = 8 0.5 us slower.) For the gather's few pairs per plane the rotations
// beat staging: Mixtral-shaped W1, 64.5 against 66.3 us with staged passes of
// up to 4 pairs.
template <typename F>
__device__ __forceinline__ void with_xq(int rows, F &&f) {
    if (rows <= 4) {
        f(std::integral_constant<int, 4>{});
        return;
    }
    if (rows <= 8) {
        f(std::integral_constant<int, 2>{});
        return;
    }
    f(std::integral_constant<int, 1>{});
}

}  // namespace mfma
}  // namespace agq
