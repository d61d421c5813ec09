// Affine group-quantized matrix-matrix product (qmm) and its expert-gathered
// form (gather_qmm) on the gfx950 matrix cores: the prefill-side products that
// "epic: CUDA (MLX backend) prefill and decode acceleration program" names in
// its Code-audit findings (qmm / gather_gemm) and whose MoE form carries that
// page's largest measured gap (Diagnosis (baseline), the MoE prefill row).
//
// Same operands as the matvec kernels: BF16 activations x [M, K] (or the x
// rows the gather's pairs select), U32-packed 4- or 8-bit codes (low-first)
// [N, K*bits/32], BF16 scale and bias per 64-column group; y [M, N] BF16.
//
// Exactness. A dequantized weight s*q + b needs up to 24 significant bits, so
// rounding it to bfloat16 for the matrix cores could cost up to 2^-8 of
// sum |x*w| per output. Instead the B operand holds values that bfloat16
// represents exactly, and the scale and bias are applied per group in fp32:
//   4-bit: B = 128 + q (a code in the low mantissa bits of 0x4300),
//          y += s*D + (b - 128*s)*X
//   8-bit: B = q (at most 8 significant bits),
//          y += s*D + b*X
// where D is the group's dot product of x with B (v_mfma_f32_16x16x32_bf16,
// exact products, fp32 sums) and X the group's sum of x (the same A operands
// against an all-ones B).
//
// Tiling. A block of 4 waves (2 x 2) computes a tile of BM = 32*TM activation
// rows by BN = 32*TN weight rows; wave (wm, wn) owns 16*TM x 16*TN of it. K
// advances one 64-column group at a time. Per group the block stages into LDS:
//  - x: BM rows x 8 words of 8 columns (16 bytes each), already in A-operand
//    order (4-bit: the bfloat16 pairs (c0,c4) (c1,c5) (c2,c6) (c3,c7) of each
//    8-column word, matching the code unpack; 8-bit: natural order);
//  - codes: BN rows x 8 words, unpacked to B-operand bfloat16 (each weight is
//    unpacked once per block and read by both waves of its column);
//  - the group's scale and bias of each of the BN rows.
// Word w of a row sits at slot w ^ (row & 7): the 16 lanes of a lane group
// read 16 rows of one word, and the XOR spreads them over all 64 banks.
// Global loads run DEPTH groups ahead in registers; the LDS tiles are double
// buffered, so each group costs one block barrier.
// (Grids of 256-row tiles that fill the device take the split-weight kernels
// below instead.)
//
// Lanes and MFMA operands (16x16x32, bf16): lane l, g = l / 16, i = l % 16.
// A: row i of the 16-row sub-tile, words 4*step + g; B: weight row i of the
// sub-tile, the same words; D: lane holds D[4*g + r][i], r < 4.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "qmm.hpp"
#include "qmv_device.hpp"

namespace agq {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kRsrc = 0x00020000;  // raw buffer, 32-bit data format
constexpr uint32_t kOne2 = 0x3F803F80u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t span(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, (int)bytes, kRsrc);
}

__device__ __forceinline__ f32x4 mma(const u32x4 &a, const u32x4 &b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0,
                                                   0, 0);
}

// A-operand order of one 8-column word of x for 4-bit codes.
__device__ __forceinline__ u32x4 x_pairs(const u32x4 &q) {
    return u32x4{byte_perm(q.z, q.x, 0x05040100u), byte_perm(q.z, q.x, 0x07060302u),
                 byte_perm(q.w, q.y, 0x05040100u), byte_perm(q.w, q.y, 0x07060302u)};
}

// B operand of one packed 4-bit word: bfloat16 (128 + q) pairs (q0,q4) (q1,q5) (q2,q6) (q3,q7).
__device__ __forceinline__ u32x4 codes4(uint32_t w) {
    const uint32_t lo = w & 0x0F0F0F0Fu, hi = (w >> 4) & 0x0F0F0F0Fu;
    return u32x4{byte_perm(kMagic43, lo, kSelEven), byte_perm(kMagic43, hi, kSelEven),
                 byte_perm(kMagic43, lo, kSelOdd), byte_perm(kMagic43, hi, kSelOdd)};
}

// B operand of two packed 8-bit words (8 codes, natural order) as bfloat16 q.
// (float)q has at most 8 significant bits, so its top half is q exactly.
__device__ __forceinline__ uint32_t pair8(float a, float b) {
    return byte_perm(__float_as_uint(b), __float_as_uint(a), 0x07060302u);
}
__device__ __forceinline__ u32x4 codes8(uint32_t w0, uint32_t w1) {
    // (float of a masked byte compiles to v_cvt_f32_ubyte{0..3})
    return u32x4{pair8((float)(w0 & 0xFFu), (float)((w0 >> 8) & 0xFFu)),
                 pair8((float)((w0 >> 16) & 0xFFu), (float)(w0 >> 24)),
                 pair8((float)(w1 & 0xFFu), (float)((w1 >> 8) & 0xFFu)),
                 pair8((float)((w1 >> 16) & 0xFFu), (float)(w1 >> 24))};
}

template <int BITS, int TM, int TN>
struct Tile {
    static constexpr int BM = 32 * TM, BN = 32 * TN;
    static constexpr int THREADS = 256;
    static constexpr int XW = BM * 8;                  // 16-byte x words per group
    static constexpr int XPT = XW / THREADS;           // per thread
    static constexpr int WB = BN * 8 * BITS;           // bytes of codes per group
    static constexpr int WPT = WB / 16 / THREADS;      // 16-byte code loads per thread (BITS * BN / 512)
    static constexpr int WPT1 = WPT > 0 ? WPT : 1;
    static constexpr int WTHREADS = WB / 16;           // threads that load codes
    // LDS per buffer: x words, B words, scale and bias (bf16 each) per weight row.
    static constexpr int LDS_X = XW * 16, LDS_W = BN * 8 * 16, LDS_SB = BN * 4;
    static constexpr int LDS_BUF = LDS_X + LDS_W + LDS_SB;
    // Deferred folding of each group's results (qmm_tile): only small wave
    // tiles have the registers for a second set of results (64x64 tiles stay
    // at 2 waves per SIMD with it; 128x64 tiles would drop to 1).
    static constexpr bool PIPE = TM * TN <= 4;
    static_assert(XW % THREADS == 0, "x tile words must divide among the threads");
    static_assert(WPT > 0 || WTHREADS <= THREADS, "a code tile smaller than the block takes one load per thread");
};

// Registers of one group's global loads.
template <int BITS, int TM, int TN>
struct Stage {
    using TT = Tile<BITS, TM, TN>;
    u32x4 x[TT::XPT];
    u32x4 w[TT::WPT1];
    uint16_t sb;  // the scale (threads < BN) or bias (threads BN .. 2*BN-1) of one weight row
};

// Which x row a tile row reads and which output row it writes.
struct DenseMap {
    int64_t m0;  // first activation row of the tile
    int64_t M;
    __device__ __forceinline__ int64_t xrow(int r) const { return m0 + r < M ? m0 + r : -1; }
    __device__ __forceinline__ int64_t yrow(int r) const { return m0 + r < M ? m0 + r : -1; }
};
struct GatherMap {
    const uint16_t *plist;  // pairs of the tile (LDS)
    const uint32_t *xlist;  // their x rows (LDS)
    int count;              // pairs in the tile
    __device__ __forceinline__ int64_t xrow(int r) const { return r < count ? (int64_t)xlist[r] : -1; }
    __device__ __forceinline__ int64_t yrow(int r) const { return r < count ? (int64_t)plist[r] : -1; }
};

// Global loads of group `grp` for the block's tile. Rows outside the tile
// (x rows past M or the pass, weight rows past N) read zero through the
// buffer ranges; every load is unconditional.
template <int BITS, int TM, int TN, typename Map>
__device__ __forceinline__ void load_group(Stage<BITS, TM, TN> &st, const QmmArgs &a, const Map &map,
                                           __amdgpu_buffer_rsrc_t xr, __amdgpu_buffer_rsrc_t wr,
                                           __amdgpu_buffer_rsrc_t sr, __amdgpu_buffer_rsrc_t br, int grp,
                                           uint32_t xbytes) {
    using TT = Tile<BITS, TM, TN>;
    const int t = threadIdx.x;
#pragma unroll
    for (int k = 0; k < TT::XPT; ++k) {
        const int idx = t + k * TT::THREADS;  // x word: row idx / 8, word idx % 8
        const int64_t row = map.xrow(idx >> 3);
        const uint32_t off = row >= 0 ? (uint32_t)(row * a.K + grp * 64 + (idx & 7) * 8) * 2u : xbytes;
        st.x[k] = __builtin_amdgcn_raw_buffer_load_b128(xr, off, 0, 0);
    }
    // Codes: weight row n = t / (BITS/2), 16-byte piece t % (BITS/2) of the row's 32*BITS/8... bytes
    // (4-bit: 32 bytes per row per group, two threads; 8-bit: 64 bytes, four threads).
    constexpr int PPR = BITS / 2;  // 16-byte pieces per row per group
#pragma unroll
    for (int k = 0; k < TT::WPT1; ++k) {
        const int idx = t + k * TT::THREADS;
        const uint32_t row = (uint32_t)(idx / PPR), piece = (uint32_t)(idx % PPR);
        const uint32_t off = row * (uint32_t)a.rowbytes + (uint32_t)grp * (uint32_t)(8 * BITS) + piece * 16u;
        st.w[k] = (TT::WPT > 0 || t < TT::WTHREADS) ? __builtin_amdgcn_raw_buffer_load_b128(wr, off, 0, 2)
                                                    : u32x4{0u, 0u, 0u, 0u};
    }
    if (t < 2 * TT::BN) {
        const uint32_t row = (uint32_t)(t % TT::BN);
        const uint32_t off = (row * (uint32_t)a.G + (uint32_t)grp) * 2u;
        st.sb = t < TT::BN ? __builtin_amdgcn_raw_buffer_load_b16(sr, off, 0, 0)
                           : __builtin_amdgcn_raw_buffer_load_b16(br, off, 0, 0);
    }
}

template <int BITS, int TM, int TN>
__device__ __forceinline__ void store_group(const Stage<BITS, TM, TN> &st, uint8_t *buf) {
    using TT = Tile<BITS, TM, TN>;
    u32x4 *xs = reinterpret_cast<u32x4 *>(buf);
    u32x4 *ws = reinterpret_cast<u32x4 *>(buf + TT::LDS_X);
    uint16_t *sb = reinterpret_cast<uint16_t *>(buf + TT::LDS_X + TT::LDS_W);
    const int t = threadIdx.x;
#pragma unroll
    for (int k = 0; k < TT::XPT; ++k) {
        const int idx = t + k * TT::THREADS;
        const int row = idx >> 3, word = idx & 7;
        xs[row * 8 + (word ^ (row & 7))] = BITS == 4 ? x_pairs(st.x[k]) : st.x[k];
    }
    constexpr int PPR = BITS / 2;
#pragma unroll
    for (int k = 0; k < TT::WPT1; ++k) {
        const int idx = t + k * TT::THREADS;
        if (TT::WPT > 0 || t < TT::WTHREADS) {
            const int row = idx / PPR, piece = idx % PPR;
            const u32x4 v = st.w[k];
            if constexpr (BITS == 4) {
                // 4 words = 4 B-operand words (8 columns each): words 4*piece .. +3
                const uint32_t d[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int word = 4 * piece + i;
                    ws[row * 8 + (word ^ (row & 7))] = codes4(d[i]);
                }
            } else {
                // 4 words = 2 B-operand words: words 2*piece, 2*piece + 1
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    const int word = 2 * piece + i;
                    ws[row * 8 + (word ^ (row & 7))] = codes8(i == 0 ? v.x : v.z, i == 0 ? v.y : v.w);
                }
            }
        }
    }
    if (t < 2 * TT::BN) sb[t] = st.sb;  // scales [0, BN), biases [BN, 2*BN)
}

// One group's matrix-core products on the wave's 16*TM x 16*TN sub-tiles,
// with the scale and the bias term of each weight row read out of LDS, so the
// fp32 epilogue can run a group later (after the next group's MFMAs are in
// flight), when the LDS buffer may already hold another group.
template <int TM, int TN>
struct GroupSums {
    f32x4 d[TM][TN], xsum[TM];
    float s[TN], c[TN];
};

template <int BITS, int TM, int TN>
__device__ __forceinline__ void mfma_group(const uint8_t *buf, int wm, int wn, GroupSums<TM, TN> &gs) {
    using TT = Tile<BITS, TM, TN>;
    const u32x4 *xs = reinterpret_cast<const u32x4 *>(buf);
    const u32x4 *ws = reinterpret_cast<const u32x4 *>(buf + TT::LDS_X);
    const uint16_t *sb = reinterpret_cast<const uint16_t *>(buf + TT::LDS_X + TT::LDS_W);
    const int lane = threadIdx.x & 63, g = lane >> 4, i = lane & 15;
    const f32x4 z = {0.f, 0.f, 0.f, 0.f};
    const u32x4 ones = {kOne2, kOne2, kOne2, kOne2};
#pragma unroll
    for (int n = 0; n < TN; ++n) {
        const int row = wn * 16 * TN + 16 * n + i;
        const float sv = bf16_lo(sb[row]), bv = bf16_lo(sb[TT::BN + row]);
        gs.s[n] = sv;
        gs.c[n] = BITS == 4 ? fmaf(-128.f, sv, bv) : bv;
    }
#pragma unroll
    for (int step = 0; step < 2; ++step) {
        const int word = 4 * step + g;
        u32x4 av[TM], bv[TN];
#pragma unroll
        for (int m = 0; m < TM; ++m) {
            const int row = wm * 16 * TM + 16 * m + i;
            av[m] = xs[row * 8 + (word ^ (row & 7))];
        }
#pragma unroll
        for (int n = 0; n < TN; ++n) {
            const int row = wn * 16 * TN + 16 * n + i;
            bv[n] = ws[row * 8 + (word ^ (row & 7))];
        }
#pragma unroll
        for (int m = 0; m < TM; ++m) {
            gs.xsum[m] = mma(av[m], ones, step == 0 ? z : gs.xsum[m]);
#pragma unroll
            for (int n = 0; n < TN; ++n) gs.d[m][n] = mma(av[m], bv[n], step == 0 ? z : gs.d[m][n]);
        }
    }
}

// acc += s * D + c * X for one group.
template <int TM, int TN>
__device__ __forceinline__ void fold_group(const GroupSums<TM, TN> &gs, f32x4 (&acc)[TM][TN]) {
#pragma unroll
    for (int n = 0; n < TN; ++n)
#pragma unroll
        for (int m = 0; m < TM; ++m)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                acc[m][n][r] = fmaf(gs.s[n], gs.d[m][n][r], fmaf(gs.c[n], gs.xsum[m][r], acc[m][n][r]));
}

// The tile rows [.., BM) of `map` against weight rows [n0, n0 + BN) of one plane.
template <int BITS, int TM, int TN, int DEPTH, bool PIPE, typename Map>
__device__ __forceinline__ void qmm_tile(const QmmArgs &a, const Map &map, const uint32_t *w, const uint16_t *s,
                                         const uint16_t *b, int64_t n0, uint8_t *lds) {
    using TT = Tile<BITS, TM, TN>;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    const int lane = threadIdx.x & 63, g = lane >> 4, i = lane & 15;
    const int64_t nrows = a.N - n0 < TT::BN ? a.N - n0 : TT::BN;
    const uint32_t xbytes = a.xbytes;
    const __amdgpu_buffer_rsrc_t xr = span(a.x, xbytes);
    const __amdgpu_buffer_rsrc_t wr = span(w + n0 * (a.rowbytes / 4), (uint32_t)(nrows * a.rowbytes));
    const __amdgpu_buffer_rsrc_t sr = span(s + n0 * a.G, (uint32_t)(nrows * a.G * 2));
    const __amdgpu_buffer_rsrc_t br = span(b + n0 * a.G, (uint32_t)(nrows * a.G * 2));

    f32x4 acc[TM][TN];
#pragma unroll
    for (int m = 0; m < TM; ++m)
#pragma unroll
        for (int n = 0; n < TN; ++n) acc[m][n] = f32x4{0.f, 0.f, 0.f, 0.f};

    Stage<BITS, TM, TN> st[DEPTH];
#pragma unroll
    for (int p = 0; p < DEPTH; ++p)
        load_group<BITS, TM, TN>(st[p], a, map, xr, wr, sr, br, p < a.G ? p : a.G - 1, xbytes);
    store_group<BITS, TM, TN>(st[0], lds);
    __syncthreads();
    // Group grp computes from LDS buffer grp & 1 while the loads of grp + DEPTH
    // go out into the register stage grp just freed. With PIPE its MFMA results
    // are folded into acc one group later, after the next group's MFMAs are
    // issued, so their latency overlaps that work (at the cost of a second set
    // of result registers).
    static_assert(DEPTH % 2 == 0, "the pending results alternate between two slots");
    GroupSums<TM, TN> gsum[2];
    for (int grp0 = 0; grp0 < a.G; grp0 += DEPTH) {
#pragma unroll
        for (int p = 0; p < DEPTH; ++p) {
            const int grp = grp0 + p;
            if (grp < a.G) {  // uniform
                mfma_group<BITS, TM, TN>(lds + (grp & 1) * TT::LDS_BUF, wm, wn, gsum[p & 1]);
                if constexpr (PIPE) {
                    if (grp > 0) fold_group<TM, TN>(gsum[(p + 1) & 1], acc);
                } else {
                    fold_group<TM, TN>(gsum[p & 1], acc);
                }
                if (grp + 1 < a.G) store_group<BITS, TM, TN>(st[(p + 1) % DEPTH], lds + ((grp + 1) & 1) * TT::LDS_BUF);
                const int nxt = grp + DEPTH;
                load_group<BITS, TM, TN>(st[p], a, map, xr, wr, sr, br, nxt < a.G ? nxt : a.G - 1, xbytes);
                __syncthreads();
            }
        }
    }
    // The last group's results (slot (G - 1) & 1; constant indices keep gsum in registers).
    if constexpr (PIPE) {
        if ((a.G - 1) & 1)
            fold_group<TM, TN>(gsum[1], acc);
        else
            fold_group<TM, TN>(gsum[0], acc);
    }
    // Store: lane holds rows 4g + r of sub-tile m, weight row i of sub-tile n.
#pragma unroll
    for (int m = 0; m < TM; ++m)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int64_t yr = map.yrow(wm * 16 * TM + 16 * m + 4 * g + r);
            if (yr < 0) continue;
#pragma unroll
            for (int n = 0; n < TN; ++n) {
                const int64_t col = wn * 16 * TN + 16 * n + i;
                if (col < nrows) a.y[yr * a.N + n0 + col] = f32_to_bf16(acc[m][n][r]);
            }
        }
}

// ---------------------------------------------------------------------------
// Large tiles: the dequantized weight split into two bfloat16 parts.
//
// Where a grid of large tiles fills the device, the per-group fp32 correction
// above costs more issue time than the matrix cores spend on the group. These
// kernels take the weight itself to the matrix cores instead: each weight is
// dequantized once per block, w = fma(s, q, b) in fp32 (the value
// agq_dequantize writes), and split into w = hi + lo with hi = bf16(w) and
// lo = bf16(w - hi). Both parts go to the B operand, so every 16x16x32 product
// runs twice (hi, lo) and accumulates across all of K in the same registers:
// no per-group fold and no sums of x. hi + lo holds 16 significant bits of w,
// all of them whenever w needs at most 16 (every weight of the quantizer's
// recipe needs at most 12 at 4 bits and 16 at 8 bits); otherwise the weight
// is off by at most 2^-17 of itself. Infinite weights give NaN (lo = inf - inf).
//
// A block of 8 waves computes BM = 32*TMW activation rows by 128 weight rows,
// one 64-column group at a time, through two LDS buffers (x: BM rows x 8
// words of 8 columns in natural order; the weights' hi and lo parts: 128 rows
// x 8 words each; word w of a row at slot w ^ (row & 7)). Waves 0-3 (2 x 2,
// 16*TMW x 64 each) only take products out of one buffer; waves 4-7 stage the
// next group into the other: x with direct-to-LDS buffer loads, and the codes
// (loaded two groups ahead) dequantized and split, 32 columns of one weight row
// per thread. One block barrier per group; one wave of each role per SIMD, so
// staging overlaps the matrix-core work (4096x4096 at M = 2048: 136 us with all
// four waves doing both in turn, 107 us with the roles split).
// (hi, lo) bfloat16 pairs of the fp32 pair (v0, v1): hi = bf16(v), lo = bf16(v - hi).
__device__ __forceinline__ void hl_split(float v0, float v1, uint32_t &hp, uint32_t &lp) {
    const f32x2 v = {v0, v1};
    hp = __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
    const f32x2 l = {v0 - __uint_as_float(hp << 16), v1 - __uint_as_float(hp & 0xFFFF0000u)};
    lp = __builtin_bit_cast(uint32_t, __builtin_convertvector(l, bf16x2));
}

// Weight formats of the split-weight tiles: what one producer thread loads per
// group (32 columns of one weight row, two groups ahead) and the B parts it
// writes for them.
//  - Affine codes (4- or 8-bit, BF16 scale and bias per 64 columns): two
//    parts, hi = bf16(w) and lo = bf16(w - hi) of w = fma(s, q, b).
//  - NVFP4 (E2M1 codes, one E4M3 scale byte per 16 columns): one part,
//    bf16(e2m1(q) * e4m3(s)), exact (at most 6 significant bits); the fp32
//    tensor scale multiplies each result once, before its bf16 rounding.
template <int BITS>
struct AffineFmt {
    static constexpr int kParts = 2;
    static constexpr int kLoads = BITS / 4 + 2;  // vector-memory instructions of one load
    static constexpr bool kScaled = false;
    struct Stage {
        u32x4 w[BITS / 4];  // the thread's 32 codes (4-bit: 16 bytes; 8-bit: 32 bytes)
        uint16_t s, b;
    };
    __device__ static __amdgpu_buffer_rsrc_t srange(const QmmArgs &a, const uint16_t *s, int64_t n0, int64_t nrows) {
        return span(s + n0 * a.G, (uint32_t)(nrows * a.G * 2));
    }
    __device__ static __amdgpu_buffer_rsrc_t brange(const QmmArgs &a, const uint16_t *b, int64_t n0, int64_t nrows) {
        return span(b + n0 * a.G, (uint32_t)(nrows * a.G * 2));
    }
    // Weight row t / 2, columns 32 * (t % 2) .. +32 of group grp.
    __device__ static void load(Stage &st, const QmmArgs &a, __amdgpu_buffer_rsrc_t wr, __amdgpu_buffer_rsrc_t sr,
                                __amdgpu_buffer_rsrc_t br, int grp, int t) {
        const uint32_t r = (uint32_t)t >> 1, h = (uint32_t)t & 1u;
#pragma unroll
        for (int c = 0; c < BITS / 4; ++c) {
            const uint32_t off = r * (uint32_t)a.rowbytes + (uint32_t)grp * (uint32_t)(8 * BITS) +
                                 h * (uint32_t)(4 * BITS) + (uint32_t)c * 16u;
            st.w[c] = __builtin_amdgcn_raw_buffer_load_b128(wr, off, 0, 2);
        }
        const uint32_t soff = (r * (uint32_t)a.G + (uint32_t)grp) * 2u;
        st.s = __builtin_amdgcn_raw_buffer_load_b16(sr, soff, 0, 0);
        st.b = __builtin_amdgcn_raw_buffer_load_b16(br, soff, 0, 0);
    }
    // The thread's four B words (8 columns each) of both parts.
    __device__ static void store(const Stage &st, u32x4 *p0, u32x4 *p1, int t) {
        const float sf = bf16_lo(st.s), bfv = bf16_lo(st.b);
        const int r = t >> 1, h = t & 1;
        const uint32_t d[8] = {st.w[0].x, st.w[0].y, st.w[0].z, st.w[0].w,
                               BITS == 8 ? st.w[BITS / 4 - 1].x : 0u, BITS == 8 ? st.w[BITS / 4 - 1].y : 0u,
                               BITS == 8 ? st.w[BITS / 4 - 1].z : 0u, BITS == 8 ? st.w[BITS / 4 - 1].w : 0u};
#pragma unroll
        for (int j = 0; j < 4; ++j) {  // B word 4h + j: columns 8j .. 8j + 7 of the thread's 32
            float v[8];
            if constexpr (BITS == 4) {
                // codes low-first: byte i of the word holds columns 2i (low nibble) and 2i + 1
                const uint32_t lo = d[j] & 0x0F0F0F0Fu, hi = (d[j] >> 4) & 0x0F0F0F0Fu;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    v[2 * i] = fmaf(sf, (float)((lo >> (8 * i)) & 0xFFu), bfv);
                    v[2 * i + 1] = fmaf(sf, (float)((hi >> (8 * i)) & 0xFFu), bfv);
                }
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    v[i] = fmaf(sf, (float)((d[2 * j] >> (8 * i)) & 0xFFu), bfv);
                    v[4 + i] = fmaf(sf, (float)((d[2 * j + 1] >> (8 * i)) & 0xFFu), bfv);
                }
            }
            uint32_t hp[4], lp[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) hl_split(v[2 * q], v[2 * q + 1], hp[q], lp[q]);
            const int word = 4 * h + j;
            p0[r * 8 + (word ^ (r & 7))] = u32x4{hp[0], hp[1], hp[2], hp[3]};
            p1[r * 8 + (word ^ (r & 7))] = u32x4{lp[0], lp[1], lp[2], lp[3]};
        }
    }
};

struct Nvfp4Fmt {
    static constexpr int kParts = 1;
    static constexpr int kLoads = 2;
    static constexpr bool kScaled = true;
    struct Stage {
        u32x4 w;     // the thread's 32 codes
        uint16_t s;  // their two E4M3 scale bytes
    };
    // (a.s points at the scale bytes, [N, K/16] uint8; there is no bias.)
    __device__ static __amdgpu_buffer_rsrc_t srange(const QmmArgs &a, const uint16_t *s, int64_t n0, int64_t nrows) {
        return span(reinterpret_cast<const uint8_t *>(s) + n0 * (a.K / 16), (uint32_t)(nrows * (a.K / 16)));
    }
    __device__ static __amdgpu_buffer_rsrc_t brange(const QmmArgs &, const uint16_t *, int64_t, int64_t) {
        return span(nullptr, 0u);
    }
    __device__ static void load(Stage &st, const QmmArgs &a, __amdgpu_buffer_rsrc_t wr, __amdgpu_buffer_rsrc_t sr,
                                __amdgpu_buffer_rsrc_t, int grp, int t) {
        const uint32_t r = (uint32_t)t >> 1, h = (uint32_t)t & 1u;
        st.w = __builtin_amdgcn_raw_buffer_load_b128(wr, r * (uint32_t)a.rowbytes + (uint32_t)grp * 32u + h * 16u, 0, 2);
        st.s = __builtin_amdgcn_raw_buffer_load_b16(sr, r * (uint32_t)(a.K / 16) + (uint32_t)grp * 4u + h * 2u, 0, 0);
    }
    // Words 0-1 of the thread's 32 codes take scale byte 0, words 2-3 byte 1.
    // The FP4 convert turns byte p of a word into the bf16 pair (column 2p,
    // column 2p + 1), exactly (scale operand 1: it applies only an exponent).
    __device__ static void store(const Stage &st, u32x4 *p0, u32x4 *, int t) {
        const int r = t >> 1, h = t & 1;
        const float sc[2] = {__builtin_amdgcn_cvt_f32_fp8((uint32_t)st.s, 0),
                             __builtin_amdgcn_cvt_f32_fp8((uint32_t)st.s, 1)};
        const uint32_t d[4] = {st.w.x, st.w.y, st.w.z, st.w.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t pr[4] = {
                __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d[j], 1.0f, 0)),
                __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d[j], 1.0f, 1)),
                __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d[j], 1.0f, 2)),
                __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d[j], 1.0f, 3))};
            const float f = sc[j >> 1];
            uint32_t o[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const f32x2 v = {__uint_as_float(pr[q] << 16) * f, __uint_as_float(pr[q] & 0xFFFF0000u) * f};
                o[q] = __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
            }
            const int word = 4 * h + j;
            p0[r * 8 + (word ^ (r & 7))] = u32x4{o[0], o[1], o[2], o[3]};
        }
    }
};

template <typename F, int TMW>
struct Hl {
    static constexpr int BM = 32 * TMW, BN = 128;
    static constexpr int LDS_X = BM * 128, LDS_B = BN * 128;
    static constexpr int LDS_BUF = LDS_X + F::kParts * LDS_B;
};

// x of group grp into the LDS buffer's x tile with direct-to-LDS loads: wave w
// writes 1 KB chunks c = w, w + 4, ... (rows 8c .. 8c + 7); lane L of a chunk
// fills slot L % 8 of row 8c + L / 8, so it fetches that row's word
// (L % 8) ^ (L / 8). Rows past the tile (or the pass) read zero.
template <int BM, typename Map>
__device__ __forceinline__ void hl_load_x(const QmmArgs &a, const Map &map, __amdgpu_buffer_rsrc_t xr, int grp,
                                          uint8_t *buf, int wave) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int k = 0; k < BM / 32; ++k) {
        const int c = wave + 4 * k;
        const int row = 8 * c + (lane >> 3);
        const int word = (lane & 7) ^ (lane >> 3);
        const int64_t xrow = map.xrow(row);
        const uint32_t off = xrow >= 0 ? (uint32_t)(xrow * a.K + grp * 64 + word * 8) * 2u : a.xbytes;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            xr, (__attribute__((address_space(3))) void *)(buf + c * 1024), 16, off, 0, 0, 0);
    }
}

// One group's products: for each of the two 32-column steps, the wave's TMW x 4
// sub-tiles take each part of the weights (hi, then lo) into their accumulators.
template <typename F, int TMW>
__device__ __forceinline__ void hl_compute(const uint8_t *buf, int wm, int wn, f32x4 (&acc)[TMW][4]) {
    using H = Hl<F, TMW>;
    const u32x4 *xs = reinterpret_cast<const u32x4 *>(buf);
    const int lane = threadIdx.x & 63, g = lane >> 4, i = lane & 15;
#pragma unroll
    for (int step = 0; step < 2; ++step) {
        const int word = 4 * step + g;
        u32x4 av[TMW], bv[F::kParts][4];
#pragma unroll
        for (int m = 0; m < TMW; ++m) {
            const int row = wm * 16 * TMW + 16 * m + i;
            av[m] = xs[row * 8 + (word ^ (row & 7))];
        }
#pragma unroll
        for (int q = 0; q < F::kParts; ++q) {
            const u32x4 *bs = reinterpret_cast<const u32x4 *>(buf + H::LDS_X + q * H::LDS_B);
#pragma unroll
            for (int n = 0; n < 4; ++n) {
                const int row = wn * 64 + 16 * n + i;
                bv[q][n] = bs[row * 8 + (word ^ (row & 7))];
            }
        }
        // Part by part: each accumulator's next product issues TMW*4 instructions later.
#pragma unroll
        for (int q = 0; q < F::kParts; ++q)
#pragma unroll
            for (int m = 0; m < TMW; ++m)
#pragma unroll
                for (int n = 0; n < 4; ++n) acc[m][n] = mma(av[m], bv[q][n], acc[m][n]);
    }
}

// Groups g0 .. g1 - 1 of the tile (all of K, or one K split); with a.part
// the fp32 results go to split blockIdx.z's plane of the partials.
template <typename F, int TMW, typename Map>
__device__ __forceinline__ void hl_tile(const QmmArgs &a, const Map &map, const uint32_t *w, const uint16_t *s,
                                        const uint16_t *b, int64_t n0, uint8_t *lds, int g0, int g1) {
    using H = Hl<F, TMW>;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63, g = lane >> 4, i = lane & 15;
    const int64_t nrows = a.N - n0 < H::BN ? a.N - n0 : H::BN;
    const int last = g1 - 1;
    // Two roles, one wave of each per SIMD: waves 4-7 stage group grp + 1 into LDS
    // buffer (grp + 1) % 2 (x with direct-to-LDS loads, the weights dequantized
    // into their B parts) while waves 0-3 take group grp's products out of buffer
    // grp % 2. One block barrier per group; both roles meet it the same number of times.
    if (wave >= 4) {
        const int pw = wave - 4, t = threadIdx.x - 256;
        const __amdgpu_buffer_rsrc_t xr = span(a.x, a.xbytes);
        const __amdgpu_buffer_rsrc_t wr = span(w + n0 * (a.rowbytes / 4), (uint32_t)(nrows * a.rowbytes));
        const __amdgpu_buffer_rsrc_t sr = F::srange(a, s, n0, nrows);
        const __amdgpu_buffer_rsrc_t br = F::brange(a, b, n0, nrows);
        // The B parts of an LDS buffer follow its x tile.
        auto part = [&](uint8_t *buf, int q) { return reinterpret_cast<u32x4 *>(buf + H::LDS_X + q * H::LDS_B); };
        // The register stage holds the codes of the next group to stage; its
        // reload goes out right after, so each load has a group's products to arrive.
        typename F::Stage st;
        hl_load_x<H::BM>(a, map, xr, g0, lds, pw);
        F::load(st, a, wr, sr, br, g0, t);
        F::store(st, part(lds, 0), part(lds, F::kParts - 1), t);
        F::load(st, a, wr, sr, br, last < g0 + 1 ? last : g0 + 1, t);
        __builtin_amdgcn_s_waitcnt(0x0F70 | F::kLoads);  // vmcnt(loads of st): x has landed
        __syncthreads();
        for (int grp = g0; grp < g1; ++grp) {
            if (grp + 1 < g1) {  // uniform
                uint8_t *nb = lds + ((grp + 1 - g0) & 1) * H::LDS_BUF;
                hl_load_x<H::BM>(a, map, xr, grp + 1, nb, pw);
                F::store(st, part(nb, 0), part(nb, F::kParts - 1), t);
                F::load(st, a, wr, sr, br, grp + 2 < last ? grp + 2 : last, t);
                __builtin_amdgcn_s_waitcnt(0x0F70 | F::kLoads);  // the staged x has landed
            }
            __syncthreads();
        }
        return;
    }
    const int wm = wave >> 1, wn = wave & 1;
    f32x4 acc[TMW][4];
#pragma unroll
    for (int m = 0; m < TMW; ++m)
#pragma unroll
        for (int n = 0; n < 4; ++n) acc[m][n] = f32x4{0.f, 0.f, 0.f, 0.f};
    __syncthreads();
    for (int grp = g0; grp < g1; ++grp) {
        hl_compute<F, TMW>(lds + ((grp - g0) & 1) * H::LDS_BUF, wm, wn, acc);
        __syncthreads();
    }
    // Store: lane holds rows 4g + r of sub-tile m, weight row i of sub-tile n.
    float *pp = a.part ? a.part + (int64_t)blockIdx.z * a.M * a.N : nullptr;
#pragma unroll
    for (int m = 0; m < TMW; ++m)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int64_t yr = map.yrow(wm * 16 * TMW + 16 * m + 4 * g + r);
            if (yr < 0) continue;
#pragma unroll
            for (int n = 0; n < 4; ++n) {
                const int64_t col = wn * 64 + 16 * n + i;
                if (col >= nrows) continue;
                if (pp) {
                    pp[yr * a.N + n0 + col] = acc[m][n][r];
                } else {
                    const float v = F::kScaled ? acc[m][n][r] * a.ts : acc[m][n][r];
                    a.y[yr * a.N + n0 + col] = f32_to_bf16(v);
                }
            }
        }
}

}  // namespace

// Dense: blockIdx.x = weight-row tile, blockIdx.y = activation-row tile.
template <int BITS, int TM, int TN, int DEPTH>
__global__ __launch_bounds__(256) void qmm_kernel(QmmArgs a) {
    extern __shared__ __attribute__((aligned(16))) uint8_t qmm_lds[];
    using TT = Tile<BITS, TM, TN>;
    const DenseMap map{(int64_t)blockIdx.y * TT::BM, a.M};
    qmm_tile<BITS, TM, TN, DEPTH, TT::PIPE>(a, map, a.w, a.s, a.b, (int64_t)blockIdx.x * TT::BN, qmm_lds);
}

// Split-weight tiles, dense: blockIdx.x = 128-row weight tile, blockIdx.y =
// activation-row tile, blockIdx.z = K split (groups z*gps .. of it); F: the
// weight format.
template <typename F, int TMW>
__global__ __launch_bounds__(512) void qmm_hl_kernel(QmmArgs a) {
    extern __shared__ __attribute__((aligned(16))) uint8_t qmm_lds[];
    const DenseMap map{(int64_t)blockIdx.y * Hl<F, TMW>::BM, a.M};
    const int g0 = (int)blockIdx.z * a.gps;
    const int g1 = a.G - g0 < a.gps ? a.G : g0 + a.gps;
    hl_tile<F, TMW>(a, map, a.w, a.s, a.b, (int64_t)blockIdx.x * Hl<F, TMW>::BN, qmm_lds, g0, g1);
}

// The K splits' partials [splits, M, N] (MN = M * N) summed in split order,
// times ts, rounded to bf16 into y [M, N]; four outputs per thread.
__global__ __launch_bounds__(256) void qmm_reduce(const float *part, uint16_t *y, int64_t MN, int splits, float ts) {
    const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
    if (i >= MN) return;
    if (MN % 4 == 0) {  // uniform: every plane starts 16-byte aligned
        f32x4 v = *reinterpret_cast<const f32x4 *>(part + i);
        for (int z = 1; z < splits; ++z) v += *reinterpret_cast<const f32x4 *>(part + (int64_t)z * MN + i);
#pragma unroll
        for (int k = 0; k < 4; ++k) y[i + k] = f32_to_bf16(v[k] * ts);
        return;
    }
    for (int k = 0; k < 4 && i + k < MN; ++k) {
        float v = part[i + k];
        for (int z = 1; z < splits; ++z) v += part[(int64_t)z * MN + i + k];
        y[i + k] = f32_to_bf16(v * ts);
    }
}

const void *qmm_reduce_kernel() { return reinterpret_cast<const void *>(&qmm_reduce); }

namespace {

// The gather's pair lists for plane blockIdx.y, in ascending p: plist holds the
// pairs routed to the plane with an in-range x row, xlist their x rows; the
// return value is their count. Blocks of plane 0 first write NaN over columns
// [n0, n0 + bn) of the rows of pairs whose indices are out of range. NT: threads
// of the block (wave_counts holds NT / 64 counts).
template <int NT>
__device__ __forceinline__ int gather_pairs(const QmmArgs &a, uint16_t *plist, uint32_t *xlist, int *wave_counts,
                                            int64_t n0, int bn) {
    const int t = threadIdx.x, lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const uint32_t e = blockIdx.y;
    const uint32_t nx = (uint32_t)a.R_x, ne = (uint32_t)a.E;

    // Block-wide ordered compaction of the pairs p < P that satisfy pred into plist.
    auto compact = [&](auto pred) {
        int total = 0;
        for (int base = 0; base < a.M; base += NT) {
            const int p = base + t;
            const bool take = p < a.M && pred(p);
            const uint64_t mask = __ballot(take);
            if (lane == 0) wave_counts[wave] = __popcll(mask);
            __syncthreads();
            int before = total;
            for (int v = 0; v < wave; ++v) before += wave_counts[v];
            if (take) plist[before + __popcll(mask & ((1ull << lane) - 1ull))] = (uint16_t)p;
#pragma unroll
            for (int v = 0; v < NT / 64; ++v) total += wave_counts[v];
            __syncthreads();
        }
        return total;
    };
    if (e == 0) {
        const int nbad = compact([&](int p) {
            const uint32_t xr = a.lhs ? a.lhs[p] : (uint32_t)p;
            const uint32_t ex = a.rhs ? a.rhs[p] : (uint32_t)p;
            return xr >= nx || ex >= ne;
        });
        for (int k = 0; k < nbad; ++k)
            for (int c = t; c < bn; c += NT)
                if (n0 + c < a.N) a.y[(int64_t)plist[k] * a.N + n0 + c] = 0x7FC0u;
        __syncthreads();
    }
    const int count = compact([&](int p) {
        const uint32_t xr = a.lhs ? a.lhs[p] : (uint32_t)p;
        const uint32_t ex = a.rhs ? a.rhs[p] : (uint32_t)p;
        return ex == e && xr < nx;
    });
    for (int k = t; k < count; k += NT) xlist[k] = a.lhs ? a.lhs[plist[k]] : (uint32_t)plist[k];
    __syncthreads();
    return count;
}

}  // namespace

// Gather: blockIdx.x = weight-row tile, blockIdx.y = expert plane e. The
// block lists the pairs routed to e (ascending p) and walks them BM at a
// time. Blocks of plane 0 also write NaN rows for pairs whose indices are out
// of range. LDS after the tile buffers: pair list (uint16) and x rows (uint32).
template <int BITS, int TM, int TN, int DEPTH>
__global__ __launch_bounds__(256) void gather_qmm_kernel(QmmArgs a) {
    extern __shared__ __attribute__((aligned(16))) uint8_t qmm_lds[];
    using TT = Tile<BITS, TM, TN>;
    uint16_t *plist = reinterpret_cast<uint16_t *>(qmm_lds + 2 * TT::LDS_BUF);
    uint32_t *xlist = reinterpret_cast<uint32_t *>(qmm_lds + 2 * TT::LDS_BUF + ((a.M * 2 + 15) / 16) * 16);
    __shared__ int wave_counts[4];
    const int64_t n0 = (int64_t)blockIdx.x * TT::BN;
    const int count = gather_pairs<256>(a, plist, xlist, wave_counts, n0, TT::BN);
    if (count == 0) return;
    const int64_t plane = (int64_t)blockIdx.y * a.N;
    const uint32_t *w = a.w + plane * (a.rowbytes / 4);
    const uint16_t *s = a.s + plane * a.G, *b = a.b + plane * a.G;
    for (int base = 0; base < count; base += TT::BM) {
        const GatherMap map{plist + base, xlist + base, count - base < TT::BM ? count - base : TT::BM};
        qmm_tile<BITS, TM, TN, DEPTH, TT::PIPE>(a, map, w, s, b, n0, qmm_lds);
        __syncthreads();  // the LDS tiles are refilled by the next pass
    }
}

// Large tiles, gathered (as gather_qmm_kernel).
template <int BITS, int TMW>
__global__ __launch_bounds__(512) void gather_qmm_hl_kernel(QmmArgs a) {
    extern __shared__ __attribute__((aligned(16))) uint8_t qmm_lds[];
    using H = Hl<AffineFmt<BITS>, TMW>;
    uint16_t *plist = reinterpret_cast<uint16_t *>(qmm_lds + 2 * H::LDS_BUF);
    uint32_t *xlist = reinterpret_cast<uint32_t *>(qmm_lds + 2 * H::LDS_BUF + ((a.M * 2 + 15) / 16) * 16);
    __shared__ int wave_counts[8];
    const int64_t n0 = (int64_t)blockIdx.x * H::BN;
    const int count = gather_pairs<512>(a, plist, xlist, wave_counts, n0, H::BN);
    if (count == 0) return;
    const int64_t plane = (int64_t)blockIdx.y * a.N;
    const uint32_t *w = a.w + plane * (a.rowbytes / 4);
    const uint16_t *s = a.s + plane * a.G, *b = a.b + plane * a.G;
    for (int base = 0; base < count; base += H::BM) {
        const GatherMap map{plist + base, xlist + base, count - base < H::BM ? count - base : H::BM};
        hl_tile<AffineFmt<BITS>, TMW>(a, map, w, s, b, n0, qmm_lds, 0, a.G);
        __syncthreads();  // the LDS tiles are refilled by the next pass
    }
}

// ---------------------------------------------------------------------------
// Kernel selection.

template <int BITS, int TM, int TN, int D>
static QmmKernel qmm_pick(bool gather) {
    QmmKernel k;
    k.sym = gather ? reinterpret_cast<const void *>(&gather_qmm_kernel<BITS, TM, TN, D>)
                   : reinterpret_cast<const void *>(&qmm_kernel<BITS, TM, TN, D>);
    k.bm = Tile<BITS, TM, TN>::BM;
    k.bn = Tile<BITS, TM, TN>::BN;
    k.lds = 2 * Tile<BITS, TM, TN>::LDS_BUF;
    return k;
}

// (GATHER a template argument: only the instantiations a call can reach are compiled.)
template <int BITS, int TMW, bool GATHER>
static QmmKernel hl_pick() {
    QmmKernel k;
    using H = Hl<AffineFmt<BITS>, TMW>;
    if constexpr (GATHER)
        k.sym = reinterpret_cast<const void *>(&gather_qmm_hl_kernel<BITS, TMW>);
    else
        k.sym = reinterpret_cast<const void *>(&qmm_hl_kernel<AffineFmt<BITS>, TMW>);
    k.bm = H::BM;
    k.bn = H::BN;
    k.lds = 2 * H::LDS_BUF;
    k.threads = 512;
    k.split_weight = true;
    return k;
}

// K splits for a grid of `tiles` split-weight tiles over G groups: as many as
// fit one block per compute unit, each of at least kQmmSplitMinGroups groups;
// none (k unchanged) unless the split grid gives 3/4 of the compute units a block.
static bool split_k(QmmKernel &k, int64_t tiles, int64_t G, int cus) {
    int64_t s = cus / tiles;
    if (s > G / kQmmSplitMinGroups) s = G / kQmmSplitMinGroups;
    if (s < 2 || 4 * tiles * s < 3 * (int64_t)cus) return false;
    k.gps = (int)((G + s - 1) / s);
    k.splits = (int)((G + k.gps - 1) / k.gps);
    return true;
}

QmmKernel qmm_kernel_for(int bits, bool gather, int64_t rows, int64_t N, int64_t K, int64_t planes, int cus,
                         bool split_ok) {
    static_assert(Tile<4, 2, 2>::BN == kQmmTileN && Tile<4, 4, 2>::BN == kQmmTileN && Tile<4, 2, 2>::BM == kQmmTileMinM,
                  "the host checks assume these tile sizes");
    static_assert(Hl<AffineFmt<4>, 8>::BN == kQmmHlTileN && Hl<AffineFmt<4>, 8>::BM >= kQmmTileMinM,
                  "the host checks assume these tile sizes");
    // Split-weight tiles where the rows fill them (dense: more than
    // kQmmHlSplitMinRows; 64-row tiles from kQmmHlSmallMinRows) and their
    // grid, or (dense, with a workspace) their grid split along K, gives every
    // compute unit a block.
    constexpr int HBM = Hl<AffineFmt<4>, 8>::BM;
    if (!gather && rows > kQmmHlSmallMinRows && rows <= kQmmHlSplitMinRows) {
        static_assert(Hl<AffineFmt<4>, 2>::BM == kQmmHlSplitMinRows, "one row of 64-row tiles");
        const int64_t tiles = planes * ((N + kQmmHlTileN - 1) / kQmmHlTileN);
        QmmKernel k = bits == 4 ? hl_pick<4, 2, false>() : hl_pick<8, 2, false>();
        const bool narrow = rows <= kQmmHlSmallNarrowRows;
        if (4 * tiles >= 3 * (int64_t)cus) {
            if (!narrow) return k;
        } else if (split_ok && split_k(k, tiles, K / 64, cus) && (!narrow || k.splits >= kQmmHlSmallMinSplits)) {
            return k;
        }
    }
    if (rows >= kQmmHlMinRows || (!gather && rows > kQmmHlSplitMinRows)) {
        const int64_t tiles = planes * ((N + kQmmHlTileN - 1) / kQmmHlTileN) * ((rows + HBM - 1) / HBM);
        QmmKernel k = gather ? (bits == 4 ? hl_pick<4, 8, true>() : hl_pick<8, 8, true>())
                             : (bits == 4 ? hl_pick<4, 8, false>() : hl_pick<8, 8, false>());
        if (4 * tiles >= 3 * (int64_t)cus) return k;
        if (!gather && split_ok && split_k(k, tiles, K / 64, cus)) return k;
    }
    constexpr int LBM = Tile<4, 4, 2>::BM;
    const int64_t large_blocks = planes * ((rows + LBM - 1) / LBM) * ((N + kQmmTileN - 1) / kQmmTileN);
    const bool small = rows <= (gather ? kQmmSmallPairs : kQmmSmallM) ||
                       large_blocks < (int64_t)kQmmLargeBlocksPerCu * cus;
    if (bits == 4) return small ? qmm_pick<4, 2, 2, 4>(gather) : qmm_pick<4, 4, 2, 2>(gather);
    return small ? qmm_pick<8, 2, 2, 4>(gather) : qmm_pick<8, 4, 2, 2>(gather);
}

// The NVFP4 GEMM for M activation rows: 256-row tiles where their grid, or
// (with a workspace) their grid split along K, gives every compute unit a
// block; 64-row tiles (split along K where that fills the device) otherwise.
QmmKernel qmm_nvfp4_kernel_for(int64_t M, int64_t N, int64_t K, int cus, bool split_ok) {
    using HL = Hl<Nvfp4Fmt, 8>;
    using HS = Hl<Nvfp4Fmt, 2>;
    static_assert(HL::BN == kQmmHlTileN && HS::BN == kQmmHlTileN && HS::BM >= kQmmTileMinM,
                  "the host checks assume these tile sizes");
    QmmKernel k;
    k.bn = HL::BN;
    k.threads = 512;
    const int64_t nt = (N + HL::BN - 1) / HL::BN;
    if (M >= kQmmHlMinRows) {
        k.sym = reinterpret_cast<const void *>(&qmm_hl_kernel<Nvfp4Fmt, 8>);
        k.bm = HL::BM;
        k.lds = 2 * HL::LDS_BUF;
        const int64_t tiles = nt * ((M + HL::BM - 1) / HL::BM);
        if (4 * tiles >= 3 * (int64_t)cus || (split_ok && split_k(k, tiles, K / 64, cus))) return k;
        k.splits = 1;
        k.gps = 0;
    }
    k.sym = reinterpret_cast<const void *>(&qmm_hl_kernel<Nvfp4Fmt, 2>);
    k.bm = HS::BM;
    k.lds = 2 * HS::LDS_BUF;
    const int64_t tiles = nt * ((M + HS::BM - 1) / HS::BM);
    if (4 * tiles < 3 * (int64_t)cus && split_ok) split_k(k, tiles, K / 64, cus);
    return k;
}

}  // namespace agq
