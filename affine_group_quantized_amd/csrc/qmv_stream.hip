// Affine group-quantized products for the bit-stream widths: 2-, 3-, 5- and
// 6-bit codes with group size 64, the other widths of the affine family that
// "MLX CUDA Cleanup Plan" (Target Architecture §1; Refactor Plan, Phase 3)
// names at 4 and 8 bits; and the batch-1 4-bit products whose grid gives
// every compute unit at least two blocks. A row's codes form one low-first
// bit stream over its uint32 words: code k occupies stream bits
// bits*k .. bits*k + bits - 1, word i holding bits 32i .. 32i + 31 (for 2 and
// 4 bits exactly the packed layout; a 3-, 5- or 6-bit code may run into the
// next word). A 64-column group is then exactly 2*bits words (16 to 48 bytes).
//
//     y[m, n] = sum_k x[m, k] * (s[n, g] * q[n, k] + b[n, g]),  g = k / 64
//             = sum_g s[n, g] * D[m, n, g] + (b[n, g] - 128 s[n, g]) * X[m, g],
//     D = sum_{k in g} x[m, k] * (128 + q[n, k]),  X = sum_{k in g} x[m, k]
// (the regrouping of the 4-bit VALU products), with the constant 128 replaced
// by a per-code constant under the window decode below.
//
// Layout of the work: lane l of a wave takes group l of a 64-group chunk of K,
// each wave 4 weight rows, a block 4 waves (16 rows; the K-split form: 8 rows,
// two waves per row set alternating chunks). Per chunk the block stages x (up
// to 8 rows) in LDS as 16-byte pieces [row][piece][group] with direct-to-LDS
// loads, so the 64 lanes read 64 consecutive pieces (no bank conflicts).
// Codes become bf16 lanes exactly (a code below 128 in the low mantissa bits
// of a bf16 with a fixed exponent), and v_dot2c_f32_bf16 takes each lane pair
// against the matching pair of activations:
//   - with one or two activation rows at 2, 3, 4 and 5 bits, the window
//     decode: codes k and k + d share a 32-bit window of the stream and one
//     and-or makes the pair (plan below);
//   - otherwise adjacent codes (2i, 2i + 1) are taken from one funnel-shifted
//     word and moved into the two bf16 lanes.
// With one or two activation rows the wave's weight rows also pass through
// LDS (loads of contiguous 16-byte pieces; a lane reading its own 24- to
// 48-byte group directly spreads each load over 2-3 times the cache lines),
// and the fetches run a step ahead of the arithmetic. The expert gather runs
// each plane's pairs as activation rows. The wave sums come from the DPP /
// permlane tree of the VALU products.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <utility>

#include "qmv_device.hpp"

namespace agq {

namespace {

constexpr int kRpw = 4;    // weight rows per wave
constexpr int kWaves = 4;  // waves per block
static_assert(kRpw * kWaves == kStreamRowsPerBlock, "rows per block");

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t span(const void *p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), 0, (int)bytes, 0x00020000);
}

// Block barrier over LDS only (a __syncthreads() fence would also wait for the
// weight loads in flight).
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// s_waitcnt: at most N vector memory operations outstanding (other counters free).
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
    asm volatile("" ::: "memory");
}

// Code j of a run of NW words holding a bit stream of BITS-bit codes.
template <int BITS, int NW>
__device__ __forceinline__ uint32_t stream_code(const uint32_t (&w)[NW], int j) {
    const int first = BITS * j, word = first >> 5, shift = first & 31;
    uint32_t v;
    if (shift + BITS <= 32)
        v = w[word] >> shift;
    else
        v = __builtin_amdgcn_alignbit(w[word + 1], w[word], (uint32_t)shift);
    return v & ((1u << BITS) - 1u);
}

// Codes 2i and 2i + 1 of a run of NW stream words as the bfloat16 pair
// (128 + q_2i, 128 + q_2i+1): both codes sit in the 32 bits from stream bit
// 2*BITS*i (one word, or a funnel shift across two).
template <int BITS, int NW>
__device__ __forceinline__ uint32_t code_pair_bf16(const uint32_t (&w)[NW], int i) {
    const int first = 2 * BITS * i, word = first >> 5, shift = first & 31;
    uint32_t t;
    if (shift + 2 * BITS <= 32)
        t = shift ? w[word] >> shift : w[word];
    else
        t = __builtin_amdgcn_alignbit(w[word + 1], w[word], (uint32_t)shift);
    constexpr uint32_t mask = (1u << BITS) - 1u;
    return ((t << (16 - BITS)) & (mask << 16)) | (t & mask) | 0x43004300u;
}

// ---- Pair plans of the one- and two-row forms (window decode at 2, 3, 4, 5 bits) ----
//
// A bfloat16 with exponent field 134 - e and a code q in mantissa bits
// [e, e + bits) reads as the exact value 2^(7-e) + q (for e + bits <= 7). So a
// code whose stream bits fall inside mantissa bits 0..6 of either half of a
// 32-bit window of the stream becomes a bf16 lane with one v_and_or_b32:
// (window & mask) | magic, the magic holding each half's exponent. Codes k and
// k + d with d = 8, 4, 5, 3 (2, 4, 3, 5 bits) lie 16, 16, 15 and 15 stream bits apart,
// so both fit one window, one in each half, and at 2 and 3 bits successive
// pairs share windows. The group's 64 codes become 32 such pairs; at 3 and 5
// bits the last four codes (which have no partner d further on) are taken as
// adjacent pairs by code_pair_bf16. Against each pair the activations go as
// the matching pair (x[k], x[k + d]), built by one byte permute, and
//     sum_k q_k x_k = D - C,  D = sum over pairs of dot(code pair, x pair),
//                             C = sum over pairs of dot(magic pair, x pair),
// with C shared by the wave's rows. At 6 bits a code fills all but one
// mantissa bit and no two codes lie 15..17 bits apart, so the 6-bit plan is
// 32 adjacent pairs. Three or more activation rows keep the adjacent pairs
// (the per-row C and pair permutes would cost what the window saves).

struct WinSlot {
    int lo, hi;      // the two codes (group positions): low and high bf16 lane
    int p;           // window start (stream bit; -1 means the word shifted left by one)
    bool win;        // false: adjacent pair (lo, lo + 1) by code_pair_bf16
    uint32_t mask;   // code bits of the window
    uint32_t magic;  // the two lanes' exponents; as bf16 values 2^(7-e_lo), 2^(7-e_hi)
    int mi;          // index of magic among the plan's distinct magics
    uint32_t sel;    // byte permute building (x[lo], x[hi]) from the natural x pairs
};

constexpr int kMaxMagics = 4;

template <int BITS>
struct WinPlan {
    WinSlot s[32];
    uint32_t magics[kMaxMagics];
    int n_magics;
    bool even[kMaxMagics];  // both lanes of the magic hold the same value c
    float c[kMaxMagics];    // that value, 2^(7-e)
};

template <int BITS>
constexpr WinPlan<BITS> make_win_plan() {
    WinPlan<BITS> pl{};
    constexpr int d = BITS == 2 ? 8 : BITS == 3 ? 5 : BITS == 4 ? 4 : BITS == 5 ? 3 : 0;  // 0: adjacent pairs only
    constexpr int room = 7 - BITS;  // largest code offset inside a mantissa
    constexpr uint32_t cm = (1u << BITS) - 1u;
    int n = 0, b0 = 0;
    for (; d > 0 && b0 + 2 * d <= 64; b0 += 2 * d) {
        int p = 0;
        bool have = false;
        for (int i = 0; i < d; ++i) {
            const int lo = b0 + i, hi = lo + d;
            const int olo = BITS * lo, ohi = BITS * hi - 16;  // high code's offset from the window's bit 16
            const int pmax = olo < ohi ? olo : ohi;
            const int pmin = (olo > ohi ? olo : ohi) - room;
            if (!have || p < pmin || p > pmax) p = pmax;  // reuse the previous window where it fits
            have = true;
            const int elo = olo - p, ehi = ohi - p;
            WinSlot &s = pl.s[n++];
            s.lo = lo;
            s.hi = hi;
            s.p = p;
            s.win = true;
            s.mask = (cm << elo) | (cm << (16 + ehi));
            s.magic = (uint32_t(134 - ehi) << 23) | (uint32_t(134 - elo) << 7);
            const uint32_t a = 2u * (uint32_t)(lo & 1), b = 4u + 2u * (uint32_t)(hi & 1);
            s.sel = a | (a + 1u) << 8 | b << 16 | (b + 1u) << 24;
        }
    }
    for (int k = b0; k < 64; k += 2) {
        WinSlot &s = pl.s[n++];
        s.lo = k;
        s.hi = k + 1;
        s.p = 0;
        s.win = false;
        s.mask = 0;
        s.magic = 0x43004300u;
        s.sel = 0;
    }
    for (int i = 0; i < 32; ++i) {
        WinSlot &s = pl.s[i];
        s.mi = -1;
        for (int j = 0; j < pl.n_magics; ++j)
            if (pl.magics[j] == s.magic) s.mi = j;
        if (s.mi < 0 && pl.n_magics < kMaxMagics) {
            s.mi = pl.n_magics;
            pl.magics[pl.n_magics++] = s.magic;
        }
    }
    for (int j = 0; j < pl.n_magics; ++j) {
        const uint32_t lo = pl.magics[j] & 0xFFFFu, hi = pl.magics[j] >> 16;
        pl.even[j] = lo == hi;
        float c = 1.f;
        for (int e = 127; e < (int)(lo >> 7); ++e) c *= 2.f;  // lo is exponent << 7, mantissa 0
        pl.c[j] = c;
    }
    return pl;
}

// Every code of the group decoded exactly once, inside the window and inside
// a mantissa.
template <int BITS>
constexpr bool win_plan_ok() {
    constexpr WinPlan<BITS> pl = make_win_plan<BITS>();
    int seen[64] = {};
    for (int i = 0; i < 32; ++i) {
        const WinSlot &s = pl.s[i];
        if (s.lo < 0 || s.hi >= 64) return false;
        ++seen[s.lo];
        ++seen[s.hi];
        if (!s.win) {
            if (s.hi != s.lo + 1 || (s.lo & 1)) return false;
            continue;
        }
        const int elo = BITS * s.lo - s.p, ehi = BITS * s.hi - 16 - s.p;
        if (elo < 0 || ehi < 0 || elo + BITS > 7 || ehi + BITS > 7 || s.p < -1) return false;
    }
    for (int k = 0; k < 64; ++k)
        if (seen[k] != 1) return false;
    for (int i = 0; i < 32; ++i)
        if (pl.s[i].mi < 0 || pl.magics[pl.s[i].mi] != pl.s[i].magic) return false;
    for (int j = 0; j < pl.n_magics; ++j)
        if ((pl.magics[j] & 0x807Fu) != 0 || (pl.even[j] && pl.c[j] * 2.f > 256.f)) return false;
    return true;
}
static_assert(win_plan_ok<2>() && win_plan_ok<3>() && win_plan_ok<4>() && win_plan_ok<5>() && win_plan_ok<6>(),
              "window plans");

template <int BITS>
constexpr WinPlan<BITS> kWinPlan = make_win_plan<BITS>();

// Stream bits [P, P + 32) of a group's NW words (zeros outside the group).
template <int P, int NW>
__device__ __forceinline__ uint32_t window(const uint32_t (&w)[NW]) {
    if constexpr (P < 0) {
        return w[0] << (-P);
    } else {
        constexpr int word = P >> 5, sh = P & 31;
        if constexpr (sh == 0)
            return w[word];
        else if constexpr (word + 1 < NW)
            return __builtin_amdgcn_alignbit(w[word + 1], w[word], (uint32_t)sh);
        else
            return w[word] >> sh;
    }
}

// (a & mask) | magic with the magic held in a VGPR: a VOP3 operation takes no
// literal here, and as two VOP2 operations it costs two instructions.
__device__ __forceinline__ uint32_t and_or(uint32_t a, uint32_t mask, uint32_t magic) {
    uint32_t r;
    asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "s"(mask), "v"(magic));
    return r;
}

// A constant in a VGPR the compiler does not fold back into literals.
__device__ __forceinline__ uint32_t vgpr_const(uint32_t c) {
    uint32_t r;
    asm volatile("v_mov_b32 %0, %1" : "=v"(r) : "s"(c));
    return r;
}

// s_waitcnt vmcnt(0) after two rows' accumulators are final: the operands keep
// it below the arithmetic that produces them (a bare wait can be scheduled
// above independent arithmetic, which would stall on loads meant to overlap it).
template <int MW>
__device__ __forceinline__ void wait_vm_after(const float (&a0)[MW], const float (&a1)[MW]) {
    static_assert(MW == 1 || MW == 2, "one or two activation rows");
    if constexpr (MW == 1)
        asm volatile("s_waitcnt vmcnt(0)" ::"v"(a0[0]), "v"(a1[0]) : "memory");
    else
        asm volatile("s_waitcnt vmcnt(0)" ::"v"(a0[0]), "v"(a0[1]), "v"(a1[0]), "v"(a1[1]) : "memory");
}

template <class F, int... I>
__device__ __forceinline__ void static_for_impl(F &f, std::integer_sequence<int, I...>) {
    (f(std::integral_constant<int, I>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F &&f) {
    static_for_impl(f, std::make_integer_sequence<int, N>{});
}


// The 2*BITS words of group g of a row: 16-byte loads where groups are 16-byte
// aligned (2 and 6 bits), 8-byte loads otherwise (3 and 5 bits). Past the
// row's range (its end, or a row past N) the words read zero. Only a 16-byte
// group (2 bits) fills whole lines per load instruction; wider groups spread
// every instruction over all lines of the wave's span, so those loads keep
// the default cache policy (non-temporal lines were fetched again).
template <int BITS>
__device__ __forceinline__ void load_group(uint32_t (&w)[2 * BITS], __amdgpu_buffer_rsrc_t r, uint32_t off) {
    if constexpr (BITS % 2 == 0) {
#pragma unroll
        for (int i = 0; i < BITS / 2; ++i) {
            const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, off + 16u * i, 0, BITS == 2 ? 2 : 0);
            w[4 * i] = v.x;
            w[4 * i + 1] = v.y;
            w[4 * i + 2] = v.z;
            w[4 * i + 3] = v.w;
        }
    } else {
#pragma unroll
        for (int i = 0; i < BITS; ++i) {
            const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, off + 8u * i, 0, 0);
            w[2 * i] = v.x;
            w[2 * i + 1] = v.y;
        }
    }
}

}  // namespace

// The kernel body; KS = 1 for qmv_stream_kernel (the products and the gather),
// KS = 2 for qmv_stream_split_kernel.
template <int BITS, int MW, bool GATHER, int KS, bool FP4 = false>
__device__ __forceinline__ void stream_body(StreamArgs a) {
    // FP4: the NVFP4 product (E2M1 codes in the 4-bit layout; s holds one E4M3
    // byte per 16 columns, four per 64-column group; no biases; y scaled by the
    // tensor scale ts before its rounding).
    static_assert(!FP4 || (BITS == 4 && MW == 1 && !GATHER && KS == 1), "NVFP4: one row, no gather or split");
    // One or two activation rows (the decode forms): the weight rows go through
    // LDS. A lane's own group is a 16- to 48-byte run, and lanes reading their
    // runs directly touch up to 2-3 times the cache lines of a contiguous read
    // per load instruction (the address unit then bounds the kernel). Instead
    // each wave brings its rows' chunk in with direct-to-LDS loads of 16
    // contiguous bytes per lane, two rows at a time, and each lane reads its
    // group back from LDS. The fetches run one step ahead of the arithmetic:
    // the second pair of rows arrives while the first is computed, and the
    // next chunk's x and first pair while the second is.
    constexpr bool kStaged = MW <= 2;
    constexpr int kGroupBytes = 8 * BITS;
    constexpr int kDmaPerRow = (64 * kGroupBytes + 1023) / 1024;
    constexpr int kRows = 2;  // staged weight rows resident at a time
    static_assert(kRpw == 2 * kRows, "two pairs of rows per wave");
    // KS = 2 (short grids with several chunks of K): waves 2i and 2i + 1 take
    // the same 4 rows and alternate chunks of K (a block then covers 8 rows),
    // and their sums meet in LDS at the end; so twice the blocks, and half the
    // chunks in each wave's chain.
    static_assert(KS == 1 || (KS == 2 && kStaged && !GATHER), "K split: the staged plain products");
    __shared__ u32x4 xs[KS * MW * 8 * 64];  // [chunk of the step][row][piece of 8 columns][group]
    __shared__ u32x4 wl[kStaged ? kWaves * kRows * kDmaPerRow * 64 : 1];  // [wave][row][1 KB piece]
    const int lane = threadIdx.x & 63, wave = wave_id();
    const int kh = KS > 1 ? wave % KS : 0;  // the wave's chunk within each step of KS chunks
    const int64_t row0 = ((int64_t)blockIdx.x * (kWaves / KS) + wave / KS) * kRpw;
    const int G = a.K / 64;
    const uint32_t rowbytes = (uint32_t)a.K / 8u * BITS;
    // The expert gather: grid row y is expert plane e. The pairs routed to e
    // (rhs[p] == e with lhs[p] < R) are listed in LDS and taken as the
    // activation rows, up to MW per pass, so each used plane streams once per
    // pass of MW pairs and an unused plane is never read. Pairs with an index
    // out of range get NaN rows, written by the plane-0 blocks. a.M holds P.
    __shared__ uint16_t plist[GATHER ? kMaxGatherPairs : 1];
    __shared__ int pcount;
    int count = a.M;
    if constexpr (GATHER) {
        const uint32_t e = blockIdx.y, nx = (uint32_t)a.R_x, ne = (uint32_t)a.E;
        const int P = a.M;
        if (e == 0)
            for (int p = threadIdx.x; p < P; p += blockDim.x) {
                const uint32_t xr = a.lhs ? a.lhs[p] : (uint32_t)p, ex = a.rhs ? a.rhs[p] : (uint32_t)p;
                if (xr < nx && ex < ne) continue;
                for (int r = 0; r < kStreamRowsPerBlock; ++r) {
                    const int64_t n = (int64_t)blockIdx.x * kStreamRowsPerBlock + r;
                    if (n < a.N) a.y[(int64_t)p * a.N + n] = 0x7FC0u;
                }
            }
        if (wave == 0) {
            int c = 0;
            for (int b0 = 0; b0 < P; b0 += 64) {
                const int p = b0 + lane;
                bool take = false;
                if (p < P) {
                    const uint32_t xr = a.lhs ? a.lhs[p] : (uint32_t)p, ex = a.rhs ? a.rhs[p] : (uint32_t)p;
                    take = ex == e && xr < nx;
                }
                const uint64_t bal = __ballot(take);
                if (take) plist[c + __popcll(bal & ((uint64_t(1) << lane) - 1))] = (uint16_t)p;
                c += __popcll(bal);
            }
            if (lane == 0) pcount = c;
        }
        __syncthreads();
        count = pcount;
        if (count == 0) return;  // the whole block: no barrier follows
        a.w += (int64_t)e * a.N * (a.K / 32 * BITS);
        a.s += (int64_t)e * a.N * (a.K / 64);
        a.b += (int64_t)e * a.N * (a.K / 64);
    }
    // Pass over activation rows [base, base + MW): x row and output row of
    // row m of the pass.
    // (One pass outside the gather, known at compile time.)
    const int passes = GATHER ? (count + MW - 1) / MW : 1;
    for (int pass = 0; pass < passes; ++pass) {
    const int base = pass * MW;
    const int mrows = GATHER ? (count - base < MW ? count - base : MW) : a.M;
    auto x_row = [&](int m) -> int64_t {
        if constexpr (GATHER) {
            const uint32_t p = __builtin_amdgcn_readfirstlane(plist[base + m]);
            return a.lhs ? (int64_t)a.lhs[p] : (int64_t)p;
        } else {
            return m;
        }
    };
    auto y_row = [&](int m) -> int64_t {
        if constexpr (GATHER)
            return plist[base + m];
        else
            return m;
    };
    float acc[kRpw][MW];
#pragma unroll
    for (int r = 0; r < kRpw; ++r)
#pragma unroll
        for (int m = 0; m < MW; ++m) acc[r][m] = 0.f;

    // x of chunk c0 with direct-to-LDS loads: instruction (m, j8) brings piece
    // j8 of every group of row m, lane g landing at slot g of [m][j8][.]. Rows
    // past M and columns past K read zero (each row's range is its own K
    // columns). The 4 waves take every fourth (m, j8).
    auto x_dma = [&](int c0) {
        for (int q = wave; q < KS * MW * 8; q += kWaves) {
            const int kk = q / (MW * 8), m = (q % (MW * 8)) >> 3, j8 = q & 7;
            const __amdgpu_buffer_rsrc_t xr = span(a.x + (m < mrows ? x_row(m) : 0) * a.K, m < mrows ? (uint32_t)a.K * 2u : 0u);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                xr, (__attribute__((address_space(3))) void *)(xs + q * 64),
                16, ((uint32_t)(c0 + 64 * kk + lane) * 64u + 8u * (uint32_t)j8) * 2u, 0, 0, 0);
        }
    };
    // Scale and bias of group c0 + lane of row r (zero past the row's groups and
    // for rows past N), and the row's code buffer.
    auto row_rsrc = [&](int r, int c0, uint32_t &s_out, uint32_t &b_out) {
        const int64_t row = row0 + r;
        const bool ok = row < a.N;
        const int64_t ro = ok ? row : 0;
        if constexpr (FP4) {  // the group's four scale bytes
            const uint8_t *s8 = reinterpret_cast<const uint8_t *>(a.s);
            s_out = __builtin_amdgcn_raw_buffer_load_b32(span(s8 + ro * G * 4, ok ? (uint32_t)G * 4u : 0u),
                                                         (uint32_t)(c0 + lane) * 4u, 0, 0);
            b_out = 0u;
        } else {
            const uint32_t sb = ok ? (uint32_t)G * 2u : 0u;
            s_out = __builtin_amdgcn_raw_buffer_load_b16(span(a.s + ro * G, sb), (uint32_t)(c0 + lane) * 2u, 0, 0);
            b_out = __builtin_amdgcn_raw_buffer_load_b16(span(a.b + ro * G, sb), (uint32_t)(c0 + lane) * 2u, 0, 0);
        }
        return span(a.w + ro * (rowbytes / 4u), ok ? rowbytes : 0u);
    };

    if constexpr (kStaged) {
        uint32_t magic_v[kMaxMagics];
#pragma unroll
        for (int j = 0; j < kWinPlan<BITS>.n_magics; ++j) magic_v[j] = vgpr_const(kWinPlan<BITS>.magics[j]);
        uint32_t sc[kRpw], bi[kRpw];
        // Rows 2h, 2h + 1 of chunk c0 into the wave's LDS rows (piece i of row rr
        // holds the row's chunk bytes [1024 i, 1024 i + 1024); past the row's
        // end, zeros), with their scales and biases.
        auto issue = [&](int h, int c0) {
            const int cw = c0 + 64 * kh;  // the wave's chunk of the step (past K: zeros)
#pragma unroll
            for (int rr = 0; rr < kRows; ++rr) {
                const __amdgpu_buffer_rsrc_t wr = row_rsrc(h * kRows + rr, cw, sc[h * kRows + rr], bi[h * kRows + rr]);
#pragma unroll
                for (int i = 0; i < kDmaPerRow; ++i)
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(
                        wr, (__attribute__((address_space(3))) void *)(wl + ((wave * kRows + rr) * kDmaPerRow + i) * 64),
                        16, (uint32_t)cw * kGroupBytes + (uint32_t)(i * 64 + lane) * 16u, 0, 0, 2);
            }
        };
        uint32_t w[kRows][2 * BITS];
        // A lane's group of each staged row, then the rows are free for the
        // next loads.
        auto read_rows = [&]() {
#pragma unroll
            for (int rr = 0; rr < kRows; ++rr) {
                const u32x4 *base = wl + (wave * kRows + rr) * kDmaPerRow * 64;
                if constexpr (BITS % 2 == 0) {
#pragma unroll
                    for (int i = 0; i < BITS / 2; ++i) {
                        const u32x4 v = base[lane * (BITS / 2) + i];
                        w[rr][4 * i] = v.x;
                        w[rr][4 * i + 1] = v.y;
                        w[rr][4 * i + 2] = v.z;
                        w[rr][4 * i + 3] = v.w;
                    }
                } else {
                    const u32x2 *b2 = reinterpret_cast<const u32x2 *>(base);
#pragma unroll
                    for (int i = 0; i < BITS; ++i) {
                        const u32x2 v = b2[lane * BITS + i];
                        w[rr][2 * i] = v.x;
                        w[rr][2 * i + 1] = v.y;
                    }
                }
            }
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        };

        x_dma(0);
        issue(0, 0);
        for (int c0 = 0; c0 < G; c0 += 64 * KS) {
            // This chunk's x (every wave's pieces) and this wave's first pair of
            // rows have landed. Tied to the last rows' sums so that no wait is
            // hoisted above the previous chunk's arithmetic.
            wait_vm_after<MW>(acc[2], acc[3]);
            lds_barrier();
            // The plan's 32 activation pairs of the lane's group per activation
            // row, with X and C. Where a magic's two lanes are equal (c, c), its
            // slots' x sums S_j give both: X += S_j, C += c S_j.
            uint32_t xp[32][MW];
            float sx[MW], cx[MW];
#pragma unroll
            for (int m = 0; m < MW; ++m) {
                uint32_t xn[32];
#pragma unroll
                for (int j8 = 0; j8 < 8; ++j8) {
                    const u32x4 v = xs[((kh * MW + m) * 8 + j8) * 64 + lane];
                    xn[4 * j8] = v.x;
                    xn[4 * j8 + 1] = v.y;
                    xn[4 * j8 + 2] = v.z;
                    xn[4 * j8 + 3] = v.w;
                }
                sx[m] = 0.f;
                cx[m] = 0.f;
                if constexpr (FP4) {  // natural pairs: the FP4 convert gives codes (2i, 2i + 1)
#pragma unroll
                    for (int i = 0; i < 32; ++i) xp[i][m] = xn[i];
                    continue;
                }
                float sj[kMaxMagics];
#pragma unroll
                for (int j = 0; j < kMaxMagics; ++j) sj[j] = 0.f;
                static_for<32>([&](auto I) {
                    constexpr WinSlot sl = kWinPlan<BITS>.s[decltype(I)::value];
                    uint32_t v;
                    if constexpr (sl.win)
                        v = __builtin_amdgcn_perm(xn[sl.hi >> 1], xn[sl.lo >> 1], sl.sel);
                    else
                        v = xn[sl.lo >> 1];
                    xp[decltype(I)::value][m] = v;
                    if constexpr (kWinPlan<BITS>.even[sl.mi]) {
                        sj[sl.mi] = dot2_bf16(v, 0x3F803F80u, sj[sl.mi]);
                    } else {
                        sx[m] = dot2_bf16(v, 0x3F803F80u, sx[m]);
                        cx[m] = dot2_bf16(v, sl.magic, cx[m]);
                    }
                });
#pragma unroll
                for (int j = 0; j < kWinPlan<BITS>.n_magics; ++j)
                    if (kWinPlan<BITS>.even[j]) {
                        sx[m] += sj[j];
                        cx[m] = fmaf(kWinPlan<BITS>.c[j], sj[j], cx[m]);
                    }
            }
            // Every wave holds the chunk's x: the next chunk's pieces may land.
            lds_barrier();
            const bool more = c0 + 64 * KS < G;
            if (more) x_dma(c0 + 64 * KS);
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                // The second pair (and the next chunk's x) after the first pair
                // is done.
                if (h == 1) wait_vm_after<MW>(acc[0], acc[1]);
                read_rows();
                if (h == 0)
                    issue(1, c0);
                else if (more)
                    issue(0, c0 + 64 * KS);
                if constexpr (FP4) {
                    // Per 16-column block j (words 2j, 2j + 1): the dot of its 8 code
                    // pairs with x, scaled by the block's E4M3 byte.
#pragma unroll
                    for (int rr = 0; rr < kRows; ++rr) {
                        const int r = h * kRows + rr;
                        static_for<4>([&](auto J) {
                            constexpr int j = decltype(J)::value;
                            float dj = 0.f;
#pragma unroll
                            for (int u = 0; u < 2; ++u) {
                                const uint32_t wd = w[rr][2 * j + u];
                                const int i0 = 4 * (2 * j + u);
                                dj = dot2_bf16(__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd, 1.0f, 0)), xp[i0][0], dj);
                                dj = dot2_bf16(__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd, 1.0f, 1)), xp[i0 + 1][0], dj);
                                dj = dot2_bf16(__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd, 1.0f, 2)), xp[i0 + 2][0], dj);
                                dj = dot2_bf16(__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wd, 1.0f, 3)), xp[i0 + 3][0], dj);
                            }
                            acc[r][0] = fmaf(__builtin_amdgcn_cvt_f32_fp8(sc[r], j), dj, acc[r][0]);
                        });
                    }
                    continue;
                }
                float d[kRows][MW];
#pragma unroll
                for (int rr = 0; rr < kRows; ++rr)
#pragma unroll
                    for (int m = 0; m < MW; ++m) d[rr][m] = 0.f;
                static_for<32>([&](auto I) {
                    constexpr WinSlot sl = kWinPlan<BITS>.s[decltype(I)::value];
#pragma unroll
                    for (int rr = 0; rr < kRows; ++rr) {
                        uint32_t cp;
                        if constexpr (sl.win)
                            cp = and_or(window<sl.p>(w[rr]), sl.mask, magic_v[sl.mi]);
                        else
                            cp = code_pair_bf16<BITS>(w[rr], sl.lo >> 1);
#pragma unroll
                        for (int m = 0; m < MW; ++m) d[rr][m] = dot2_bf16(xp[decltype(I)::value][m], cp, d[rr][m]);
                    }
                });
#pragma unroll
                for (int rr = 0; rr < kRows; ++rr) {
                    const int r = h * kRows + rr;
                    const float s = bf16_lo(sc[r]), b = bf16_lo(bi[r]);
#pragma unroll
                    for (int m = 0; m < MW; ++m) acc[r][m] = fmaf(s, d[rr][m] - cx[m], fmaf(b, sx[m], acc[r][m]));
                }
            }
        }
    } else {
        // Three to eight activation rows: adjacent pairs, each code pair taken
        // against every activation row, weights read directly into registers.
        for (int c0 = 0; c0 < G; c0 += 64) {
            lds_barrier();  // the previous chunk's pieces have been read
            x_dma(c0);
            // Issued behind x so that the two fetches overlap.
            uint32_t w[kRpw][2 * BITS];
            uint32_t sc[kRpw], bi[kRpw];
#pragma unroll
            for (int r = 0; r < kRpw; ++r)
                load_group<BITS>(w[r], row_rsrc(r, c0, sc[r], bi[r]), (uint32_t)(c0 + lane) * kGroupBytes);
            // Every fetch so far has landed (no count of them is assumed: the
            // compiler may merge loads), then every wave's x pieces.
            wait_vm<0>();
            lds_barrier();
            float d[kRpw][MW], sx[MW];
#pragma unroll
            for (int m = 0; m < MW; ++m) {
                sx[m] = 0.f;
#pragma unroll
                for (int r = 0; r < kRpw; ++r) d[r][m] = 0.f;
            }
#pragma unroll
            for (int j8 = 0; j8 < 8; ++j8) {
                u32x4 xv[MW];
#pragma unroll
                for (int m = 0; m < MW; ++m) {
                    xv[m] = xs[(m * 8 + j8) * 64 + lane];
                    sx[m] = dot2_bf16(xv[m].x, 0x3F803F80u, sx[m]);
                    sx[m] = dot2_bf16(xv[m].y, 0x3F803F80u, sx[m]);
                    sx[m] = dot2_bf16(xv[m].z, 0x3F803F80u, sx[m]);
                    sx[m] = dot2_bf16(xv[m].w, 0x3F803F80u, sx[m]);
                }
#pragma unroll
                for (int r = 0; r < kRpw; ++r)
#pragma unroll
                    for (int p = 0; p < 4; ++p) {
                        const uint32_t cp = code_pair_bf16<BITS>(w[r], 4 * j8 + p);
#pragma unroll
                        for (int m = 0; m < MW; ++m) {
                            const uint32_t xq = p == 0 ? xv[m].x : p == 1 ? xv[m].y : p == 2 ? xv[m].z : xv[m].w;
                            d[r][m] = dot2_bf16(xq, cp, d[r][m]);
                        }
                    }
            }
#pragma unroll
            for (int r = 0; r < kRpw; ++r) {
                const float s = bf16_lo(sc[r]);
                const float c = fmaf(-128.f, s, bf16_lo(bi[r]));
#pragma unroll
                for (int m = 0; m < MW; ++m) acc[r][m] = fmaf(c, sx[m], fmaf(s, d[r][m], acc[r][m]));
            }
        }
    }

    if constexpr (KS > 1) {
        // The second wave of each pair hands its per-lane sums to the first
        // (one block barrier; the sum's order is fixed).
        __shared__ float kred[kWaves / KS][kRpw * MW][64];
        if (kh == 1)
#pragma unroll
            for (int r = 0; r < kRpw; ++r)
#pragma unroll
                for (int m = 0; m < MW; ++m) kred[wave / KS][r * MW + m][lane] = acc[r][m];
        lds_barrier();
        if (kh == 1) return;
#pragma unroll
        for (int r = 0; r < kRpw; ++r)
#pragma unroll
            for (int m = 0; m < MW; ++m) acc[r][m] += kred[wave / KS][r * MW + m][lane];
    }
    // Wave sums: value i = r*MW + m sits in every lane of row rho of t[i/4]
    // with i % 4 == sum_slot(rho); lane 16*rho stores those values.
    constexpr int V = kRpw * MW;
    float v[V];
#pragma unroll
    for (int r = 0; r < kRpw; ++r)
#pragma unroll
        for (int m = 0; m < MW; ++m) v[r * MW + m] = acc[r][m];
    float t[sum_regs(V)];
    wave_sums<V>(v, t);
    if ((lane & 15) == 0) {
        const int slot = sum_slot(lane >> 4);
#pragma unroll
        for (int q = 0; q < sum_regs(V); ++q) {
            const int i = 4 * q + slot;
            if (i >= V) continue;
            const int r = i / MW, m = i % MW;
            const int64_t row = row0 + r;
            if (row < a.N && m < mrows) a.y[y_row(m) * a.N + row] = f32_to_bf16(FP4 ? t[q] * a.ts : t[q]);
        }
    }
    }  // pass
}

template <int BITS, int MW, bool GATHER = false>
__global__ __launch_bounds__(256) void qmv_stream_kernel(StreamArgs a) {
    stream_body<BITS, MW, GATHER, 1>(a);
}

// The NVFP4 batch-1 product (large grids).
__global__ __launch_bounds__(256) void qmv_stream_nvfp4_kernel(StreamArgs a) {
    stream_body<4, 1, false, 1, true>(a);
}

// The K-split form: 8 rows per block, waves 2i and 2i + 1 alternating chunks of K.
template <int BITS, int MW>
__global__ __launch_bounds__(256) void qmv_stream_split_kernel(StreamArgs a) {
    stream_body<BITS, MW, false, 2>(a);
}

// One thread per 32 codes (BITS words): w = fma(s, q, b) written as fp32 [N, K].
template <int BITS>
__global__ __launch_bounds__(256) void dequant_stream_kernel(const uint32_t *__restrict__ w, const uint16_t *__restrict__ s,
                                                             const uint16_t *__restrict__ b, float *__restrict__ out,
                                                             int64_t chunks, int64_t chunks_per_row, int64_t K,
                                                             int64_t gs) {
    const int64_t groups = K / gs;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < chunks;
         i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t row = i / chunks_per_row;
        const int64_t k0 = (i - row * chunks_per_row) * 32;
        const int64_t g = row * groups + k0 / gs;  // 32 codes share one group (gs >= 32)
        const float sf = bf16_lo(s[g]);
        const float bf = bf16_lo(b[g]);
        uint32_t wd[BITS];
#pragma unroll
        for (int j = 0; j < BITS; ++j) wd[j] = w[i * BITS + j];
        float4 *o = reinterpret_cast<float4 *>(out + row * K + k0);
#pragma unroll
        for (int j = 0; j < 8; ++j)
            o[j] = make_float4(fmaf(sf, (float)stream_code<BITS>(wd, 4 * j), bf),
                               fmaf(sf, (float)stream_code<BITS>(wd, 4 * j + 1), bf),
                               fmaf(sf, (float)stream_code<BITS>(wd, 4 * j + 2), bf),
                               fmaf(sf, (float)stream_code<BITS>(wd, 4 * j + 3), bf));
    }
}

// Widening to 8-bit codes, one thread per 32 codes: `bits` stream words in,
// eight words out holding the same codes one per byte, low first (the 8-bit
// layout). Rows are whole multiples of 32 codes, so unit i is words
// [bits*i, bits*i + bits) in and [8i, 8i + 8) out across all rows alike.
template <int BITS>
__global__ __launch_bounds__(256) void stream_to_u8_kernel(const uint32_t *__restrict__ w, uint32_t *__restrict__ out,
                                                          int64_t units) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= units) return;
    uint32_t wd[BITS];
#pragma unroll
    for (int j = 0; j < BITS; ++j) wd[j] = w[i * BITS + j];
    uint32_t o[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
        o[j] = stream_code<BITS>(wd, 4 * j) | stream_code<BITS>(wd, 4 * j + 1) << 8 |
               stream_code<BITS>(wd, 4 * j + 2) << 16 | stream_code<BITS>(wd, 4 * j + 3) << 24;
    u32x4 *dst = reinterpret_cast<u32x4 *>(out + i * 8);
    dst[0] = u32x4{o[0], o[1], o[2], o[3]};
    dst[1] = u32x4{o[4], o[5], o[6], o[7]};
}

template <int BITS>
static const void *stream_kernel_mw(int M) {
    if (M <= 1) return reinterpret_cast<const void *>(&qmv_stream_kernel<BITS, 1>);
    if (M <= 2) return reinterpret_cast<const void *>(&qmv_stream_kernel<BITS, 2>);
    if (M <= 4) return reinterpret_cast<const void *>(&qmv_stream_kernel<BITS, 4>);
    return reinterpret_cast<const void *>(&qmv_stream_kernel<BITS, 8>);
}

const void *stream_kernel(int bits, int M) {
    if (M < 1 || M > 8) return nullptr;
    if (bits == 4) return M == 1 ? reinterpret_cast<const void *>(&qmv_stream_kernel<4, 1>) : nullptr;
    switch (bits) {
        case 2: return stream_kernel_mw<2>(M);
        case 3: return stream_kernel_mw<3>(M);
        case 5: return stream_kernel_mw<5>(M);
        case 6: return stream_kernel_mw<6>(M);
    }
    return nullptr;
}

template <int BITS>
static const void *stream_gather_mw(int mw) {
    if (mw <= 1) return reinterpret_cast<const void *>(&qmv_stream_kernel<BITS, 1, true>);
    if (mw <= 2) return reinterpret_cast<const void *>(&qmv_stream_kernel<BITS, 2, true>);
    if (mw <= 4) return reinterpret_cast<const void *>(&qmv_stream_kernel<BITS, 4, true>);
    return reinterpret_cast<const void *>(&qmv_stream_kernel<BITS, 8, true>);
}

template <int BITS>
static const void *stream_split_mw(int M) {
    if (M <= 1) return reinterpret_cast<const void *>(&qmv_stream_split_kernel<BITS, 1>);
    if (M <= 2) return reinterpret_cast<const void *>(&qmv_stream_split_kernel<BITS, 2>);
    return nullptr;
}

const void *stream_split_kernel(int bits, int M) {
    switch (bits) {
        case 2: return stream_split_mw<2>(M);
        case 3: return stream_split_mw<3>(M);
        case 5: return stream_split_mw<5>(M);
        case 6: return stream_split_mw<6>(M);
    }
    return nullptr;
}

const void *stream_nvfp4_kernel() { return reinterpret_cast<const void *>(&qmv_stream_nvfp4_kernel); }

const void *stream_gather_kernel(int bits, int mw) {
    if (mw < 1 || mw > 8) return nullptr;
    switch (bits) {
        case 2: return stream_gather_mw<2>(mw);
        case 3: return stream_gather_mw<3>(mw);
        case 5: return stream_gather_mw<5>(mw);
        case 6: return stream_gather_mw<6>(mw);
    }
    return nullptr;
}

const void *stream_to_u8_kernel(int bits) {
    switch (bits) {
        case 2: return reinterpret_cast<const void *>(&stream_to_u8_kernel<2>);
        case 3: return reinterpret_cast<const void *>(&stream_to_u8_kernel<3>);
        case 5: return reinterpret_cast<const void *>(&stream_to_u8_kernel<5>);
        case 6: return reinterpret_cast<const void *>(&stream_to_u8_kernel<6>);
    }
    return nullptr;
}

const void *stream_dequant_kernel(int bits) {
    switch (bits) {
        case 2: return reinterpret_cast<const void *>(&dequant_stream_kernel<2>);
        case 3: return reinterpret_cast<const void *>(&dequant_stream_kernel<3>);
        case 5: return reinterpret_cast<const void *>(&dequant_stream_kernel<5>);
        case 6: return reinterpret_cast<const void *>(&dequant_stream_kernel<6>);
    }
    return nullptr;
}

}  // namespace agq
