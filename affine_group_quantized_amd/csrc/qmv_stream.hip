// Affine group-quantized products for the bit-stream widths: 2-, 3-, 5- and
// 6-bit codes with group size 64, the other widths of the affine family that
// "MLX CUDA Cleanup Plan" (Target Architecture §1; Refactor Plan, Phase 3)
// names at 4 and 8 bits. A row's codes form one low-first bit stream over its
// uint32 words: code k occupies stream bits bits*k .. bits*k + bits - 1, word
// i holding bits 32i .. 32i + 31 (for 2 bits, k / 16 and k % 16 exactly as the
// 4- and 8-bit layouts; a 3-, 5- or 6-bit code may run into the next word).
// A 64-column group is then exactly 2*bits words (16, 24, 40 or 48 bytes).
//
//     y[m, n] = sum_k x[m, k] * (s[n, g] * q[n, k] + b[n, g]),  g = k / 64
//             = sum_g s[n, g] * D[m, n, g] + (b[n, g] - 128 s[n, g]) * X[m, g],
//     D = sum_{k in g} x[m, k] * (128 + q[n, k]),  X = sum_{k in g} x[m, k]
// (the regrouping of the 4-bit VALU products). Each pair of adjacent codes
// becomes the bfloat16 pair (128 + q, 128 + q') exactly (a code below 128 in
// the low mantissa bits of 0x4300), and one v_dot2c_f32_bf16 per activation
// row takes it against the pair of activations in natural order: about two
// VALU instructions per code (a shift or funnel shift, two and-ors and a
// shift per pair) plus half a dot per code and row.
//
// Layout of the work: lane l of a wave takes group l of a 64-group chunk of K,
// so a wave reads one weight row's chunk as one contiguous run; each wave
// takes 4 weight rows, a block 4 waves. Per chunk the block stages x (up to 8
// rows) in LDS as 16-byte pieces [row][piece][group], so the 64 lanes read 64
// consecutive pieces (no bank conflicts), once for the wave's 4 rows, with
// their sums X. The wave sums come from the DPP / permlane tree of the VALU
// products.

#include <hip/hip_runtime.h>
#include <stdint.h>

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

// The 2*BITS words of group g of a row: 16-byte loads where groups are 16-byte
// aligned (2 and 6 bits), 8-byte loads otherwise (3 and 5 bits). Past the
// row's range (its end, or a row past N) the words read zero.
template <int BITS>
__device__ __forceinline__ void load_group(uint32_t (&w)[2 * BITS], __amdgpu_buffer_rsrc_t r, uint32_t off) {
    if constexpr (BITS % 2 == 0) {
#pragma unroll
        for (int i = 0; i < BITS / 2; ++i) {
            const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, off + 16u * i, 0, 2);
            w[4 * i] = v.x;
            w[4 * i + 1] = v.y;
            w[4 * i + 2] = v.z;
            w[4 * i + 3] = v.w;
        }
    } else {
#pragma unroll
        for (int i = 0; i < BITS; ++i) {
            const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, off + 8u * i, 0, 2);
            w[2 * i] = v.x;
            w[2 * i + 1] = v.y;
        }
    }
}

}  // namespace

template <int BITS, int MW>
__global__ __launch_bounds__(256) void qmv_stream_kernel(StreamArgs a) {
    __shared__ u32x4 xs[MW * 8 * 64];  // [row][piece of 8 columns][group]
    const int lane = threadIdx.x & 63;
    const int64_t row0 = ((int64_t)blockIdx.x * kWaves + wave_id()) * kRpw;
    const int G = a.K / 64;
    const uint32_t rowbytes = (uint32_t)a.K / 8u * BITS;
    const __amdgpu_buffer_rsrc_t xr = span(a.x, (uint32_t)a.M * (uint32_t)a.K * 2u);
    float acc[kRpw][MW];
#pragma unroll
    for (int r = 0; r < kRpw; ++r)
#pragma unroll
        for (int m = 0; m < MW; ++m) acc[r][m] = 0.f;

    for (int c0 = 0; c0 < G; c0 += 64) {
        // x of the chunk with direct-to-LDS loads, issued first: instruction
        // (m, j8) brings piece j8 of every group of row m, lane g landing at slot
        // g of [m][j8][.]. Rows past M and columns past K read zero (each row's
        // range is its own K columns). The 4 waves take every fourth (m, j8).
        lds_barrier();  // the previous chunk's pieces have been read
        for (int q = wave_id(); q < MW * 8; q += kWaves) {
            const int m = q >> 3, j8 = q & 7;
            const __amdgpu_buffer_rsrc_t xr = span(a.x + (int64_t)(m < a.M ? m : 0) * a.K, m < a.M ? (uint32_t)a.K * 2u : 0u);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                xr, (__attribute__((address_space(3))) void *)(xs + q * 64),
                16, ((uint32_t)(c0 + lane) * 64u + 8u * (uint32_t)j8) * 2u, 0, 0, 0);
        }
        // The codes, scale and bias of group c0 + lane of each of the wave's rows
        // (zeros past the row's groups and for rows past N), issued behind x so
        // that the two fetches overlap.
        uint32_t w[kRpw][2 * BITS];
        uint32_t sc[kRpw], bi[kRpw];
#pragma unroll
        for (int r = 0; r < kRpw; ++r) {
            const int64_t row = row0 + r;
            const bool ok = row < a.N;
            const int64_t rr = ok ? row : 0;
            load_group<BITS>(w[r], span(a.w + rr * (rowbytes / 4u), ok ? rowbytes : 0u),
                             (uint32_t)(c0 + lane) * 8u * BITS);
            const uint32_t sb = ok ? (uint32_t)G * 2u : 0u;
            sc[r] = __builtin_amdgcn_raw_buffer_load_b16(span(a.s + rr * G, sb), (uint32_t)(c0 + lane) * 2u, 0, 0);
            bi[r] = __builtin_amdgcn_raw_buffer_load_b16(span(a.b + rr * G, sb), (uint32_t)(c0 + lane) * 2u, 0, 0);
        }
        // Both fetches are in flight together; wait for all of them (the compiler
        // may merge the weight loads, so no count of them is assumed), then for
        // every wave's pieces at the barrier.
        wait_vm<0>();
        lds_barrier();
        // D per row and activation row, and X, over the lane's group.
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
                        const uint32_t xp = p == 0 ? xv[m].x : p == 1 ? xv[m].y : p == 2 ? xv[m].z : xv[m].w;
                        d[r][m] = dot2_bf16(xp, cp, d[r][m]);
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
            if (row < a.N && m < a.M) a.y[(int64_t)m * a.N + row] = f32_to_bf16(t[q]);
        }
    }
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

template <int BITS>
static const void *stream_kernel_mw(int M) {
    if (M <= 1) return reinterpret_cast<const void *>(&qmv_stream_kernel<BITS, 1>);
    if (M <= 2) return reinterpret_cast<const void *>(&qmv_stream_kernel<BITS, 2>);
    if (M <= 4) return reinterpret_cast<const void *>(&qmv_stream_kernel<BITS, 4>);
    return reinterpret_cast<const void *>(&qmv_stream_kernel<BITS, 8>);
}

const void *stream_kernel(int bits, int M) {
    if (M < 1 || M > 8) return nullptr;
    switch (bits) {
        case 2: return stream_kernel_mw<2>(M);
        case 3: return stream_kernel_mw<3>(M);
        case 5: return stream_kernel_mw<5>(M);
        case 6: return stream_kernel_mw<6>(M);
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
