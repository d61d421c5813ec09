// NVFP4 matrix-vector product for gfx950: the format path that "MLX CUDA
// Cleanup Plan", Phase 3b, keeps structurally separate from the affine one
// (mode nvfp4, group size 16). Each weight is
//     w[n, k] = e2m1(q[n, k]) * e4m3(s[n, k/16]) * tensor_scale
// with q a 4-bit E2M1 code (8 per U32, low-first, as the affine 4-bit codes),
// s one E4M3 byte per 16 consecutive columns, and one fp32 tensor scale; y is
// BF16 of the fp32 sum over k of x * w, for 1 to 4 activation rows.
//
// Work decomposition as the affine VALU kernels (row walk, K split, ring of
// row buffers, transposed wave reductions; qmv_core.hpp): lane l of a wave
// owns 16-byte chunks seg + 64 j + l of every row, 32 codes = two scale
// blocks each, and keeps its x slice in VGPRs as bf16 pairs in natural order.
// Per chunk and row: one 16-byte code load and one 2-byte load of the chunk's
// two scale bytes.
//
// Decode. v_cvt_scalef32_pk_bf16_fp4 turns byte p of a code word into the
// bf16 pair (element 2p, element 2p + 1) exactly (scale 1; the instruction
// applies only the exponent of its fp32 scale, so the block scale is applied
// afterwards in fp32). v_dot2c_f32_bf16 multiplies the pairs by the matching
// x pairs; each 16-code block's sum takes its scale from v_cvt_f32_fp8 (OCP
// E4M3): acc += e4m3(s0) * d0 + e4m3(s1) * d1. Each chunk is decoded once for
// all activation rows: about 0.6 + 0.5 * M VALU ops per code.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "plan.hpp"
#include "qmv_core.hpp"
#include "qmv_device.hpp"
#include "qmv_kernels.hpp"

namespace agq {

namespace {

// One iteration's codes and scale bytes for R weight rows.
template <int CPT, int R>
struct Fp4Buf {
    u32x4 w[R][CPT];
    uint16_t s[R][CPT];  // the chunk's two E4M3 scale bytes
};

// Every load of rows [rb, rb + R) at once; rows past `end` and chunks past the
// row read zero through their descriptors (no load is conditional).
template <int CPT, int R>
__device__ __forceinline__ void load_fp4_rows(Fp4Buf<CPT, R> &buf, const Nvfp4Args &a, int64_t rb, int64_t end,
                                              const uint32_t (&woff)[CPT], const uint32_t (&soff)[CPT]) {
    const uint32_t rowbytes = (uint32_t)a.C * 16u, srow = (uint32_t)a.C * 2u;
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const bool in = rb + r < end;
        const int64_t row = in ? rb + r : 0;
        const __amdgpu_buffer_rsrc_t wr = byte_range(a.w + row * a.C, in ? rowbytes : 0u);
#pragma unroll
        for (int j = 0; j < CPT; ++j) buf.w[r][j] = __builtin_amdgcn_raw_buffer_load_b128(wr, woff[j], 0, kLoadNT);
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const bool in = rb + r < end;
        const int64_t row = in ? rb + r : 0;
        const __amdgpu_buffer_rsrc_t sr = byte_range(a.s + row * (int64_t)srow, in ? srow : 0u);
#pragma unroll
        for (int j = 0; j < CPT; ++j) buf.s[r][j] = __builtin_amdgcn_raw_buffer_load_b16(sr, soff[j], 0, kLoadNT);
    }
}

// The 16 bf16 pairs of one 16-byte chunk (32 codes), in natural order.
__device__ __forceinline__ void fp4_pairs(const u32x4 &wv, uint32_t (&pw)[16]) {
    const uint32_t w[4] = {wv.x, wv.y, wv.z, wv.w};
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        // (the byte selector must be a literal)
        pw[4 * t + 0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[t], 1.0f, 0));
        pw[4 * t + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[t], 1.0f, 1));
        pw[4 * t + 2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[t], 1.0f, 2));
        pw[4 * t + 3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[t], 1.0f, 3));
    }
}

// acc + e4m3(s0) * (first 16 codes . x) + e4m3(s1) * (last 16 codes . x) for one activation row.
__device__ __forceinline__ float fp4_dot(const uint32_t (&pw)[16], float s0, float s1, const uint32_t (&xv)[16],
                                        float acc) {
    float d0 = 0.f, d1 = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) d0 = dot2_bf16(pw[i], xv[i], d0);
#pragma unroll
    for (int i = 8; i < 16; ++i) d1 = dot2_bf16(pw[i], xv[i], d1);
    return fmaf(s1, d1, fmaf(s0, d0, acc));
}

// Output rows: y[m, n] = bf16(v * tensor_scale).
struct Fp4Out {
    static constexpr bool kGlu = false;
    uint16_t *y;
    int64_t N;
    float ts;
    __device__ __forceinline__ void put(int m, int64_t n, float v) const { y[(int64_t)m * N + n] = f32_to_bf16(v * ts); }
};

}  // namespace

template <int CPT, int MW, int R, int NB>
__global__ __launch_bounds__(512) void nvfp4_kernel(Nvfp4Args a) {
    __shared__ float red[kRedFloats];
    const int lane = threadIdx.x & 63;
    const int wave = wave_id();
    const int S = a.S;
    const int wig = wave % S, grp = wave / S;
    const int64_t rg = (int64_t)blockIdx.x * a.GPB + grp;
    const RowWalk walk{rg * R, (int64_t)gridDim.x * a.GPB * R, a.N};
    // Waves without rows leave only when they meet no block barrier (S == 1).
    if (S == 1 && walk.first >= walk.end) return;
    const int iters = (int)(a.RPG / R);  // a multiple of NB

    int chunk[CPT];
    bool cv[CPT];
    uint32_t woff[CPT], soff[CPT];
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
        chunk[j] = (wig * CPT + j) * 64 + lane;
        cv[j] = chunk[j] < a.C;
        woff[j] = (uint32_t)chunk[j] * 16u;
        soff[j] = (uint32_t)chunk[j] * 2u;
    }
    // x: 64 bytes (32 bf16, 16 natural pairs) per chunk and activation row;
    // lanes past the row end keep zeros.
    u32x4 xraw[MW][CPT][4];
#pragma unroll
    for (int m = 0; m < MW; ++m)
#pragma unroll
        for (int j = 0; j < CPT; ++j) {
            const u32x4 *p = reinterpret_cast<const u32x4 *>(a.x + (int64_t)m * a.K) + (int64_t)(cv[j] ? chunk[j] : 0) * 4;
#pragma unroll
            for (int t = 0; t < 4; ++t) xraw[m][j][t] = p[t];
        }
    __builtin_amdgcn_sched_barrier(0);
    Fp4Buf<CPT, R> buf[NB];
    load_fp4_rows<CPT, R>(buf[0], a, walk.at(0), walk.end, woff, soff);
    __builtin_amdgcn_sched_barrier(0);
    uint32_t xv[MW][CPT][16];
#pragma unroll
    for (int m = 0; m < MW; ++m)
#pragma unroll
        for (int j = 0; j < CPT; ++j) {
            const uint32_t keep = cv[j] ? 0xFFFFFFFFu : 0u;
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const u32x4 q = xraw[m][j][t] & keep;
                xv[m][j][4 * t + 0] = q.x;
                xv[m][j][4 * t + 1] = q.y;
                xv[m][j][4 * t + 2] = q.z;
                xv[m][j][4 * t + 3] = q.w;
            }
        }
#pragma unroll
    for (int p = 1; p < NB; ++p) load_fp4_rows<CPT, R>(buf[p], a, walk.at(p), walk.end, woff, soff);
    __builtin_amdgcn_sched_barrier(0);

    const Fp4Out out{a.y, a.N, a.ts};
    float acc[R][MW], pend = 0.f;
    auto step = [&](const Fp4Buf<CPT, R> &b, int it) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
#pragma unroll
            for (int m = 0; m < MW; ++m) acc[r][m] = 0.f;
#pragma unroll
            for (int j = 0; j < CPT; ++j) {
                uint32_t pw[16];
                fp4_pairs(b.w[r][j], pw);  // decoded once for every activation row
                const float s0 = __builtin_amdgcn_cvt_f32_fp8((uint32_t)b.s[r][j], 0);
                const float s1 = __builtin_amdgcn_cvt_f32_fp8((uint32_t)b.s[r][j], 1);
#pragma unroll
                for (int m = 0; m < MW; ++m) acc[r][m] = fp4_dot(pw, s0, s1, xv[m][j], acc[r][m]);
            }
        }
        finish_rows<MW, R>(acc, out, walk, it, iters, S, wig, grp, lane, red, pend);
    };
    int it0 = 0;
    for (; it0 + NB < iters; it0 += NB) {
#pragma unroll
        for (int p = 0; p < NB; ++p) {
            step(buf[p], it0 + p);
            load_fp4_rows<CPT, R>(buf[p], a, walk.at(it0 + p + NB), walk.end, woff, soff);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
#pragma unroll
    for (int p = 0; p < NB; ++p) step(buf[p], it0 + p);
}

// ---------------------------------------------------------------------------
// Kernel selection: the plans plan_shape() gives for 1-4 activation rows of
// 32-code chunks, with x staged by each wave.

namespace {

template <int MW, int CPT>
const void *nvfp4_sym(int R, int NB) {
    constexpr int RS = plan_rows(CPT, MW, false), RD = plan_rows(CPT, MW, true);
    constexpr int NS = plan_stages(MW, false), ND = plan_stages(MW, true);
    constexpr int RW = plan_rows(CPT, MW, false, true), NW = plan_stages(MW, false, true, CPT);
    if (R == RS && NB == NS) return reinterpret_cast<const void *>(&nvfp4_kernel<CPT, MW, RS, NS>);
    if constexpr (RD != RS || ND != NS) {
        if (R == RD && NB == ND) return reinterpret_cast<const void *>(&nvfp4_kernel<CPT, MW, RD, ND>);
    }
    if constexpr (MW > 1 && (RW != RS || NW != NS)) {
        if (R == RW && NB == NW) return reinterpret_cast<const void *>(&nvfp4_kernel<CPT, MW, RW, NW>);
    }
    return nullptr;
}

template <int MW>
const void *nvfp4_by_cpt(int cpt, int R, int NB) {
    if constexpr (MW == 1) {
        switch (cpt) {
            case 1: return nvfp4_sym<1, 1>(R, NB);
            case 2: return nvfp4_sym<1, 2>(R, NB);
            case 3: return nvfp4_sym<1, 3>(R, NB);
            case 4: return nvfp4_sym<1, 4>(R, NB);
            case 5: return nvfp4_sym<1, 5>(R, NB);
            case 6: return nvfp4_sym<1, 6>(R, NB);
            case 7: return nvfp4_sym<1, 7>(R, NB);
        }
    } else if constexpr (MW == 2) {
        switch (cpt) {
            case 1: return nvfp4_sym<2, 1>(R, NB);
            case 2: return nvfp4_sym<2, 2>(R, NB);
            case 3: return nvfp4_sym<2, 3>(R, NB);
            case 4: return nvfp4_sym<2, 4>(R, NB);
        }
    } else {
        switch (cpt) {
            case 1: return nvfp4_sym<MW, 1>(R, NB);
            case 2: return nvfp4_sym<MW, 2>(R, NB);
        }
    }
    return nullptr;
}

}  // namespace

const void *nvfp4_kernel_for(int mw, int cpt, int R, int NB) {
    static_assert(kMaxCpt == 7 && kXRegBudget == 8, "instantiations above cover the plans of 1-4 rows");
    switch (mw) {
        case 1: return nvfp4_by_cpt<1>(cpt, R, NB);
        case 2: return nvfp4_by_cpt<2>(cpt, R, NB);
        case 3: return nvfp4_by_cpt<3>(cpt, R, NB);
        case 4: return nvfp4_by_cpt<4>(cpt, R, NB);
    }
    return nullptr;
}

}  // namespace agq
