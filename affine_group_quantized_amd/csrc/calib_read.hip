// Streaming-read calibration for the benchmark (libagq_calib.so).
//
// Not part of the product: the benchmark loads this library to measure what a
// plain read of N bytes from HBM costs on the machine it runs on, so each
// product's time can be set against the practical ceiling for its byte count
// as well as against the 8 TB/s peak. The roofline-attainment figures of "epic:
// CUDA (MLX backend) prefill and decode acceleration program", Diagnosis
// (baseline), are the kind of comparison this serves.
//
// Kernel: every lane reads 16 bytes per load with a non-temporal buffer load
// (one 1 KB piece per wave instruction) and folds the words into an XOR that
// is stored only if it equals a value no data here produces, so the loads
// cannot be dropped. Two layouts of the pieces:
//  - interleaved: piece i goes to wave i mod W, so at any moment the grid reads
//    one compact band of the buffer (the walk of the product kernels);
//  - contiguous: wave w reads its own run of pieces.
// Each wave keeps U pieces in flight per stage over two stages (loads for the
// next stage go out before the current stage's data is consumed).
// An empty kernel gives the launch floor of back-to-back launches.

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kRsrcW3 = 0x00020000;  // raw buffer, 32-bit data format
constexpr int kNT = 2;               // non-temporal load policy
constexpr uint32_t kNever = 0x9E3779B9u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t range_of(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, (int)bytes, kRsrcW3);
}

// iters: stages each wave walks. Loads of stages past the walk, and of pieces
// past the buffer, take an offset at the descriptor's end and read zero
// without touching memory, so every load is unconditional (the compiler's
// wait counts stay exact) and the loop needs no tail.
template <int U, bool CONTIG>
__global__ __launch_bounds__(256) void read_kernel(const uint8_t *buf, uint32_t bytes, uint32_t iters,
                                                   uint32_t *sink) {
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6));
    const uint32_t waves = gridDim.x * (blockDim.x >> 6);
    const __amdgpu_buffer_rsrc_t r = range_of(buf, bytes);
    // Byte offset of the lane's 16 bytes of stage `it`, slot u: piece
    // (it*U + u)*waves + wave (interleaved) or (wave*iters + it)*U + u (contiguous).
    auto off = [&](uint32_t it, int u) -> uint32_t {
        const uint32_t p = CONTIG ? (wave * iters + it) * U + (uint32_t)u : (it * U + (uint32_t)u) * waves + wave;
        return it < iters ? p * 1024u + lane * 16u : bytes;
    };
    u32x4 a[U], b[U];
    uint32_t acc = 0;
#pragma unroll
    for (int u = 0; u < U; ++u) a[u] = __builtin_amdgcn_raw_buffer_load_b128(r, off(0, u), 0, kNT);
    for (uint32_t it = 0; it < iters; it += 2) {
        // a holds stage it; b takes stage it + 1 while a is folded, then a takes it + 2.
#pragma unroll
        for (int u = 0; u < U; ++u) b[u] = __builtin_amdgcn_raw_buffer_load_b128(r, off(it + 1, u), 0, kNT);
#pragma unroll
        for (int u = 0; u < U; ++u) acc ^= a[u].x ^ a[u].y ^ a[u].z ^ a[u].w;
#pragma unroll
        for (int u = 0; u < U; ++u) a[u] = __builtin_amdgcn_raw_buffer_load_b128(r, off(it + 2, u), 0, kNT);
#pragma unroll
        for (int u = 0; u < U; ++u) acc ^= b[u].x ^ b[u].y ^ b[u].z ^ b[u].w;
    }
    if (acc == kNever) sink[wave * 64u + lane] = acc;
}

__global__ void empty_kernel() {}

template <int U, bool C>
const void *sym() {
    return reinterpret_cast<const void *>(&read_kernel<U, C>);
}

}  // namespace

extern "C" {

// Read `bytes` (a multiple of 1024, below 2^31) at `buf` with `waves` waves of
// 256-thread blocks (waves a multiple of 4, at most 65536; byte offsets then stay
// below 2^32), `u` pieces per stage (1, 2 or 4),
// interleaved (contig 0) or contiguous (1). `sink` holds at least waves*64
// uint32 and is written only in the impossible case. Returns 0, or -1 for bad
// arguments, or the HIP error code of the launch.
int agqc_read(const void *buf, int64_t bytes, uint32_t *sink, int waves, int u, int contig, void *stream) {
    if (!buf || !sink || bytes <= 0 || bytes % 1024 || bytes >= (int64_t(1) << 31) || waves <= 0 || waves % 4 ||
        waves > 65536)
        return -1;
    const int64_t pieces = bytes / 1024;
    const int64_t per_stage = (int64_t)waves * u;
    const uint32_t iters = (uint32_t)((pieces + per_stage - 1) / per_stage);
    const void *k = nullptr;
    switch (u * 2 + (contig ? 1 : 0)) {
        case 2: k = sym<1, false>(); break;
        case 3: k = sym<1, true>(); break;
        case 4: k = sym<2, false>(); break;
        case 5: k = sym<2, true>(); break;
        case 8: k = sym<4, false>(); break;
        case 9: k = sym<4, true>(); break;
        default: return -1;
    }
    const uint8_t *b = static_cast<const uint8_t *>(buf);
    uint32_t nb = (uint32_t)bytes;
    void *args[] = {&b, &nb, const_cast<uint32_t *>(&iters), &sink};
    hipError_t e = hipLaunchKernel(k, dim3((unsigned)(waves / 4)), dim3(256), args, 0,
                                   static_cast<hipStream_t>(stream));
    return e == hipSuccess ? 0 : (int)e;
}

// One launch of an empty kernel of `blocks` blocks of 64 threads.
int agqc_empty(int blocks, void *stream) {
    if (blocks <= 0) return -1;
    hipError_t e = hipLaunchKernel(reinterpret_cast<const void *>(&empty_kernel), dim3((unsigned)blocks), dim3(64),
                                   nullptr, 0, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? 0 : (int)e;
}

}  // extern "C"
