// C ABI of libagq: argument validation, launch planning and kernel launches.
//
// The boundary follows the accelerator interface of "MLX CUDA Cleanup Plan",
// Target Architecture §2-§4 and Hard Constraints. Callers pass borrowed device
// buffers. A call adds no host or device copies and no synchronization. It
// falls back to no other path: a shape it does not implement returns
// AGQ_ENOTSUP to the caller.
//
// Every argument check runs before the first HIP call.

#include <hip/hip_runtime_api.h>

#include <atomic>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "agq.h"
#include "plan.hpp"
#include "moe.hpp"
#include "plan_mfma.hpp"
#include "qmm.hpp"
#include "qmv_kernels.hpp"

namespace {

thread_local char g_err[512] = "";

agq_status fail(agq_status st, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return st;
}

constexpr int kMaxDevices = 64;

struct DeviceInfo {
    std::atomic<int> state{0};  // 0 unknown, 1 ready
    int cus = 0;
    bool gfx950 = false;
    char arch[64] = "";
};

DeviceInfo g_dev[kMaxDevices];
std::mutex g_dev_mu;

// Current device's compute-unit count; checks once per device that it is gfx950.
agq_status current_device(int *cus, int *ordinal) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(AGQ_EHIP, "hipGetDevice failed: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices) return fail(AGQ_EHIP, "device ordinal %d out of range", dev);
    DeviceInfo &d = g_dev[dev];
    if (d.state.load(std::memory_order_acquire) == 0) {
        std::lock_guard<std::mutex> lock(g_dev_mu);
        if (d.state.load(std::memory_order_relaxed) == 0) {
            hipDeviceProp_t prop;
            e = hipGetDeviceProperties(&prop, dev);
            if (e != hipSuccess)
                return fail(AGQ_EHIP, "hipGetDeviceProperties(%d) failed: %s", dev, hipGetErrorString(e));
            std::snprintf(d.arch, sizeof d.arch, "%s", prop.gcnArchName);
            d.gfx950 = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
            d.cus = prop.multiProcessorCount;
            d.state.store(1, std::memory_order_release);
        }
    }
    if (!d.gfx950) return fail(AGQ_ENOTSUP, "device %d is %s; libagq is built for gfx950 only", dev, d.arch);
    *cus = d.cus;
    *ordinal = dev;
    return AGQ_OK;
}

// Blocks of `sym` resident per compute unit, from the HIP occupancy query,
// cached per kernel, block size, dynamic LDS and device. (One kernel can run
// with several block sizes: the K split S sets the waves per block.)
struct OccEntry {
    const void *sym;
    int dev;
    int threads;
    size_t lds;
    int blocks_per_cu;
};
constexpr int kOccSlots = 256;
OccEntry g_occ[kOccSlots];
int g_occ_n = 0;
std::mutex g_occ_mu;

// Each thread first looks in its own small direct-mapped copy of the cache, so
// a steady stream of calls takes no lock and scans nothing.
constexpr int kOccLocal = 16;
thread_local OccEntry t_occ[kOccLocal];

agq_status resident_waves(const void *sym, int threads, size_t lds, int cus, int dev, int64_t *waves) {
    OccEntry &mine = t_occ[(reinterpret_cast<uintptr_t>(sym) >> 6 ^ (uintptr_t)threads ^ lds ^ (uintptr_t)dev) %
                           kOccLocal];
    if (mine.sym == sym && mine.dev == dev && mine.threads == threads && mine.lds == lds) {
        *waves = (int64_t)cus * mine.blocks_per_cu * (threads / 64);
        return AGQ_OK;
    }
    int bpc = -1;
    {
        std::lock_guard<std::mutex> lock(g_occ_mu);
        for (int i = 0; i < g_occ_n; ++i)
            if (g_occ[i].sym == sym && g_occ[i].dev == dev && g_occ[i].threads == threads && g_occ[i].lds == lds)
                bpc = g_occ[i].blocks_per_cu;
    }
    if (bpc < 0) {
        hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&bpc, sym, threads, lds);
        if (e != hipSuccess) return fail(AGQ_EHIP, "occupancy query failed: %s", hipGetErrorString(e));
        if (bpc < 1) bpc = 1;
        std::lock_guard<std::mutex> lock(g_occ_mu);
        if (g_occ_n < kOccSlots) g_occ[g_occ_n++] = OccEntry{sym, dev, threads, lds, bpc};
    }
    mine = OccEntry{sym, dev, threads, lds, bpc};
    *waves = (int64_t)cus * bpc * (threads / 64);
    return AGQ_OK;
}

// Dynamic LDS above the runtime's default 64 KB needs the kernel's limit raised
// first (once per kernel, device and size).
constexpr size_t kDefaultDynLds = 65536;
constexpr size_t kMaxDynLds = 160 * 1024;
struct LdsEntry {
    const void *sym;
    int dev;
    size_t bytes;
};
LdsEntry g_lds[64];
int g_lds_n = 0;
std::mutex g_lds_mu;

agq_status allow_lds(const void *sym, size_t bytes, int dev) {
    if (bytes <= kDefaultDynLds) return AGQ_OK;
    if (bytes > kMaxDynLds) return fail(AGQ_ENOTSUP, "%zu bytes of LDS exceed the compute unit's", bytes);
    std::lock_guard<std::mutex> lock(g_lds_mu);
    for (int i = 0; i < g_lds_n; ++i)
        if (g_lds[i].sym == sym && g_lds[i].dev == dev && g_lds[i].bytes >= bytes) return AGQ_OK;
    hipError_t e = hipFuncSetAttribute(sym, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
    if (e != hipSuccess) return fail(AGQ_EHIP, "raising the kernel's LDS limit failed: %s", hipGetErrorString(e));
    if (g_lds_n < 64) g_lds[g_lds_n++] = LdsEntry{sym, dev, bytes};
    return AGQ_OK;
}

bool misaligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) != 0; }

constexpr int64_t kMaxN = int64_t(1) << 40;
constexpr int64_t kMaxK = int64_t(1) << 30;

// Format checks shared by every entry point.
agq_status check_format(int64_t N, int64_t K, int bits, int group_size) {
    if (N <= 0 || K <= 0)
        return fail(AGQ_EINVAL, "N and K must be positive (N=%lld, K=%lld)", (long long)N, (long long)K);
    if (N > kMaxN || K > kMaxK)
        return fail(AGQ_EINVAL, "N or K too large (N=%lld, K=%lld)", (long long)N, (long long)K);
    if (group_size <= 0) return fail(AGQ_EINVAL, "group_size must be positive (got %d)", group_size);
    if (bits != 2 && bits != 3 && bits != 4 && bits != 5 && bits != 6 && bits != 8)
        return fail(AGQ_ENOTSUP, "bits=%d not supported (2, 3, 4, 5, 6 or 8)", bits);
    if (group_size != 32 && group_size != 64 && group_size != 128)
        return fail(AGQ_ENOTSUP, "group_size=%d not supported (32, 64 or 128)", group_size);
    if (K % group_size != 0) return fail(AGQ_EINVAL, "K=%lld is not a multiple of group_size", (long long)K);
    return AGQ_OK;
}

// The bit-stream widths (2, 3, 5, 6 bits): the matvec, quantize and dequantize
// forms only.
bool stream_bits(int bits) { return bits != 4 && bits != 8; }
agq_status need_4_or_8(int bits, const char *what) {
    if (stream_bits(bits)) return fail(AGQ_ENOTSUP, "bits=%d: %s takes 4- or 8-bit codes", bits, what);
    return AGQ_OK;
}

// Format and operand checks shared by the products and dequantize.
agq_status check_operands(const void *x, const void *w, const void *s, const void *b, const void *y, int64_t N,
                          int64_t K, int bits, int group_size, bool need_x) {
    if ((need_x && !x) || !w || !s || !b || !y) return fail(AGQ_EINVAL, "null tensor pointer");
    agq_status st = check_format(N, K, bits, group_size);
    if (st != AGQ_OK) return st;
    if ((need_x && misaligned(x, 16)) || misaligned(w, 16))
        return fail(AGQ_EINVAL, "x and w must be 16-byte aligned");
    if (misaligned(s, 2) || misaligned(b, 2) || misaligned(y, 2))
        return fail(AGQ_EINVAL, "scales, biases and y must be 2-byte aligned");
    return AGQ_OK;
}

// Kernel and tiling for a product on the current device: the grid holds one
// row group per resident wave set of the chosen kernel. Walks of at least
// kDeepRows rows per group use the deep-load instantiation.
agq_status launch_plan(int64_t M, int64_t N, int64_t K, int bits, int64_t experts, agq::Plan *plan,
                       const void **sym) {
    const int64_t rows = experts > 0 ? agq::kGatherMW : M;
    if (agq::plan_shape(rows, K, bits, experts, plan) != AGQ_OK)
        return fail(AGQ_ENOTSUP, "K=%lld too large for %lld activation rows at %d bits", (long long)K,
                    (long long)rows, bits);
    int cus = 0, dev = 0;
    agq_status st = current_device(&cus, &dev);
    if (st != AGQ_OK) return st;
    for (int pass = 0; pass < 2; ++pass) {
        *sym = agq::product_kernel(bits, plan->mw, plan->cpt, plan->R, plan->NB,
                                   plan->x_lds_bytes > 0 ? plan->S : 0, experts > 0);
        if (!*sym)
            return fail(AGQ_ENOTSUP, "no kernel for bits=%d rows=%d cpt=%d R=%d", bits, plan->mw, plan->cpt,
                        plan->R);
        int64_t waves = 0;
        st = resident_waves(*sym, plan->threads, (size_t)plan->x_lds_bytes, cus, dev, &waves);
        if (st != AGQ_OK) return st;
        if (pass == 0 && agq::wants_deep(N, waves, plan->S, experts)) {
            agq::plan_shape(rows, K, bits, experts, plan, true);
            continue;
        }
        agq::plan_grid(N, waves, experts, plan);
        return AGQ_OK;
    }
    return AGQ_OK;
}

// Matrix-core plan on the current device: the grid is sized from the
// occupancy of the chosen kernel at its block size.
agq_status launch_mfma_plan(int64_t M, int64_t N, int64_t K, int64_t experts, agq::MfmaPlan *plan,
                            const void **sym, int passes = 1) {
    agq::mfma_shape(N, K, experts, plan);
    agq::mfma_lds(experts, M, plan);  // (gather: M is the pair count P)
    int cus = 0, dev = 0;
    agq_status st = current_device(&cus, &dev);
    if (st != AGQ_OK) return st;
    *sym = agq::mfma_kernel(plan->T, experts > 0, (int)(M < 16 ? M : 16));
    if (!*sym) return fail(AGQ_ENOTSUP, "no matrix-core kernel for %d tiles", plan->T);
    int64_t waves = 0;
    st = resident_waves(*sym, plan->threads, (size_t)plan->lds_bytes, cus, dev, &waves);
    if (st != AGQ_OK) return st;
    // Passes of 16 rows in one launch share the residency, so they run together.
    agq::mfma_grid(waves / passes, experts, plan);
    return AGQ_OK;
}

void export_mfma_plan(const agq::MfmaPlan &p, int64_t K, agq_plan *out) {
    *out = agq_plan{};
    out->bits = 4;
    out->chunks_per_row = (int32_t)(K / 32);
    out->cpt = 0;
    out->mw = p.pass_rows;
    out->rows_per_iter = 16 * p.T;
    out->stages = agq::kMfmaRing;
    out->waves_per_group = p.S;
    out->groups_per_block = 1;
    out->threads_per_block = p.threads;
    out->rows_per_group = (int64_t)p.BPG * 16 * p.T;
    out->row_groups = p.groups;
    out->blocks = p.groups;
    out->row_order = 0;
    out->x_lds_bytes = 0;
    out->resident_waves = (int32_t)p.resident;
    out->engine = 1;
}

agq::MfmaArgs make_mfma_args(const void *x, const uint32_t *w, const void *s, const void *b, void *y, int64_t N,
                             int64_t K, int M, const agq::MfmaPlan &p) {
    agq::MfmaArgs a{};
    a.x = static_cast<const uint16_t *>(x);
    a.w = w;
    a.s = static_cast<const uint16_t *>(s);
    a.b = static_cast<const uint16_t *>(b);
    a.y = static_cast<uint16_t *>(y);
    a.N = N;
    a.K = (int32_t)K;
    a.G = (int32_t)(K / 64);
    a.M = M;
    a.S = p.S;
    a.SPW = p.SPW;
    a.BPG = p.BPG;
    return a;
}

void export_plan(const agq::Plan &p, agq_plan *out) {
    *out = agq_plan{};
    out->bits = p.bits;
    out->chunks_per_row = p.C;
    out->cpt = p.cpt;
    out->mw = p.mw;
    out->rows_per_iter = p.R;
    out->stages = p.NB;
    out->waves_per_group = p.S;
    out->groups_per_block = p.GPB;
    out->threads_per_block = p.threads;
    out->rows_per_group = p.RPG;
    out->row_groups = p.TG;
    out->blocks = p.blocks;
    out->row_order = 0;
    out->x_lds_bytes = p.x_lds_bytes;
    out->resident_waves = (int32_t)p.resident;
    out->engine = 0;
}

// Batch-1 4-bit products (group size 64) whose grid of 16-row blocks gives
// every compute unit at least two run on the bit-stream kernel: its weight
// rows pass through LDS in contiguous loads and the fetches run a step ahead,
// which beats the VALU plans there (lm_head 128256x4096: 43.6 against 45.4 us;
// gate_up 28672x4096: 12.7 against 13.3 us). Short grids (N = 4096 at K =
// 14336: one wave per SIMD) stay on the VALU plans.
bool stream4(int64_t M, int64_t N, int bits, int group_size, int64_t experts, int cus) {
    return bits == 4 && group_size == 64 && M == 1 && experts == 0 &&
           (N + agq::kStreamRowsPerBlock - 1) / agq::kStreamRowsPerBlock >= 2 * (int64_t)cus;
}

// The launch plan record of the bit-stream kernel (engine 2).
void export_stream_plan(int64_t N, int64_t K, int bits, int64_t resident, agq_plan *out) {
    *out = agq_plan{};
    out->bits = bits;
    out->chunks_per_row = (int32_t)(K * bits / 128);
    out->cpt = 0;
    out->mw = 1;
    out->rows_per_iter = 4;
    out->stages = 2;
    out->waves_per_group = 1;
    out->groups_per_block = 4;
    out->threads_per_block = 256;
    out->rows_per_group = 4;
    out->blocks = (N + agq::kStreamRowsPerBlock - 1) / agq::kStreamRowsPerBlock;
    out->row_groups = out->blocks * 4;
    out->row_order = 1;
    out->x_lds_bytes = 8192;
    out->resident_waves = (int32_t)resident;
    out->engine = 2;
}

agq::ProductArgs make_args(const void *x, const uint32_t *w, const void *s, const void *b, void *y, int64_t N,
                           int64_t K, int bits, int M, const agq::Plan &p, int group_size) {
    agq::ProductArgs a{};
    a.x = static_cast<const uint16_t *>(x);
    a.w = reinterpret_cast<const agq::u32x4 *>(w);
    a.s = static_cast<const uint16_t *>(s);
    a.b = static_cast<const uint16_t *>(b);
    a.y = static_cast<uint16_t *>(y);
    a.N = N;
    a.RPG = p.RPG;
    a.K = (int32_t)K;
    a.C = (int32_t)(K * bits / 128);
    a.G = (int32_t)(K / group_size);
    int cpg = group_size * bits / 128;  // 16-byte chunks per group: 1, 2, 4 or 8
    a.gshift = 0;
    while (cpg > 1) {
        cpg >>= 1;
        ++a.gshift;
    }
    a.M = M;
    a.S = p.S;
    a.GPB = p.GPB;
    return a;
}

agq_status launch(const void *sym, dim3 grid, dim3 block, size_t lds, void *arg, void *stream) {
    void *args[] = {arg};
    hipError_t e = hipLaunchKernel(sym, grid, block, args, lds, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(AGQ_EHIP, "kernel launch failed: %s", hipGetErrorString(e));
    return AGQ_OK;
}

agq_status dense_product(const void *x, const uint32_t *w, const void *s, const void *b, void *y, int64_t M,
                         int64_t N, int64_t K, int bits, int group_size, void *stream) {
    agq_status st = check_operands(x, w, s, b, y, N, K, bits, group_size, true);
    if (st != AGQ_OK) return st;
    if (M <= 0) return fail(AGQ_EINVAL, "M must be positive (got %lld)", (long long)M);
    if (M > 8) return fail(AGQ_ENOTSUP, "M=%lld > 8 is a quantized GEMM, not a matvec", (long long)M);
    bool on_stream = stream_bits(bits);
    if (bits == 4 && group_size == 64 && M == 1) {
        // The 4-bit K limit holds on either kernel (and is checked before any HIP call).
        agq::Plan limit;
        if (agq::plan_shape(M, K, bits, 0, &limit) != AGQ_OK)
            return fail(AGQ_ENOTSUP, "K=%lld too large for M=%lld at %d bits", (long long)K, (long long)M, bits);
        int cus = 0, dev = 0;
        st = current_device(&cus, &dev);
        if (st != AGQ_OK) return st;
        on_stream = stream4(M, N, bits, group_size, 0, cus);
    }
    if (on_stream) {
        if (group_size != 64) return fail(AGQ_ENOTSUP, "bits=%d takes group size 64", bits);
        if (M * K * 2 >= (int64_t(1) << 31)) return fail(AGQ_ENOTSUP, "x must stay below 2 GiB (M*K*2 bytes)");
        if ((N + agq::kStreamRowsPerBlock - 1) / agq::kStreamRowsPerBlock > INT32_MAX)
            return fail(AGQ_ENOTSUP, "N=%lld too large", (long long)N);
        agq::StreamArgs a{static_cast<const uint16_t *>(x), w, static_cast<const uint16_t *>(s),
                          static_cast<const uint16_t *>(b), static_cast<uint16_t *>(y), N, (int32_t)K, (int32_t)M};
        const int64_t blocks = (N + agq::kStreamRowsPerBlock - 1) / agq::kStreamRowsPerBlock;
        if (M <= 2 && K / 64 >= 128 && stream_bits(bits)) {
            // Short grids over several chunks of K: the K-split form, 8 rows per
            // block, two waves per row set alternating chunks.
            int cus = 0, dev = 0;
            st = current_device(&cus, &dev);
            if (st != AGQ_OK) return st;
            if (blocks < 2 * (int64_t)cus)
                return launch(agq::stream_split_kernel(bits, (int)M), dim3((unsigned)((N + 7) / 8)), dim3(256), 0, &a,
                              stream);
        }
        return launch(agq::stream_kernel(bits, (int)M), dim3((unsigned)blocks), dim3(256), 0, &a, stream);
    }
    if (group_size == 64 && agq::mfma_eligible(M, K, bits, 0, M)) {
        agq::MfmaPlan mp;
        const void *sym = nullptr;
        st = launch_mfma_plan(M, N, K, 0, &mp, &sym);
        if (st != AGQ_OK) return st;
        agq::MfmaArgs a = make_mfma_args(x, w, s, b, y, N, K, (int)M, mp);
        return launch(sym, dim3((unsigned)mp.groups), dim3(mp.threads), (size_t)mp.lds_bytes, &a, stream);
    }
    agq::Plan plan;
    if (agq::plan_shape(M, K, bits, 0, &plan) != AGQ_OK)  // host-only check before any HIP call
        return fail(AGQ_ENOTSUP, "K=%lld too large for M=%lld at %d bits", (long long)K, (long long)M, bits);
    const void *sym = nullptr;
    st = launch_plan(M, N, K, bits, 0, &plan, &sym);
    if (st != AGQ_OK) return st;
    agq::ProductArgs a = make_args(x, w, s, b, y, N, K, bits, (int)M, plan, group_size);
    return launch(sym, dim3((unsigned)plan.blocks), dim3(plan.threads), (size_t)plan.x_lds_bytes, &a, stream);
}

// Declared here, defined after the entry points that use it.
agq_status moe_decode(const void *x, const uint32_t *w_gate, const void *s_gate, const void *b_gate,
                      const uint32_t *w_up, const void *s_up, const void *b_up, const uint32_t *w_down,
                      const void *s_down, const void *b_down, const uint32_t *experts, const float *weights,
                      void *y, void *workspace, int64_t workspace_bytes, int64_t T, int64_t k, int64_t E,
                      int64_t H, int64_t F, int bits, int group_size, void *stream, bool use_scratch);
// Non-null stand-in for the scratch pointer during the host checks.
const int kScratchStandIn = 0;

}  // namespace

extern "C" {

int agq_version(void) { return 100; }

const char *agq_status_str(agq_status status) {
    switch (status) {
        case AGQ_OK: return "AGQ_OK";
        case AGQ_EINVAL: return "AGQ_EINVAL";
        case AGQ_ENOTSUP: return "AGQ_ENOTSUP";
        case AGQ_EHIP: return "AGQ_EHIP";
    }
    return "AGQ_UNKNOWN";
}

const char *agq_last_error(void) { return g_err; }

agq_status agq_qmv(const void *x, const uint32_t *w, const void *scales, const void *biases, void *y, int64_t N,
                   int64_t K, int bits, int group_size, void *stream) {
    return dense_product(x, w, scales, biases, y, 1, N, K, bits, group_size, stream);
}

agq_status agq_qmv_wide(const void *x, const uint32_t *w, const void *scales, const void *biases, void *y,
                        int64_t M, int64_t N, int64_t K, int bits, int group_size, void *stream) {
    return dense_product(x, w, scales, biases, y, M, N, K, bits, group_size, stream);
}

agq_status agq_qmv_fused(const void *x, const void *norm_weight, float eps, const uint32_t *w, const void *scales,
                         const void *biases, const void *residual, int act, void *y, int64_t N, int64_t K, int bits,
                         int group_size, void *stream) {
    agq_status st = check_operands(x, w, scales, biases, y, N, K, bits, group_size, true);
    if (st != AGQ_OK) return st;
    st = need_4_or_8(bits, "the fused projection");
    if (st != AGQ_OK) return st;
    if (act < AGQ_ACT_NONE || act > AGQ_ACT_GEGLU) return fail(AGQ_EINVAL, "act=%d is not 0, 1 or 2", act);
    if (act != AGQ_ACT_NONE && (N % 2 != 0 || residual))
        return fail(AGQ_EINVAL, "a gated epilogue needs an even N (interleaved gate and up rows) and no residual");
    if (!(eps >= 0.f) || eps > 3.0e38f) return fail(AGQ_EINVAL, "eps must be finite and >= 0");
    if (misaligned(norm_weight, 16)) return fail(AGQ_EINVAL, "norm_weight must be 16-byte aligned");
    if (misaligned(residual, 2)) return fail(AGQ_EINVAL, "residual must be 2-byte aligned");
    if (N >= (int64_t(1) << 31)) return fail(AGQ_ENOTSUP, "N=%lld too large for the fused projection", (long long)N);
    // No stage to fuse: the plain batch-1 product.
    if (!norm_weight && !residual && act == AGQ_ACT_NONE)
        return dense_product(x, w, scales, biases, y, 1, N, K, bits, group_size, stream);
    const bool glu = act != AGQ_ACT_NONE;
    const bool norm = norm_weight != nullptr;
    const int epi = glu ? act : residual ? 0 : 3;
    agq::Plan plan;
    if (agq::plan_fused_shape(K, bits, &plan) != AGQ_OK)  // host-only check before any HIP call
        return fail(AGQ_ENOTSUP, "K=%lld too large for the fused projection at %d bits", (long long)K, bits);
    int cus = 0, dev = 0;
    st = current_device(&cus, &dev);
    if (st != AGQ_OK) return st;
    const void *sym = nullptr;
    for (int pass = 0; pass < 2; ++pass) {
        sym = agq::fused_kernel(bits, plan.cpt, plan.R, plan.NB, plan.x_lds_bytes > 0 ? plan.S : 0, epi, norm);
        if (!sym) return fail(AGQ_ENOTSUP, "no fused kernel for bits=%d cpt=%d R=%d", bits, plan.cpt, plan.R);
        int64_t waves = 0;
        st = resident_waves(sym, plan.threads, (size_t)plan.x_lds_bytes, cus, dev, &waves);
        if (st != AGQ_OK) return st;
        if (pass == 0 && agq::wants_deep(N, waves, plan.S, 0)) {
            agq::plan_fused_shape(K, bits, &plan, true);
            continue;
        }
        agq::plan_grid(N, waves, 0, &plan);
        break;
    }
    agq::FusedArgs f{};
    f.p = make_args(x, w, scales, biases, y, N, K, bits, 1, plan, group_size);
    f.gamma = static_cast<const uint16_t *>(norm_weight);
    f.res = static_cast<const uint16_t *>(residual);
    f.eps = eps;
    f.inv_k = 1.f / (float)K;
    return launch(sym, dim3((unsigned)plan.blocks), dim3(plan.threads), (size_t)plan.x_lds_bytes, &f, stream);
}

agq_status agq_qmv_nvfp4(const void *x, const uint32_t *w, const void *scales, float tensor_scale, void *y, int64_t M,
                         int64_t N, int64_t K, void *stream) {
    if (!x || !w || !scales || !y) return fail(AGQ_EINVAL, "null tensor pointer");
    if (M <= 0 || N <= 0 || K <= 0)
        return fail(AGQ_EINVAL, "M, N and K must be positive (M=%lld, N=%lld, K=%lld)", (long long)M, (long long)N,
                    (long long)K);
    if (N > kMaxN || K > kMaxK) return fail(AGQ_EINVAL, "N or K too large (N=%lld, K=%lld)", (long long)N, (long long)K);
    if (K % 16 != 0) return fail(AGQ_EINVAL, "K=%lld is not a multiple of the NVFP4 block of 16", (long long)K);
    if (K % 32 != 0) return fail(AGQ_ENOTSUP, "K=%lld: the NVFP4 kernel reads 32-code chunks", (long long)K);
    if (M > 4) return fail(AGQ_ENOTSUP, "M=%lld > 4 activation rows for the NVFP4 product", (long long)M);
    if (!(tensor_scale == tensor_scale) || tensor_scale > 3.0e38f || tensor_scale < -3.0e38f)
        return fail(AGQ_EINVAL, "tensor_scale must be finite");
    if (misaligned(x, 16) || misaligned(w, 16)) return fail(AGQ_EINVAL, "x and w must be 16-byte aligned");
    if (misaligned(scales, 2) || misaligned(y, 2)) return fail(AGQ_EINVAL, "scales and y must be 2-byte aligned");
    agq::Plan plan;
    if (agq::plan_shape(M, K, 4, 0, &plan) != AGQ_OK)  // host-only check before any HIP call
        return fail(AGQ_ENOTSUP, "K=%lld too large for M=%lld NVFP4 rows", (long long)K, (long long)M);
    int cus = 0, dev = 0;
    agq_status st = current_device(&cus, &dev);
    if (st != AGQ_OK) return st;
    if (M == 1 && K % 64 == 0 && !misaligned(scales, 4) &&
        (N + agq::kStreamRowsPerBlock - 1) / agq::kStreamRowsPerBlock >= 2 * (int64_t)cus) {
        // Large batch-1 grids: the bit-stream kernel's NVFP4 form, as for the
        // affine 4-bit products.
        agq::StreamArgs a{};
        a.x = static_cast<const uint16_t *>(x);
        a.w = w;
        a.s = static_cast<const uint16_t *>(scales);  // E4M3 bytes [N, K/16]
        a.y = static_cast<uint16_t *>(y);
        a.N = N;
        a.K = (int32_t)K;
        a.M = 1;
        a.ts = tensor_scale;
        return launch(agq::stream_nvfp4_kernel(),
                      dim3((unsigned)((N + agq::kStreamRowsPerBlock - 1) / agq::kStreamRowsPerBlock)), dim3(256), 0, &a,
                      stream);
    }
    const void *sym = nullptr;
    for (int pass = 0; pass < 2; ++pass) {
        sym = agq::nvfp4_kernel_for(plan.mw, plan.cpt, plan.R, plan.NB);
        if (!sym) return fail(AGQ_ENOTSUP, "no NVFP4 kernel for rows=%d cpt=%d R=%d", plan.mw, plan.cpt, plan.R);
        int64_t waves = 0;
        st = resident_waves(sym, plan.threads, 0, cus, dev, &waves);
        if (st != AGQ_OK) return st;
        if (pass == 0 && agq::wants_deep(N, waves, plan.S, 0)) {
            agq::plan_shape(M, K, 4, 0, &plan, true);
            continue;
        }
        agq::plan_grid(N, waves, 0, &plan);
        break;
    }
    agq::Nvfp4Args a{};
    a.x = static_cast<const uint16_t *>(x);
    a.w = reinterpret_cast<const agq::u32x4 *>(w);
    a.s = static_cast<const uint8_t *>(scales);
    a.y = static_cast<uint16_t *>(y);
    a.N = N;
    a.RPG = plan.RPG;
    a.K = (int32_t)K;
    a.C = (int32_t)(K / 32);
    a.S = plan.S;
    a.GPB = plan.GPB;
    a.ts = tensor_scale;
    return launch(sym, dim3((unsigned)plan.blocks), dim3(plan.threads), 0, &a, stream);
}

// Whether M > 4 rows of an NVFP4 product run faster as passes of 4 rows of the
// matvec kernel (each pass streams the weights once) than on the GEMM, whose
// blocks walk K one 64-column group at a time (about 0.6 us per group, latency-
// bound, when the grid is small). A pass costs about its weight bytes at 4.5 TB/s
// plus 3 us. Measured (us, GEMM / passes): 4096x4096 at M = 16 / 32: 37.9 / 22.3,
// 39.1 / 44.4; 28672x4096 at M = 8 / 16: 53.8 / 39.8, 52.8 / 77.3; 4096x14336 at
// M = 32 / 64: 138.5 / 99.5, 142.1 / 196.1.
// With a K split each block walks its split's groups, and the partials cost
// their bytes twice at 4 TB/s plus a launch.
bool nvfp4_passes_win(int64_t M, int64_t N, int64_t K, int cus, const agq::QmmKernel &k) {
    const double pass_us = (double)N * (double)K * 0.5625 / 4.5e6 + 3.0;
    const double passes_us = (double)((M + 3) / 4) * pass_us;
    const int64_t blocks = ((M + k.bm - 1) / k.bm) * ((N + k.bn - 1) / k.bn) * k.splits;
    const double groups = k.splits > 1 ? (double)k.gps : (double)(K / 64);
    const double reduce_us = k.splits > 1 ? 2.0 * (double)agq::qmm_split_bytes(k, M, N) / 4.0e6 + 3.0 : 0.0;
    const double gemm_us = groups * 0.6 * (double)((blocks + cus - 1) / cus) + reduce_us;
    return passes_us < gemm_us;
}

// Workspace checks of the GEMM entry points: NULL (no K split), or at least
// `need` bytes, 16-byte aligned.
agq_status check_workspace(const void *ws, int64_t ws_bytes, int64_t need) {
    if (!ws) return AGQ_OK;
    if (misaligned(ws, 16)) return fail(AGQ_EINVAL, "workspace must be 16-byte aligned");
    if (ws_bytes < need)
        return fail(AGQ_EINVAL, "workspace of %lld bytes is below the %lld this call needs", (long long)ws_bytes,
                    (long long)need);
    return AGQ_OK;
}

// The GEMM launch, then (with a K split) the reduction of the partials into y.
agq_status launch_qmm(const agq::QmmKernel &k, agq::QmmArgs &a, int64_t M, int64_t N, void *ws, int dev,
                      void *stream) {
    const int64_t mt = (M + k.bm - 1) / k.bm, nt = (N + k.bn - 1) / k.bn;
    agq_status st = allow_lds(k.sym, (size_t)k.lds, dev);
    if (st != AGQ_OK) return st;
    if (k.splits <= 1) {
        a.gps = a.G;
        return launch(k.sym, dim3((unsigned)nt, (unsigned)mt), dim3(k.threads), (size_t)k.lds, &a, stream);
    }
    a.part = static_cast<float *>(ws);
    a.gps = k.gps;
    st = launch(k.sym, dim3((unsigned)nt, (unsigned)mt, (unsigned)k.splits), dim3(k.threads), (size_t)k.lds, &a,
                stream);
    if (st != AGQ_OK) return st;
    int64_t MN = M * N;
    const float *part = a.part;
    uint16_t *y = a.y;
    int splits = k.splits;
    float ts = a.ts;
    void *args[] = {&part, &y, &MN, &splits, &ts};
    hipError_t e = hipLaunchKernel(agq::qmm_reduce_kernel(), dim3((unsigned)((MN + 1023) / 1024)), dim3(256), args, 0,
                                   static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(AGQ_EHIP, "kernel launch failed: %s", hipGetErrorString(e));
    return AGQ_OK;
}

// Whether an NVFP4 GEMM call takes the matrix-core kernels (else passes of the
// matvec kernel), and which, on `cus` compute units.
bool nvfp4_gemm_plan(int64_t M, int64_t N, int64_t K, int cus, bool split_ok, agq::QmmKernel *k) {
    *k = agq::qmm_nvfp4_kernel_for(M, N, K, cus, split_ok);
    return K % 64 == 0 && !nvfp4_passes_win(M, N, K, cus, *k);
}

int64_t agq_qmm_nvfp4_workspace(int64_t M, int64_t N, int64_t K) {
    if (M <= 4 || N <= 0 || K <= 0 || K % 32 != 0 || N > kMaxN || K > kMaxK) return 0;
    if (M * K * 2 >= (int64_t(1) << 31)) return 0;
    int cus = 0, dev = 0;
    if (current_device(&cus, &dev) != AGQ_OK) return 0;
    agq::QmmKernel k;
    return nvfp4_gemm_plan(M, N, K, cus, true, &k) ? agq::qmm_split_bytes(k, M, N) : 0;
}

agq_status agq_qmm_nvfp4(const void *x, const uint32_t *w, const void *scales, float tensor_scale, void *y, int64_t M,
                         int64_t N, int64_t K, void *workspace, int64_t workspace_bytes, void *stream) {
    if (M <= 4) return agq_qmv_nvfp4(x, w, scales, tensor_scale, y, M, N, K, stream);
    if (!x || !w || !scales || !y) return fail(AGQ_EINVAL, "null tensor pointer");
    if (workspace && misaligned(workspace, 16)) return fail(AGQ_EINVAL, "workspace must be 16-byte aligned");
    if (N <= 0 || K <= 0) return fail(AGQ_EINVAL, "N and K must be positive (N=%lld, K=%lld)", (long long)N, (long long)K);
    if (N > kMaxN || K > kMaxK) return fail(AGQ_EINVAL, "N or K too large (N=%lld, K=%lld)", (long long)N, (long long)K);
    if (K % 16 != 0) return fail(AGQ_EINVAL, "K=%lld is not a multiple of the NVFP4 block of 16", (long long)K);
    if (K % 32 != 0) return fail(AGQ_ENOTSUP, "K=%lld: the NVFP4 kernels read 32-code chunks", (long long)K);
    if (!(tensor_scale == tensor_scale) || tensor_scale > 3.0e38f || tensor_scale < -3.0e38f)
        return fail(AGQ_EINVAL, "tensor_scale must be finite");
    if (misaligned(x, 16) || misaligned(w, 16)) return fail(AGQ_EINVAL, "x and w must be 16-byte aligned");
    if (misaligned(scales, 2) || misaligned(y, 2)) return fail(AGQ_EINVAL, "scales and y must be 2-byte aligned");
    if (M * K * 2 >= (int64_t(1) << 31)) return fail(AGQ_ENOTSUP, "x must stay below 2 GiB (M*K*2 bytes)");
    if ((int64_t)agq::kQmmHlTileN * (K / 2) >= (int64_t(1) << 31)) return fail(AGQ_ENOTSUP, "K too large");
    if ((M + agq::kQmmTileMinM - 1) / agq::kQmmTileMinM > 65535 || (N + agq::kQmmHlTileN - 1) / agq::kQmmHlTileN > INT32_MAX)
        return fail(AGQ_ENOTSUP, "grid too large (M=%lld, N=%lld)", (long long)M, (long long)N);
    int cus = 0, dev = 0;
    agq_status st = current_device(&cus, &dev);
    if (st != AGQ_OK) return st;
    agq::QmmKernel k;
    if (!nvfp4_gemm_plan(M, N, K, cus, workspace != nullptr, &k)) {
        // Passes of up to 4 rows through the matvec kernel.
        for (int64_t r0 = 0; r0 < M; r0 += 4) {
            st = agq_qmv_nvfp4(static_cast<const uint16_t *>(x) + r0 * K, w, scales, tensor_scale,
                               static_cast<uint16_t *>(y) + r0 * N, M - r0 < 4 ? M - r0 : 4, N, K, stream);
            if (st != AGQ_OK) return st;
        }
        return AGQ_OK;
    }
    st = check_workspace(workspace, workspace_bytes, agq::qmm_split_bytes(k, M, N));
    if (st != AGQ_OK) return st;
    agq::QmmArgs a{};
    a.x = static_cast<const uint16_t *>(x);
    a.w = w;
    a.s = static_cast<const uint16_t *>(scales);  // scale bytes, addressed bytewise by the kernel
    a.y = static_cast<uint16_t *>(y);
    a.N = N;
    a.M = (int32_t)M;
    a.K = (int32_t)K;
    a.G = (int32_t)(K / 64);
    a.rowbytes = (int32_t)(K / 2);
    a.xbytes = (uint32_t)(M * K * 2);
    a.ts = tensor_scale;
    return launch_qmm(k, a, M, N, workspace, dev, stream);
}

// The expert gather at the bit-stream widths (agq_gather_qmv and
// agq_gather_qmm alike): one grid row per expert plane, whose pairs run as
// the activation rows of the matvec kernel, up to mw per pass (mw from the
// mean pairs per plane). Index arguments are checked by the callers.
agq_status stream_gather(const void *x, const uint32_t *w, const void *scales, const void *biases,
                         const uint32_t *lhs_indices, const uint32_t *rhs_indices, void *y, int64_t P, int64_t R,
                         int64_t E, int64_t N, int64_t K, int bits, int group_size, void *stream) {
    if (group_size != 64) return fail(AGQ_ENOTSUP, "bits=%d takes group size 64", bits);
    if (K * 2 >= (int64_t(1) << 31)) return fail(AGQ_ENOTSUP, "K too large");
    if ((N + agq::kStreamRowsPerBlock - 1) / agq::kStreamRowsPerBlock > INT32_MAX)
        return fail(AGQ_ENOTSUP, "N=%lld too large", (long long)N);
    agq::StreamArgs a{};
    a.x = static_cast<const uint16_t *>(x);
    a.w = w;
    a.s = static_cast<const uint16_t *>(scales);
    a.b = static_cast<const uint16_t *>(biases);
    a.y = static_cast<uint16_t *>(y);
    a.N = N;
    a.K = (int32_t)K;
    a.M = (int32_t)P;
    a.lhs = lhs_indices;
    a.rhs = rhs_indices;
    a.R_x = (int32_t)R;
    a.E = (int32_t)E;
    static_assert(agq::kMaxGatherPairs >= agq::kMaxPairs, "pair list");
    const int64_t per_plane = (P + E - 1) / E;
    const int mw = per_plane <= 1 ? 1 : per_plane <= 2 ? 2 : per_plane <= 4 ? 4 : 8;
    return launch(agq::stream_gather_kernel(bits, mw),
                  dim3((unsigned)((N + agq::kStreamRowsPerBlock - 1) / agq::kStreamRowsPerBlock), (unsigned)E),
                  dim3(256), 0, &a, stream);
}

agq_status agq_gather_qmv(const void *x, const uint32_t *w, const void *scales, const void *biases,
                          const uint32_t *lhs_indices, const uint32_t *rhs_indices, void *y, int64_t P, int64_t R,
                          int64_t E, int64_t N, int64_t K, int bits, int group_size, void *stream) {
    agq_status st = check_operands(x, w, scales, biases, y, N, K, bits, group_size, true);
    if (st != AGQ_OK) return st;
    if (P <= 0 || R <= 0 || E <= 0)
        return fail(AGQ_EINVAL, "P, R and E must be positive (P=%lld, R=%lld, E=%lld)", (long long)P,
                    (long long)R, (long long)E);
    if (!lhs_indices && R != P) return fail(AGQ_EINVAL, "lhs_indices == NULL requires R == P");
    if (!rhs_indices && E != P) return fail(AGQ_EINVAL, "rhs_indices == NULL requires E == P");
    if (misaligned(lhs_indices, 4) || misaligned(rhs_indices, 4))
        return fail(AGQ_EINVAL, "index arrays must be 4-byte aligned");
    if (P > agq::kMaxPairs) return fail(AGQ_ENOTSUP, "P=%lld pairs exceeds %d", (long long)P, agq::kMaxPairs);
    if (R > INT32_MAX) return fail(AGQ_EINVAL, "R too large");
    if (E > 65535) return fail(AGQ_ENOTSUP, "E=%lld expert planes exceeds 65535", (long long)E);
    if (E * N > kMaxN) return fail(AGQ_EINVAL, "E*N too large");
    if (stream_bits(bits))
        return stream_gather(x, w, scales, biases, lhs_indices, rhs_indices, y, P, R, E, N, K, bits, group_size,
                             stream);
    if (group_size == 64 && agq::mfma_eligible(8, K, bits, E, R)) {
        agq::MfmaPlan mp;
        const void *sym = nullptr;
        st = launch_mfma_plan(P, N, K, E, &mp, &sym);
        if (st != AGQ_OK) return st;
        agq::MfmaArgs a = make_mfma_args(x, w, scales, biases, y, N, K, (int)P, mp);
        a.lhs = lhs_indices;
        a.rhs = rhs_indices;
        a.R_x = (int32_t)R;
        a.E = (int32_t)E;
        return launch(sym, dim3((unsigned)mp.groups, (unsigned)E), dim3(mp.threads), (size_t)mp.lds_bytes, &a,
                      stream);
    }
    agq::Plan plan;
    if (agq::plan_shape(8, K, bits, E, &plan) != AGQ_OK)  // host-only check before any HIP call
        return fail(AGQ_ENOTSUP, "K=%lld too large for the gather at %d bits", (long long)K, bits);
    const void *sym = nullptr;
    st = launch_plan(8, N, K, bits, E, &plan, &sym);
    if (st != AGQ_OK) return st;
    agq::ProductArgs a = make_args(x, w, scales, biases, y, N, K, bits, (int)P, plan, group_size);
    a.lhs = lhs_indices;
    a.rhs = rhs_indices;
    a.R_x = (int32_t)R;
    a.E = (int32_t)E;
    return launch(sym, dim3((unsigned)plan.blocks, (unsigned)E), dim3(plan.threads), (size_t)plan.x_lds_bytes, &a,
                  stream);
}

// The GEMM of an agq_qmm call of M > 8 rows on `cus` compute units, or false
// for passes of the matrix-core matvec kernel: up to kQmmPassRows rows of its
// formats, unless more than kQmmHlSmallMinRows rows get split-weight tiles
// that fill the device.
bool qmm_gemm_plan(int64_t M, int64_t N, int64_t K, int bits, int cus, bool split_ok, agq::QmmKernel *k) {
    *k = agq::qmm_kernel_for(bits, false, M, N, K, 1, cus, split_ok);
    if (M <= agq::kQmmPassRows && agq::mfma_eligible(M, K, bits, 0, M))
        return M > agq::kQmmHlSmallMinRows && k->split_weight;
    return true;
}

// qmm at the bit-stream widths from this many rows, given a workspace: the
// codes widened to the 8-bit layout in the workspace, then the 8-bit GEMM.
// (Fewer rows: passes of 8 rows through the stream matvec, which read the
// stream codes once per pass, cost less than writing and reading N*K bytes.)
constexpr int64_t kStreamGemmMinRows = 64;

int64_t stream_codes_bytes(int64_t N, int64_t K) { return (N * K + 255) / 256 * 256; }

int64_t agq_qmm_workspace(int64_t M, int64_t N, int64_t K, int bits, int group_size) {
    if (stream_bits(bits)) {
        if (M < kStreamGemmMinRows || group_size != 64 || N <= 0 || K <= 0 || N > kMaxN || K > kMaxK ||
            K % 64 != 0 || M * K * 2 >= (int64_t(1) << 31) || (int64_t)agq::kQmmHlTileN * K >= (int64_t(1) << 31))
            return 0;
        return stream_codes_bytes(N, K) + agq_qmm_workspace(M, N, K, 8, 64);
    }
    if (M <= 8 || N <= 0 || K <= 0 || N > kMaxN || K > kMaxK || (bits != 4 && bits != 8) || group_size != 64)
        return 0;
    if (K % 64 != 0 || M * K * 2 >= (int64_t(1) << 31)) return 0;
    int cus = 0, dev = 0;
    if (current_device(&cus, &dev) != AGQ_OK) return 0;
    agq::QmmKernel k;
    return qmm_gemm_plan(M, N, K, bits, cus, true, &k) ? agq::qmm_split_bytes(k, M, N) : 0;
}

agq_status agq_qmm(const void *x, const uint32_t *w, const void *scales, const void *biases, void *y, int64_t M,
                   int64_t N, int64_t K, int bits, int group_size, void *workspace, int64_t workspace_bytes,
                   void *stream) {
    agq_status st = check_operands(x, w, scales, biases, y, N, K, bits, group_size, true);
    if (st != AGQ_OK) return st;
    if (workspace && misaligned(workspace, 16)) return fail(AGQ_EINVAL, "workspace must be 16-byte aligned");
    if (M <= 0) return fail(AGQ_EINVAL, "M must be positive (got %lld)", (long long)M);
    if (M * K * 2 >= (int64_t(1) << 31)) return fail(AGQ_ENOTSUP, "x must stay below 2 GiB (M*K*2 bytes)");
    // Up to 8 rows: the matvec kernels. Up to kQmmPassRows rows of 4-bit codes (K
    // a multiple of 512): the matrix-core matvec kernel, one grid row per pass of
    // 16 rows, unless (beyond kQmmHlSplitMinRows rows) the split-weight tiles
    // fill the device. Beyond: the tiled GEMM.
    if (M <= 8) return dense_product(x, w, scales, biases, y, M, N, K, bits, group_size, stream);
    if (stream_bits(bits)) {
        // With a workspace, from kStreamGemmMinRows rows: the codes widened to
        // 8 bits in the workspace, then the 8-bit GEMM (the rest of the
        // workspace serves its K split). Else passes of up to 8 rows through the
        // bit-stream matvec.
        const int64_t need = workspace ? agq_qmm_workspace(M, N, K, bits, group_size) : 0;
        if (need > 0) {
            st = check_workspace(workspace, workspace_bytes, need);
            if (st != AGQ_OK) return st;
            const uint32_t *src = w;
            uint32_t *codes8 = static_cast<uint32_t *>(workspace);
            int64_t units = N * K / 32;  // the kernel's three parameters, in order
            void *targs[] = {&src, &codes8, &units};
            const hipError_t e = hipLaunchKernel(agq::stream_to_u8_kernel(bits), dim3((unsigned)((units + 255) / 256)),
                                                 dim3(256), targs, 0, static_cast<hipStream_t>(stream));
            if (e != hipSuccess) return fail(AGQ_EHIP, "kernel launch failed: %s", hipGetErrorString(e));
            const int64_t cb = stream_codes_bytes(N, K);
            return agq_qmm(x, codes8, scales, biases, y, M, N, K, 8, 64, static_cast<char *>(workspace) + cb,
                           workspace_bytes - cb, stream);
        }
        for (int64_t r0 = 0; r0 < M; r0 += 8) {
            st = dense_product(static_cast<const uint16_t *>(x) + r0 * K, w, scales, biases,
                               static_cast<uint16_t *>(y) + r0 * N, M - r0 < 8 ? M - r0 : 8, N, K, bits, group_size,
                               stream);
            if (st != AGQ_OK) return st;
        }
        return AGQ_OK;
    }
    if (group_size != 64) return fail(AGQ_ENOTSUP, "qmm beyond 8 rows takes group size 64");
    const bool pass_ok = M <= agq::kQmmPassRows && agq::mfma_eligible(M, K, bits, 0, M);
    // (The GEMM: the weight range for the widest tile; the grid for the smallest.)
    const bool k_ok = (int64_t)agq::kQmmHlTileN * (K * bits / 8) < (int64_t(1) << 31);
    const bool grid_ok = (M + agq::kQmmTileMinM - 1) / agq::kQmmTileMinM <= 65535 &&
                         (N + agq::kQmmTileN - 1) / agq::kQmmTileN <= INT32_MAX;
    if (!pass_ok && !k_ok) return fail(AGQ_ENOTSUP, "K too large");
    if (!pass_ok && !grid_ok)
        return fail(AGQ_ENOTSUP, "grid too large (M=%lld, N=%lld)", (long long)M, (long long)N);
    int cus = 0, dev = 0;
    st = current_device(&cus, &dev);
    if (st != AGQ_OK) return st;
    agq::QmmKernel k;
    if (!(k_ok && grid_ok && qmm_gemm_plan(M, N, K, bits, cus, workspace != nullptr, &k))) {
        agq::MfmaPlan mp;
        const void *sym = nullptr;
        const int passes = (int)((M + 15) / 16);
        st = launch_mfma_plan(M, N, K, 0, &mp, &sym, passes);
        if (st != AGQ_OK) return st;
        agq::MfmaArgs a = make_mfma_args(x, w, scales, biases, y, N, K, (int)M, mp);
        return launch(sym, dim3((unsigned)mp.groups, (unsigned)passes), dim3(mp.threads), (size_t)mp.lds_bytes, &a,
                      stream);
    }
    st = check_workspace(workspace, workspace_bytes, agq::qmm_split_bytes(k, M, N));
    if (st != AGQ_OK) return st;
    agq::QmmArgs a{};
    a.x = static_cast<const uint16_t *>(x);
    a.w = w;
    a.s = static_cast<const uint16_t *>(scales);
    a.b = static_cast<const uint16_t *>(biases);
    a.y = static_cast<uint16_t *>(y);
    a.N = N;
    a.M = (int32_t)M;
    a.K = (int32_t)K;
    a.G = (int32_t)(K / 64);
    a.rowbytes = (int32_t)(K * bits / 8);
    a.xbytes = (uint32_t)(M * K * 2);
    a.ts = 1.0f;
    return launch_qmm(k, a, M, N, workspace, dev, stream);
}

agq_status agq_gather_qmm(const void *x, const uint32_t *w, const void *scales, const void *biases,
                          const uint32_t *lhs_indices, const uint32_t *rhs_indices, void *y, int64_t P, int64_t R,
                          int64_t E, int64_t N, int64_t K, int bits, int group_size, void *stream) {
    agq_status st = check_operands(x, w, scales, biases, y, N, K, bits, group_size, true);
    if (st != AGQ_OK) return st;
    if (P <= 0 || R <= 0 || E <= 0)
        return fail(AGQ_EINVAL, "P, R and E must be positive (P=%lld, R=%lld, E=%lld)", (long long)P,
                    (long long)R, (long long)E);
    if (!lhs_indices && R != P) return fail(AGQ_EINVAL, "lhs_indices == NULL requires R == P");
    if (!rhs_indices && E != P) return fail(AGQ_EINVAL, "rhs_indices == NULL requires E == P");
    if (misaligned(lhs_indices, 4) || misaligned(rhs_indices, 4))
        return fail(AGQ_EINVAL, "index arrays must be 4-byte aligned");
    if (P > agq::kMaxPairs) return fail(AGQ_ENOTSUP, "P=%lld pairs exceeds %d", (long long)P, agq::kMaxPairs);
    if (E > 65535) return fail(AGQ_ENOTSUP, "E=%lld expert planes exceeds 65535", (long long)E);
    if (E * N > kMaxN) return fail(AGQ_EINVAL, "E*N too large");
    if (R > INT32_MAX) return fail(AGQ_EINVAL, "R too large");
    if (stream_bits(bits))
        return stream_gather(x, w, scales, biases, lhs_indices, rhs_indices, y, P, R, E, N, K, bits, group_size,
                             stream);
    if (R * K * 2 >= (int64_t(1) << 31)) return fail(AGQ_ENOTSUP, "x must stay below 2 GiB (R*K*2 bytes)");
    if (group_size != 64) return fail(AGQ_ENOTSUP, "gather_qmm takes group size 64");
    if ((int64_t)agq::kQmmHlTileN * (K * bits / 8) >= (int64_t(1) << 31)) return fail(AGQ_ENOTSUP, "K too large");
    if ((N + agq::kQmmTileN - 1) / agq::kQmmTileN > INT32_MAX) return fail(AGQ_ENOTSUP, "N too large");
    int cus = 0, dev = 0;
    st = current_device(&cus, &dev);
    if (st != AGQ_OK) return st;
    const agq::QmmKernel k = agq::qmm_kernel_for(bits, true, (P + E - 1) / E, N, K, E, cus, false);
    const int64_t nt = (N + k.bn - 1) / k.bn;
    agq::QmmArgs a{};
    a.x = static_cast<const uint16_t *>(x);
    a.w = w;
    a.s = static_cast<const uint16_t *>(scales);
    a.b = static_cast<const uint16_t *>(biases);
    a.y = static_cast<uint16_t *>(y);
    a.lhs = lhs_indices;
    a.rhs = rhs_indices;
    a.N = N;
    a.M = (int32_t)P;
    a.K = (int32_t)K;
    a.G = (int32_t)(K / 64);
    a.rowbytes = (int32_t)(K * bits / 8);
    a.xbytes = (uint32_t)(R * K * 2);
    a.R_x = (int32_t)R;
    a.E = (int32_t)E;
    a.gps = a.G;
    const size_t lds = (size_t)k.lds + (size_t)((P * 2 + 15) / 16 * 16 + P * 4);
    st = allow_lds(k.sym, lds, dev);
    if (st != AGQ_OK) return st;
    return launch(k.sym, dim3((unsigned)nt, (unsigned)E), dim3(k.threads), lds, &a, stream);
}

int64_t agq_moe_decode_workspace(int64_t T, int64_t k, int64_t H, int64_t F) {
    if (T <= 0 || k <= 0 || H <= 0 || F <= 0) return 0;
    return 4 * T * k * F + 4 * T * k * H;  // per pair: two bf16 rows of F (h), one fp32 row of H (o)
}

agq_status agq_moe_decode(const void *x, const uint32_t *w_gate, const void *s_gate, const void *b_gate,
                          const uint32_t *w_up, const void *s_up, const void *b_up, const uint32_t *w_down,
                          const void *s_down, const void *b_down, const uint32_t *experts, const float *weights,
                          void *y, void *workspace, int64_t workspace_bytes, int64_t T, int64_t k, int64_t E,
                          int64_t H, int64_t F, int bits, int group_size, void *stream) {
    return moe_decode(x, w_gate, s_gate, b_gate, w_up, s_up, b_up, w_down, s_down, b_down, experts, weights, y,
                      workspace, workspace_bytes, T, k, E, H, F, bits, group_size, stream, false);
}

agq_status agq_moe_decode_noalloc(const void *x, const uint32_t *w_gate, const void *s_gate, const void *b_gate,
                                  const uint32_t *w_up, const void *s_up, const void *b_up, const uint32_t *w_down,
                                  const void *s_down, const void *b_down, const uint32_t *experts,
                                  const float *weights, void *y, int64_t T, int64_t k, int64_t E, int64_t H,
                                  int64_t F, int bits, int group_size, void *stream) {
    // The workspace pointer is filled in from the device's scratch array once
    // every host check has passed (a non-null stand-in passes the null check).
    return moe_decode(x, w_gate, s_gate, b_gate, w_up, s_up, b_up, w_down, s_down, b_down, experts, weights, y,
                      const_cast<int *>(&kScratchStandIn), agq::kMoeScratchBytes, T, k, E, H, F, bits, group_size,
                      stream, true);
}

}  // extern "C"

namespace {

agq_status moe_decode(const void *x, const uint32_t *w_gate, const void *s_gate, const void *b_gate,
                      const uint32_t *w_up, const void *s_up, const void *b_up, const uint32_t *w_down,
                      const void *s_down, const void *b_down, const uint32_t *experts, const float *weights,
                      void *y, void *workspace, int64_t workspace_bytes, int64_t T, int64_t k, int64_t E,
                      int64_t H, int64_t F, int bits, int group_size, void *stream, bool use_scratch) {
    if (!x || !w_gate || !s_gate || !b_gate || !w_up || !s_up || !b_up || !w_down || !s_down || !b_down || !experts ||
        !weights || !y || !workspace)
        return fail(AGQ_EINVAL, "null pointer");
    if (T <= 0 || k <= 0 || E <= 0 || H <= 0 || F <= 0)
        return fail(AGQ_EINVAL, "T, k, E, H and F must be positive");
    agq_status st = check_format(F, H, bits, group_size);
    if (st != AGQ_OK) return st;
    st = check_format(H, F, bits, group_size);
    if (st != AGQ_OK) return st;
    if (misaligned(x, 16) || misaligned(w_gate, 16) || misaligned(w_up, 16) || misaligned(w_down, 16) ||
        (!use_scratch && misaligned(workspace, 16)))
        return fail(AGQ_EINVAL, "x, the code planes and the workspace must be 16-byte aligned");
    if (misaligned(s_gate, 2) || misaligned(b_gate, 2) || misaligned(s_up, 2) || misaligned(b_up, 2) ||
        misaligned(s_down, 2) || misaligned(b_down, 2) || misaligned(y, 2) || misaligned(experts, 4) ||
        misaligned(weights, 4))
        return fail(AGQ_EINVAL, "misaligned scales, biases, y, experts or weights");
    if (bits != 4 || group_size != 64 || H % 512 != 0 || F % 512 != 0)
        return fail(AGQ_ENOTSUP, "the fused MoE takes 4-bit codes, group size 64, H and F multiples of 512");
    if (T > agq::kMoeMaxTokens) return fail(AGQ_ENOTSUP, "T=%lld tokens exceeds %d", (long long)T, agq::kMoeMaxTokens);
    const int64_t P = T * k;
    if (P > agq::kMaxPairs) return fail(AGQ_ENOTSUP, "T*k=%lld pairs exceeds %d", (long long)P, agq::kMaxPairs);
    if (E > 65535) return fail(AGQ_ENOTSUP, "E=%lld expert planes exceeds 65535", (long long)E);
    if (E * (H > F ? H : F) > kMaxN) return fail(AGQ_EINVAL, "E*H or E*F too large");
    if (2 * P * F * 2 >= (int64_t(1) << 32) || T * H * 2 >= (int64_t(1) << 31) || P * H * 4 >= (int64_t(1) << 40))
        return fail(AGQ_ENOTSUP, "activations too large");
    if (workspace_bytes < agq_moe_decode_workspace(T, k, H, F)) {
        if (use_scratch)
            return fail(AGQ_ENOTSUP, "T*k*F needs %lld bytes of scratch; the allocation-free call holds %lld",
                        (long long)agq_moe_decode_workspace(T, k, H, F), (long long)workspace_bytes);
        return fail(AGQ_EINVAL, "workspace of %lld bytes is below the %lld needed", (long long)workspace_bytes,
                    (long long)agq_moe_decode_workspace(T, k, H, F));
    }
    int cus = 0, dev = 0;
    st = current_device(&cus, &dev);
    if (st != AGQ_OK) return st;
    if (use_scratch) {
        hipError_t e = agq::moe_scratch(dev, &workspace);
        if (e != hipSuccess)
            return fail(AGQ_EHIP, "scratch address of device %d: %s", dev, hipGetErrorString(e));
    }
    agq::MoeArgs a{};
    a.x = static_cast<const uint16_t *>(x);
    a.h = static_cast<uint16_t *>(workspace);
    a.y = static_cast<uint16_t *>(y);
    a.wg = w_gate;
    a.sg = static_cast<const uint16_t *>(s_gate);
    a.bg = static_cast<const uint16_t *>(b_gate);
    a.wu = w_up;
    a.su = static_cast<const uint16_t *>(s_up);
    a.bu = static_cast<const uint16_t *>(b_up);
    a.wd = w_down;
    a.sd = static_cast<const uint16_t *>(s_down);
    a.bd = static_cast<const uint16_t *>(b_down);
    a.experts = experts;
    a.weights = weights;
    a.T = (int32_t)T;
    a.k = (int32_t)k;
    a.P = (int32_t)P;
    a.E = (int32_t)E;
    a.H = H;
    a.F = F;
    // Launch 1: dual bands of 16 units, K = H split over at most 2 waves, the
    // grid oversubscribed like the gather's.
    const int b4h = (int)(H / 512);
    a.S1 = b4h % 2 == 0 ? 2 : 1;
    a.SPW1 = (int)(H / 128) / a.S1;
    const int64_t bands1 = (F + 15) / 16;
    const void *k1 = agq::moe_kernel(0, 0);
    const size_t lds1 = (size_t)((P * 2 + 15) / 16 * 16 + P * 4);
    int64_t waves1 = 0;
    st = resident_waves(k1, 64 * a.S1, lds1, cus, dev, &waves1);
    if (st != AGQ_OK) return st;
    int64_t budget = waves1 * agq::kGatherOversub / a.S1 / E;
    if (budget < 1) budget = 1;
    a.BPG1 = (int32_t)((bands1 + budget - 1) / budget);
    const int64_t groups1 = (bands1 + a.BPG1 - 1) / a.BPG1;
    // Launch 2: the down projection's gather, bands of 32 output rows when they
    // give one band-wave per SIMD or more, K = F split over at most 2 waves.
    a.o = reinterpret_cast<float *>(static_cast<uint8_t *>(workspace) + 4 * P * F);
    const int b4f = (int)(F / 512);
    a.S2 = b4f % 2 == 0 ? 2 : 1;
    a.SPW2 = (int)(F / 128) / a.S2;
    const int tiles2 = ((H + 31) / 32) * a.S2 * E >= 1024 ? 2 : 1;
    const int64_t bands2 = (H + 16 * tiles2 - 1) / (16 * tiles2);
    const void *k2 = agq::moe_kernel(1, tiles2);
    const size_t lds2 = (size_t)((P * 2 + 15) / 16 * 16);
    int64_t waves2 = 0;
    st = resident_waves(k2, 64 * a.S2, lds2, cus, dev, &waves2);
    if (st != AGQ_OK) return st;
    budget = waves2 * agq::kGatherOversub / a.S2 / E;
    if (budget < 1) budget = 1;
    a.BPG2 = (int32_t)((bands2 + budget - 1) / budget);
    const int64_t groups2 = (bands2 + a.BPG2 - 1) / a.BPG2;
    // Launch 3: the slot sum, one thread per output.
    const void *k3 = agq::moe_kernel(2, 0);
    int64_t blocks3 = (T * H + 255) / 256;
    if (blocks3 > (int64_t)cus * 8) blocks3 = (int64_t)cus * 8;
    st = launch(k1, dim3((unsigned)groups1, (unsigned)E), dim3(64 * a.S1), lds1, &a, stream);
    if (st != AGQ_OK) return st;
    st = launch(k2, dim3((unsigned)groups2, (unsigned)E), dim3(64 * a.S2), lds2, &a, stream);
    if (st != AGQ_OK) return st;
    return launch(k3, dim3((unsigned)blocks3), dim3(256), 0, &a, stream);
}

}  // namespace

extern "C" {

agq_status agq_quantize(const void *w, int w_dtype, uint32_t *codes, void *scales, void *biases, int64_t rows,
                        int64_t K, int bits, int group_size, void *stream) {
    if (!w || !codes || !scales || !biases) return fail(AGQ_EINVAL, "null tensor pointer");
    if (w_dtype != AGQ_DTYPE_F32 && w_dtype != AGQ_DTYPE_BF16)
        return fail(AGQ_EINVAL, "w_dtype must be AGQ_DTYPE_F32 or AGQ_DTYPE_BF16 (got %d)", w_dtype);
    agq_status st = check_format(rows, K, bits, group_size);
    if (st != AGQ_OK) return st;
    if (misaligned(w, w_dtype == AGQ_DTYPE_F32 ? 4 : 2) || misaligned(codes, 4) || misaligned(scales, 2) ||
        misaligned(biases, 2))
        return fail(AGQ_EINVAL, "misaligned tensor pointer");
    int cus = 0, dev = 0;
    st = current_device(&cus, &dev);
    if (st != AGQ_OK) return st;
    int64_t groups = rows * (K / group_size);
    int64_t blocks = (groups + 255) / 256;
    if (blocks > (int64_t)cus * 16) blocks = (int64_t)cus * 16;
    int gsi = group_size;
    void *args[] = {&w, &groups, &K, &gsi, &codes, &scales, &biases};
    hipError_t e = hipLaunchKernel(agq::quantize_kernel_for(bits, w_dtype == AGQ_DTYPE_BF16), dim3((unsigned)blocks),
                                   dim3(256), args, 0, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(AGQ_EHIP, "kernel launch failed: %s", hipGetErrorString(e));
    return AGQ_OK;
}

agq_status agq_dequantize(const uint32_t *w, const void *scales, const void *biases, float *out, int64_t rows,
                          int64_t K, int bits, int group_size, void *stream) {
    agq_status st = check_operands(nullptr, w, scales, biases, out, rows, K, bits, group_size, false);
    if (st != AGQ_OK) return st;
    if (misaligned(out, 16)) return fail(AGQ_EINVAL, "out must be 16-byte aligned");
    int cus = 0, dev = 0;
    st = current_device(&cus, &dev);
    if (st != AGQ_OK) return st;
    // One thread per packed word (4 and 8 bits) or per 32 codes (the bit-stream widths).
    const bool streamed = stream_bits(bits);
    int64_t per_row = streamed ? K / 32 : K * bits / 32;
    int64_t units = rows * per_row;
    int64_t blocks = (units + 255) / 256;
    int64_t cap = (int64_t)cus * 32;
    if (blocks > cap) blocks = cap;
    const void *sym = streamed ? agq::stream_dequant_kernel(bits) : agq::dequant_kernel_sym(bits);
    int64_t gs = group_size;
    void *args[] = {&w, &scales, &biases, &out, &units, &per_row, &K, &gs};
    hipError_t e = hipLaunchKernel(sym, dim3((unsigned)blocks), dim3(256), args, 0, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(AGQ_EHIP, "kernel launch failed: %s", hipGetErrorString(e));
    return AGQ_OK;
}

agq_status agq_plan_product(int64_t M, int64_t N, int64_t K, int bits, int group_size, int num_cus,
                            int waves_per_cu, int64_t experts, agq_plan *out) {
    if (!out) return fail(AGQ_EINVAL, "null plan pointer");
    if (bits == 2 || bits == 3 || bits == 5 || bits == 6) return need_4_or_8(bits, "a launch plan");
    agq_status st = check_format(N, K, bits, group_size);
    if (st != AGQ_OK) return st;
    if (experts < 0) return fail(AGQ_EINVAL, "experts must be >= 0");
    if (experts == 0 && M <= 0) return fail(AGQ_EINVAL, "M must be positive");
    if (experts == 0 && M > 8) return fail(AGQ_ENOTSUP, "M > 8");
    if (num_cus <= 0 || waves_per_cu <= 0) return fail(AGQ_EINVAL, "num_cus and waves_per_cu must be positive");
    if (stream4(M, N, bits, group_size, experts, num_cus)) {
        export_stream_plan(N, K, bits, (int64_t)num_cus * waves_per_cu, out);
        return AGQ_OK;
    }
    if (group_size == 64 && agq::mfma_eligible(M, K, bits, experts, experts ? 1 : M)) {
        agq::MfmaPlan mp;
        agq::mfma_shape(N, K, experts, &mp);
        agq::mfma_lds(experts, 32, &mp);  // (gather plans assume 32 pairs)
        agq::mfma_grid((int64_t)num_cus * waves_per_cu, experts, &mp);
        export_mfma_plan(mp, K, out);
        return AGQ_OK;
    }
    agq::Plan p;
    if (agq::make_plan(experts ? agq::kGatherMW : M, N, K, bits, (int64_t)num_cus * waves_per_cu, experts, &p) !=
        AGQ_OK)
        return fail(AGQ_ENOTSUP, "K too large");
    export_plan(p, out);
    return AGQ_OK;
}

agq_status agq_plan_launch(int64_t M, int64_t N, int64_t K, int bits, int group_size, int64_t experts,
                           agq_plan *out) {
    if (!out) return fail(AGQ_EINVAL, "null plan pointer");
    if (bits == 2 || bits == 3 || bits == 5 || bits == 6) return need_4_or_8(bits, "a launch plan");
    agq_status st = check_format(N, K, bits, group_size);
    if (st != AGQ_OK) return st;
    if (experts < 0) return fail(AGQ_EINVAL, "experts must be >= 0");
    if (experts == 0 && M <= 0) return fail(AGQ_EINVAL, "M must be positive");
    if (experts == 0 && M > 8) return fail(AGQ_ENOTSUP, "M > 8");
    if (bits == 4 && group_size == 64 && M == 1 && experts == 0) {
        int cus = 0, dev = 0;
        st = current_device(&cus, &dev);
        if (st != AGQ_OK) return st;
        if (stream4(M, N, bits, group_size, experts, cus)) {
            int64_t resident = 0;
            st = resident_waves(agq::stream_kernel(4, 1), 256, 0, cus, dev, &resident);
            if (st != AGQ_OK) return st;
            export_stream_plan(N, K, bits, resident, out);
            return AGQ_OK;
        }
    }
    if (group_size == 64 && agq::mfma_eligible(M, K, bits, experts, experts ? 1 : M)) {
        agq::MfmaPlan mp;
        const void *sym = nullptr;
        st = launch_mfma_plan(M, N, K, experts, &mp, &sym);
        if (st != AGQ_OK) return st;
        export_mfma_plan(mp, K, out);
        return AGQ_OK;
    }
    agq::Plan p;
    const void *sym = nullptr;
    st = launch_plan(M, N, K, bits, experts, &p, &sym);
    if (st != AGQ_OK) return st;
    export_plan(p, out);
    return AGQ_OK;
}

}  // extern "C"
