/*
 * agq.h: C ABI of libagq, the affine group-quantized matrix-vector product
 * for AMD Instinct MI355X (gfx950).
 *
 * What it computes. An activation row x (BF16) multiplies a weight matrix W
 * stored as U32-packed affine codes with BF16 per-group scales and biases.
 * This is the operand triple named in "MLX CUDA Cleanup Plan", Target
 * Architecture §1, with its rank-2 and rank-3-plane forms. Refactor Plan
 * Phase 3 of that page fixes the formats: BF16 inputs, 4-bit or 8-bit codes,
 * group size 64. For output row n:
 *
 *     y[m, n] = sum_k x[m, k] * (scale[n, k/64] * q[n, k] + bias[n, k/64])
 *
 * Code q[n, k] is stored low-first: it is bits [bits*k, bits*k + bits) of
 * packed row n's little-endian bit stream, word i holding stream bits
 * 32i .. 32i + 31. For 4 and 8 bits (and 2) that is bits
 * [bits*(k % (32/bits)), +bits) of word k / (32/bits). The other widths of the
 * affine family, 2, 3, 5 and 6 bits, use the same stream (a 3-, 5- or 6-bit
 * code may run into the next word; a 64-column group is 2*bits words); the
 * pages name 4 and 8. W is [N out, K in]. Arithmetic is in fp32, and outputs
 * are BF16, rounded to nearest even.
 *
 * The product entry points map to the kernels those pages discuss:
 *  - agq_qmv is the batch-1 matvec;
 *  - agq_qmv_wide is the small-batch "qmv_wide" / multirow variant for
 *    M*B > 1, named in "epic: CUDA (MLX backend) prefill and decode
 *    acceleration program", Code-audit findings, and in the post-reboot
 *    re-measurement pasted into mlxcel PR #727;
 *  - agq_gather_qmv is the expert-gathered (MoE) form of the gather_qmm path
 *    in the same epic;
 *  - agq_qmm and agq_gather_qmm are the matrix-matrix (prefill) forms of the
 *    two;
 *  - agq_moe_decode is a whole decode MoE layer (gate, up, SwiGLU, down and
 *    the router-weighted sum) in three launches.
 *
 * Conventions shared by every entry point:
 *  - Tensor pointers are DEVICE pointers to contiguous row-major arrays. The
 *    caller owns them; they must stay valid until the work queued on
 *    `stream` completes. Outputs must not overlap inputs.
 *  - `stream` is a hipStream_t (NULL = the null stream). Each call queues
 *    its kernels on that stream and returns at once. It never synchronizes,
 *    allocates or copies; scratch memory, where a call needs it, is a
 *    workspace the caller passes in. The current HIP device must be the one that holds
 *    the buffers.
 *  - BF16 tensors are passed as `const void *` and hold raw bfloat16 bit
 *    patterns.
 *  - Alignment: x and w 16 bytes; scales, biases and y 2 bytes; indices 4 bytes.
 *  - Every argument check runs on the host before any HIP call, so a
 *    rejected call touches no device state. AGQ_EINVAL means malformed
 *    arguments. AGQ_ENOTSUP means well-formed but outside what this library
 *    implements (including a current device other than gfx950); this is a
 *    decline with no fallback path. AGQ_EHIP means the HIP runtime failed (no
 *    device, or a launch error). agq_last_error() then holds a message for
 *    the calling thread.
 *  - Calls are reentrant and keep no state between calls besides a cached
 *    per-device property record.
 */
#ifndef AGQ_H
#define AGQ_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum agq_status {
    AGQ_OK = 0,
    AGQ_EINVAL = 1,
    AGQ_ENOTSUP = 2,
    AGQ_EHIP = 3
} agq_status;

/* Library ABI version (major*10000 + minor*100 + patch). */
int agq_version(void);

/*
 * Status handling. "MLX CUDA Cleanup Plan", Target Architecture §4, keeps the
 * runtime-facing layer to small safe wrappers for status handling, streams
 * and memory; these two calls are that wrapper here.
 * agq_status_str: human-readable name of a status code (a static string).
 * agq_last_error: detail message of the last non-OK status returned on the
 * calling thread ("" if none); valid until the thread's next failing call.
 */
const char *agq_status_str(agq_status status);
const char *agq_last_error(void);

/*
 * Batch-1 matvec: y[n] = sum_k x[k] * w_hat[n, k].
 *   x      [K] BF16
 *   w      [N, K*bits/32] U32 packed codes
 *   scales [N, K/group_size] BF16
 *   biases [N, K/group_size] BF16
 *   y      [N] BF16 (written)
 * bits must be 2, 3, 4, 5, 6 or 8 and group_size 32, 64 or 128 (else
 * AGQ_ENOTSUP; the bit-stream widths 2, 3, 5 and 6 take group size 64 only);
 * K must be a positive multiple of group_size, and N positive (else
 * AGQ_EINVAL). K above 114688 (4-bit) or 57344 (8-bit) is AGQ_ENOTSUP; the
 * bit-stream widths walk K in chunks of 4096 columns and take any K with
 * M*K*2 < 2^31 bytes of x. 4-bit products with group size 64 whose N gives
 * at least two 16-row blocks per compute unit run on the bit-stream kernel
 * (the plan's engine 2), under the same 4-bit K limit.
 */
agq_status agq_qmv(const void *x, const uint32_t *w, const void *scales, const void *biases,
                   void *y, int64_t N, int64_t K, int bits, int group_size, void *stream);

/*
 * Small-batch matvec ("qmv_wide"): y[m, n] = sum_k x[m, k] * w_hat[n, k] for
 * 1 <= M <= 8 activation rows, streaming each weight byte once for all M rows.
 *   x [M, K] BF16, y [M, N] BF16; w, scales and biases as in agq_qmv.
 * M > 8 is AGQ_ENOTSUP; that is a quantized GEMM, not a matvec. With 4-bit
 * codes, group size 64, M >= 4 and K a multiple of 512 the product runs on
 * the matrix cores and K is limited only by M*K*2 < 2^31 bytes of x. Otherwise the K limit
 * shrinks with M: K <= 16384 * c for 4-bit and 8192 * c for 8-bit, with
 * c = min(7, floor(8/M)) (larger K is AGQ_ENOTSUP). The bit-stream widths as
 * for agq_qmv.
 */
agq_status agq_qmv_wide(const void *x, const uint32_t *w, const void *scales, const void *biases,
                        void *y, int64_t M, int64_t N, int64_t K, int bits, int group_size,
                        void *stream);

/*
 * Expert-gathered matvec for MoE decode. For each (token, expert) pair p:
 *     y[p, n] = sum_k x[lhs[p], k] * w_hat[rhs[p]][n, k]
 *   x       [R, K] BF16 activation rows
 *   w       [E, N, K*bits/32] U32, stacked expert planes
 *   scales  [E, N, K/group_size] BF16; biases the same
 *   lhs_indices [P] uint32 row of x per pair. NULL means lhs[p] = p and requires R == P.
 *   rhs_indices [P] uint32 expert per pair. NULL means rhs[p] = p and requires E == P.
 *   y       [P, N] BF16 (written)
 * Each expert plane that some pair uses is streamed from memory once for all
 * of its pairs. Unused planes are never read. No router weighting and no sum
 * over the top-k slots is applied. P may be at most 4096. Index values are
 * device data and cannot be checked on the host. A pair whose lhs >= R or
 * rhs >= E gets an all-NaN output row, and no memory outside the arrays is
 * read. With 4-bit codes, group size 64 and K a multiple of 512 the gather
 * runs on the matrix cores, 16 pairs per pass, and K is limited only by R*K*2 < 2^31
 * bytes of x; otherwise K limits are those of agq_qmv_wide at M = 8. At the
 * bit-stream widths (2, 3, 5, 6 bits; group size 64, else AGQ_ENOTSUP) the
 * pairs of each used plane run as the activation rows of the bit-stream
 * matvec, up to 1, 2, 4 or 8 per pass (from the mean pairs per plane, P/E),
 * so a plane streams once per pass. agq_gather_qmm takes the same forms.
 */
agq_status agq_gather_qmv(const void *x, const uint32_t *w, const void *scales, const void *biases,
                          const uint32_t *lhs_indices, const uint32_t *rhs_indices, void *y,
                          int64_t P, int64_t R, int64_t E, int64_t N, int64_t K,
                          int bits, int group_size, void *stream);

/*
 * Quantized matrix-matrix product ("qmm", the prefill form): for any M >= 1,
 *     y[m, n] = sum_k x[m, k] * w_hat[n, k]
 *   x [M, K] BF16, y [M, N] BF16; w, scales and biases as in agq_qmv.
 * The quantized GEMM that "epic: CUDA (MLX backend) prefill and decode
 * acceleration program", Code-audit findings, names beside qmv_wide (its
 * JIT-compiled qmm), and that Phase 6 of that epic (#637, quantized GEMM for
 * prefill) plans. It runs on the matrix cores with bfloat16 operands that
 * hold the codes exactly (128 + q for 4-bit, q for 8-bit) and applies each
 * group's scale and bias in fp32, so its error bound is that of the matvec
 * forms. M*K*2 must stay below 2^31 (else AGQ_ENOTSUP). Beyond 8 rows it
 * takes group size 64 (else AGQ_ENOTSUP). The bit-stream widths (2, 3, 5, 6
 * bits) run as passes of up to 8 rows of agq_qmv_wide's kernel; from 64 rows,
 * given a workspace, the codes are first widened to the 8-bit layout in the
 * workspace (N*K bytes, every code value kept) and the 8-bit GEMM runs on them
 * with the same scales and biases. Argument checks and errors as for agq_qmv.
 *
 * workspace (optional, owned by the caller): device scratch for a K split,
 * and at the bit-stream widths for the widened codes.
 * Where the output tiles alone leave compute units idle (a few hundred rows
 * against a few thousand weight rows), the tiles split K and write fp32
 * partial sums to the workspace, and a second launch on `stream` adds the
 * splits in a fixed order and rounds once to bf16, so results stay bitwise
 * deterministic (they differ from the unsplit kernels' only in fp32 rounding
 * order). NULL runs without a split. A non-NULL workspace must be 16-byte
 * aligned and hold at least agq_qmm_workspace(M, N, K, bits, group_size)
 * bytes (else AGQ_EINVAL); its contents on return are unspecified, and two
 * calls that overlap in time must not share one.
 */
int64_t agq_qmm_workspace(int64_t M, int64_t N, int64_t K, int bits, int group_size);
agq_status agq_qmm(const void *x, const uint32_t *w, const void *scales, const void *biases, void *y,
                   int64_t M, int64_t N, int64_t K, int bits, int group_size,
                   void *workspace, int64_t workspace_bytes, void *stream);

/*
 * Fused batch-1 projection: the decode layer's neighbouring stages that "MLX
 * CUDA Cleanup Plan", Phase 5, moves onto the device (RMS norm, residual add,
 * GeGLU; projections that share an input concatenated: q/k/v, gate/up),
 * folded into one agq_qmv launch:
 *     x_n[k] = bf16(x[k] * rs * norm_weight[k]),  rs = 1 / sqrt(sum_k x[k]^2 / K + eps)
 *              (when norm_weight != NULL; else x_n = x)
 *     v[n]   = sum_k x_n[k] * (s[n, k/gs] * q[n, k] + b[n, k/gs])
 *   act 0: y[n] = v[n] + residual[n] (residual may be NULL),   y [N] BF16
 *   act 1: y[j] = silu(v[2j]) * v[2j + 1],  silu(z) = z / (1 + exp(-z)),   y [N/2] BF16
 *   act 2: y[j] = gelu(v[2j]) * v[2j + 1],  gelu in its tanh form,         y [N/2] BF16
 * For acts 1 and 2 the gate and up projections are concatenated with their
 * rows interleaved (row 2j of w is gate row j, row 2j + 1 up row j), N even,
 * and residual must be NULL. x [K], norm_weight [K] and residual [N] are BF16;
 * w, scales and biases as for agq_qmv. The normalized activation is rounded to
 * BF16 (the layer's activation type) before the product; rs and the products
 * are fp32. residual may be the same buffer as y (an in-place residual add);
 * no other overlap of y with an input is allowed. One kernel launch on
 * `stream`. Supports bits 4 and 8, group sizes 32, 64 and 128, K up to 65536
 * (4-bit) or 32768 (8-bit), N below 2^31; else AGQ_ENOTSUP. eps must be
 * finite and >= 0. Argument checks and errors as for agq_qmv.
 */
#define AGQ_ACT_NONE 0
#define AGQ_ACT_SWIGLU 1
#define AGQ_ACT_GEGLU 2
agq_status agq_qmv_fused(const void *x, const void *norm_weight, float eps, const uint32_t *w,
                         const void *scales, const void *biases, const void *residual, int act,
                         void *y, int64_t N, int64_t K, int bits, int group_size, void *stream);

/*
 * NVFP4 matrix-vector product: the format path that "MLX CUDA Cleanup Plan",
 * Phase 3b, names for the local checkpoint (mode nvfp4, group size 16) and
 * keeps structurally separate from the affine path. The page names the
 * format only; this reads it from the public NVFP4 definition:
 *     y[m, n] = sum_k x[m, k] * e2m1(q[n, k]) * e4m3(s[n, k/16]) * tensor_scale
 *   x      [M, K] BF16, 16-byte aligned, 1 <= M <= 4
 *   w      [N, K/8] U32: 4-bit E2M1 codes (1 sign, 2 exponent bits with bias 1,
 *          1 mantissa bit; values +-{0, 0.5, 1, 1.5, 2, 3, 4, 6}), 8 per word,
 *          low-first, 16-byte aligned
 *   scales [N, K/16] bytes: E4M3 (OCP e4m3fn: bias 7, no infinities,
 *          S.1111.111 = NaN), 2-byte aligned
 *   tensor_scale  fp32, finite
 *   y      [M, N] BF16 (written)
 * fp32 accumulation, one rounding of the sum to BF16. K must be a multiple
 * of 16 (else AGQ_EINVAL) and of 32 (else AGQ_ENOTSUP), M at most 4 and K at
 * most 114688 at M = 1 (as agq_qmv_wide at 4 bits); else AGQ_ENOTSUP. One
 * kernel launch on `stream`. Argument checks and errors as for agq_qmv.
 */
agq_status agq_qmv_nvfp4(const void *x, const uint32_t *w, const void *scales, float tensor_scale, void *y,
                         int64_t M, int64_t N, int64_t K, void *stream);

/*
 * NVFP4 product for any number of activation rows (prefill as well as decode):
 * the same operands and result as agq_qmv_nvfp4, with M >= 1. Up to 4 rows it
 * is agq_qmv_nvfp4. Beyond, either passes of up to 4 rows through that kernel
 * (few rows, or K not a multiple of 64) or a matrix-core GEMM: each weight's
 * value e2m1(q) * e4m3(s) has at most 6 significant bits, so it goes to the
 * matrix cores as an exact bfloat16, with fp32 accumulation over K and the
 * tensor scale applied to each result once before its bfloat16 rounding. The
 * choice is made on the host from the shape. M*K*2 must stay below 2^31.
 * Same argument checks and errors as agq_qmv_nvfp4 otherwise. workspace and
 * workspace_bytes as for agq_qmm, sized by agq_qmm_nvfp4_workspace; with a K
 * split the tensor scale multiplies the sum of the splits.
 */
int64_t agq_qmm_nvfp4_workspace(int64_t M, int64_t N, int64_t K);
agq_status agq_qmm_nvfp4(const void *x, const uint32_t *w, const void *scales, float tensor_scale, void *y,
                         int64_t M, int64_t N, int64_t K, void *workspace, int64_t workspace_bytes,
                         void *stream);

/*
 * Expert-gathered matrix-matrix product (MoE prefill, the gather_qmm of the
 * same epic: its Diagnosis (baseline) MoE prefill row is the largest measured
 * gap on those pages, and Phase 3 (#629) targets it). Same arguments and
 * result as agq_gather_qmv, for any number of pairs per expert: each plane
 * that some pair uses streams once per 64 of its pairs, with every tile of x
 * rows gathered through the pair's lhs index. P may be at most 4096; R*K*2
 * must stay below 2^31 (4 and 8 bits); group size 64. Out-of-range indices
 * give NaN rows, as in agq_gather_qmv. At the bit-stream widths (2, 3, 5, 6
 * bits) the pairs run through the bit-stream matvec as in agq_gather_qmv.
 */
agq_status agq_gather_qmm(const void *x, const uint32_t *w, const void *scales, const void *biases,
                          const uint32_t *lhs_indices, const uint32_t *rhs_indices, void *y,
                          int64_t P, int64_t R, int64_t E, int64_t N, int64_t K,
                          int bits, int group_size, void *stream);

/*
 * Fused decode MoE layer with SwiGLU experts: the fused decode-MoE kernel of
 * "epic: CUDA (MLX backend) prefill and decode acceleration program",
 * Code-audit findings (+55% decode on qwen3-30b-a3b) and Phase 2 (#626), with
 * the GLU stage that "MLX CUDA Cleanup Plan", Phase 5, moves onto the device.
 * For token t and its experts e_j = experts[t, j] with router weights
 * r[t, j] (j < k):
 *     h_j  = silu(W_gate[e_j] x_t) * (W_up[e_j] x_t),  silu(z) = z / (1 + exp(-z))
 *     y_t  = sum_j r[t, j] * (W_down[e_j] h_j)
 *   x            [T, H] BF16
 *   w_gate, w_up [E, F, H*bits/32] U32; s_gate, b_gate, s_up, b_up [E, F, H/64] BF16
 *   w_down       [E, H, F*bits/32] U32; s_down, b_down [E, H, F/64] BF16
 *   experts      [T, k] uint32 expert per (token, slot)
 *   weights      [T, k] float router weights (applied as given, not normalized)
 *   y            [T, H] BF16 (written)
 *   workspace    device scratch of at least agq_moe_decode_workspace(T, k, H, F)
 *                bytes (4*T*k*(F + H)), 16-byte aligned, owned by the caller;
 *                its contents on return are unspecified. Two calls that
 *                overlap in time must not share one.
 * Three kernel launches on `stream`: the gate and up projections with the
 * SwiGLU, and the down projection with the router weight, both as expert
 * gathers (each used expert's planes streamed once for all of its pairs);
 * then the sum over each token's k slots in slot order (bitwise
 * deterministic). The intermediate h keeps about 17 significant bits.
 * Supports 4-bit codes, group size 64, H and F multiples of 512, T <= 256
 * tokens and T*k <= 4096 (else AGQ_ENOTSUP). A token with an expert id >= E
 * gets an all-NaN output row. Argument checks and errors as for agq_qmv; a
 * workspace below the size needed is AGQ_EINVAL.
 */
int64_t agq_moe_decode_workspace(int64_t T, int64_t k, int64_t H, int64_t F);
agq_status agq_moe_decode(const void *x, const uint32_t *w_gate, const void *s_gate, const void *b_gate,
                          const uint32_t *w_up, const void *s_up, const void *b_up,
                          const uint32_t *w_down, const void *s_down, const void *b_down,
                          const uint32_t *experts, const float *weights, void *y,
                          void *workspace, int64_t workspace_bytes,
                          int64_t T, int64_t k, int64_t E, int64_t H, int64_t F,
                          int bits, int group_size, void *stream);

/*
 * agq_moe_decode without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation). The workspace lives in a scratch array
 * the library holds on each device (8 MiB, kept until the process ends):
 * 4*T*k*(F + H) bytes must fit in it, else AGQ_ENOTSUP.
 * The call allocates nothing. Every call on a device shares that array and it
 * keeps the last call's contents, so calls that overlap in time on one device
 * (on different streams) race and must not be issued. Otherwise the same
 * arguments, result and errors as agq_moe_decode.
 */
agq_status agq_moe_decode_noalloc(const void *x, const uint32_t *w_gate, const void *s_gate, const void *b_gate,
                                  const uint32_t *w_up, const void *s_up, const void *b_up,
                                  const uint32_t *w_down, const void *s_down, const void *b_down,
                                  const uint32_t *experts, const float *weights, void *y,
                                  int64_t T, int64_t k, int64_t E, int64_t H, int64_t F,
                                  int bits, int group_size, void *stream);

/*
 * Affine group quantizer on the device: the step before the products, which
 * "MLX CUDA Cleanup Plan", Phase 5, moves off the host (repeated host-side
 * quantization is one of the per-op overheads it lists), and which the
 * quantized KV cache of "epic: CUDA (MLX backend) prefill and decode
 * acceleration program", Phase 5 (#635), needs. Per row and group of
 * group_size columns, in binary32:
 *     scale = bf16((max - min) / (2^bits - 1)),  bias = bf16(min),
 *     q = clamp(rint((w - bias) / scale), 0, 2^bits - 1)   (q = 0 where scale is 0)
 * with correctly rounded division, rint to nearest even and the rounded scale
 * and bias; codes packed into each row's low-first bit stream.
 *   w       [rows, K] float (w_dtype AGQ_DTYPE_F32) or BF16 (AGQ_DTYPE_BF16)
 *   codes   [rows, K*bits/32] U32 (written); scales, biases [rows, K/group_size] BF16 (written)
 * bits 2, 3, 4, 5, 6 or 8; group_size 32, 64 or 128. Inputs must be finite.
 * Errors as for agq_dequantize.
 */
#define AGQ_DTYPE_F32 0
#define AGQ_DTYPE_BF16 1
agq_status agq_quantize(const void *w, int w_dtype, uint32_t *codes, void *scales, void *biases, int64_t rows,
                        int64_t K, int bits, int group_size, void *stream);

/*
 * The dequantization step on its own, as a check of the unpack and affine map
 * of "MLX CUDA Cleanup Plan", Target Architecture §1 (U32-packed codes with
 * BF16 scales and biases), against which the products can be verified bit for
 * bit. Dequantize to fp32: out[n, k] = scale[n, k/gs] * q[n, k] + bias[n, k/gs]
 * (gs = group_size: 32, 64 or 128),
 * formed with one fused multiply-add, so each output is the exact value
 * rounded once to binary32. The exact value is representable, and the result
 * therefore exact, unless the bias exceeds the scale by more than about 2^15
 * (BF16 scale and bias hold 8 significant bits each).
 * `rows` covers stacked planes: pass E*N for a [E, N, .] tensor. Every width
 * (2, 3, 4, 5, 6, 8 bits) and group size (32, 64, 128).
 *   w [rows, K*bits/32] U32; scales/biases [rows, K/group_size] BF16; out [rows, K] fp32.
 */
agq_status agq_dequantize(const uint32_t *w, const void *scales, const void *biases, float *out,
                          int64_t rows, int64_t K, int bits, int group_size, void *stream);

/*
 * Launch plan (host-only introspection; no HIP call). It describes how the
 * product kernels would tile a problem of this shape on a device with
 * `num_cus` compute units holding `waves_per_cu` waves of the chosen kernel
 * at once. The product entry points use the same tiling, with the residency
 * that the HIP occupancy query reports for the kernel. `experts` is 0 for
 * agq_qmv / agq_qmv_wide and E for agq_gather_qmv (whose plan ignores M and
 * sizes for 8 rows per pass).
 */
typedef struct agq_plan {
    int32_t bits;            /* 4 or 8 (the bit-stream widths have no launch plan: AGQ_ENOTSUP) */
    int32_t chunks_per_row;  /* 16-byte chunks of packed codes per weight row */
    int32_t cpt;             /* chunks per lane within a wave's K segment */
    int32_t mw;              /* activation rows handled per pass */
    int32_t rows_per_iter;   /* weight rows in flight per wave iteration */
    int32_t waves_per_group; /* waves splitting K for one set of rows */
    int32_t groups_per_block;
    int32_t threads_per_block;
    int64_t rows_per_group;  /* rows each group visits: iterations x rows_per_iter */
    int64_t row_groups;      /* groups launched (blocks x groups_per_block) */
    int64_t blocks;          /* grid size (per expert for gather) */
    int32_t row_order;       /* 0: group g takes rows (it*row_groups + g)*R + r (round-robin);
                                1: group g takes rows [g*rows_per_group, (g+1)*rows_per_group) */
    int32_t x_lds_bytes;     /* LDS per block holding x (0: waves read x from global memory) */
    int32_t stages;          /* depth of each wave's ring of in-flight row loads; rows_per_group is a
                                multiple of stages x rows_per_iter */
    int32_t resident_waves;  /* waves of the chosen kernel the device holds at once, at this block size
                                (agq_plan_product: num_cus x waves_per_cu); the grid is sized from it */
    int32_t engine;          /* 0: VALU dot products (the fields above as described);
                                1: matrix cores (4-bit, K % 512 == 0, several activation rows or the
                                gather): bands of rows_per_iter = 16*tiles rows, waves_per_group waves
                                splitting K per block, one band group per block (groups_per_block 1,
                                blocks = row_groups), mw = 16 rows per pass, cpt = 0, stages = 128-column
                                segments in flight per wave;
                                2: the bit-stream kernel (4-bit, group size 64, M = 1, at least two
                                16-row blocks per compute unit): blocks of 4 waves (groups_per_block 4,
                                threads_per_block 256), each wave 4 consecutive rows (rows_per_iter =
                                rows_per_group = 4, row_order 1), its rows staged through LDS two at a
                                time (stages 2), x in LDS per 4096-column chunk (x_lds_bytes), cpt = 0 */
} agq_plan;

agq_status agq_plan_product(int64_t M, int64_t N, int64_t K, int bits, int group_size,
                            int num_cus, int waves_per_cu, int64_t experts, agq_plan *plan);

/*
 * The plan the product entry points launch on the current HIP device: the
 * same tiling, with the residency the HIP occupancy query reports for the
 * chosen kernel. Makes HIP calls (device properties, occupancy) but launches
 * nothing. Errors as for the products.
 */
agq_status agq_plan_launch(int64_t M, int64_t N, int64_t K, int bits, int group_size, int64_t experts,
                           agq_plan *plan);

#ifdef __cplusplus
}
#endif

#endif /* AGQ_H */
