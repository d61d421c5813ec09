/*
 * CPU oracle for the affine group-quantized matrix-vector product.
 *
 * TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load or call this library. The GPU library
 * never links, includes or calls it, and it shares no code with the GPU library.
 *
 * It is plain, slow, single-threaded C in double precision. It takes the
 * method's steps in order (unpack -> dequantize -> dot product), with no
 * blocking, fusion or reordering.
 *
 * Sources:
 *  - Operand formats: "MLX CUDA Cleanup Plan", Target Architecture §1. The
 *    accelerated op multiplies BF16 activations by U32-packed affine-quantized
 *    weights with BF16 scales and biases, in rank-2 and rank-3-plane
 *    (per-expert) forms.
 *  - Bit widths and group size: same page, Refactor Plan, Phase 3. BF16
 *    inputs, 4-bit and 8-bit affine packed weights, group size 64.
 *  - "gemma-4 decode carries ~44 ms/token model-specific fixed overhead on
 *    GB10", Re-scope: the MLP projections are 8-bit, group size 64.
 *  - The expert-gathered form is the gather_qmm path of "epic: CUDA (MLX
 *    backend) prefill and decode acceleration program", Code-audit findings.
 *
 * The pages name the format ("affine") but print neither the affine map nor
 * the bit order. Readings adopted:
 *  - a weight is w = scale * q + bias, one (scale, bias) per 64 consecutive
 *    input columns of a row;
 *  - element k of a row occupies bits [bits*k, bits*k + bits) of the row's
 *    little-endian bit stream, word i holding stream bits 32i .. 32i + 31
 *    (low-first). For 4 and 8 bits, the widths the pages name, element k is
 *    in word k / (32/bits) at bit offset bits * (k % (32/bits)); the other
 *    widths of the affine family (2, 3, 5, 6) take the same stream, so a 3-,
 *    5- or 6-bit code may straddle two words and a group of 64 columns is
 *    exactly 2 * bits words;
 *  - W is [N out, K in] and y[m, n] = sum_k x[m, k] * w[n, k].
 *
 * The decode MoE layer (agqo_moe_swiglu) composes these steps the way the
 * fused decode-MoE kernel of "epic: CUDA (MLX backend) prefill and decode
 * acceleration program" (Code-audit findings; Phase 2, #626) does: each
 * token's top-k experts take a gate and an up projection of the token, the
 * gated unit silu(gate) * up (the GLU stage the "MLX CUDA Cleanup Plan",
 * Phase 5, moves onto the device), a down projection, and the router-weighted
 * sum over the k experts. The pages name the kernel and the stages but print
 * no formula; this is the plainest reading, in exact float64 with no
 * intermediate rounding.
 *
 * The NVFP4 product (agqo_qmv_nvfp4) is the structurally separate path of
 * "MLX CUDA Cleanup Plan", Phase 3b (mode nvfp4, group size 16). The page
 * names the format only. Readings: the public NVFP4 definition, 4-bit E2M1
 * elements (1 sign, 2 exponent bits with bias 1, 1 mantissa bit) with one
 * E4M3 scale (1 sign, 4 exponent bits with bias 7, 3 mantissa bits, no
 * infinities, S.1111.111 = NaN) per 16 consecutive columns, and one fp32
 * tensor scale; w = e2m1(q) * e4m3(s) * tensor_scale. Codes pack 8 per U32,
 * low-first, as the affine 4-bit codes; scales are bytes [N, K/16].
 *
 * The fused batch-1 projection (agqo_qmv_fused) adds the neighbouring stages
 * that "MLX CUDA Cleanup Plan", Phase 5, lists for the device-resident decode
 * layer: RMS norm before the product, residual add or a GLU (SwiGLU, GeGLU)
 * after it, on projections that share one input (gate and up interleaved).
 * The page names the stages only. Readings: RMS norm scales by
 * 1/sqrt(mean(x^2) + eps) times a per-column weight and its output is a BF16
 * activation (rounded to nearest even, as the layer's activations are BF16);
 * gelu is the tanh form; silu(z) = z / (1 + e^-z).
 *
 * Every function here is pinned by the CPU test suite to known-answer words,
 * closed forms, exact rational brute force and a float64 BLAS product.
 */
#include <stdint.h>
#include <string.h>
#include <math.h>
#include <stdlib.h>

#define AGQO_OK 0
#define AGQO_EARG (-1)
#define AGQO_EINDEX (-2)

/* A bfloat16 is the top half of an IEEE binary32, so the value is exact. */
static double bf16_value(uint16_t h)
{
    uint32_t u = ((uint32_t)h) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

static int bits_ok(int bits) { return bits >= 2 && bits <= 8 && bits != 7; }

static int check_format(int64_t K, int bits, int group_size)
{
    if (!bits_ok(bits)) return AGQO_EARG;
    if (group_size <= 0 || K <= 0 || K % group_size != 0) return AGQO_EARG;
    if ((K * bits) % 32 != 0) return AGQO_EARG;  /* whole words per row */
    return AGQO_OK;
}

/* Step 1, unpack: the integer code of element k of one packed row, bits
 * [bits*k, bits*k + bits) of its stream (the word after, where they run past
 * a word's end). */
static uint32_t code_at(const uint32_t *packed_row, int64_t k, int bits)
{
    int64_t first = (int64_t)bits * k;
    uint64_t pair = packed_row[first / 32];
    if (first % 32 + bits > 32) pair |= (uint64_t)packed_row[first / 32 + 1] << 32;
    uint32_t mask = (1u << bits) - 1u;
    return (uint32_t)(pair >> (first % 32)) & mask;
}

/* Step 2, dequantize: w = scale * q + bias, in double (exact for bf16 scale/bias). */
static double weight_at(const uint32_t *packed_row, const uint16_t *scale_row,
                        const uint16_t *bias_row, int64_t k, int bits, int group_size)
{
    int64_t g = k / group_size;
    double q = (double)code_at(packed_row, k, bits);
    return bf16_value(scale_row[g]) * q + bf16_value(bias_row[g]);
}

/* Step 3, dot product of one activation row with one weight row, in increasing k.
 * Also returns sum_k |x_k * w_k|, the scale of the rounding tolerance. */
static void row_dot(const uint16_t *x_row, const uint32_t *packed_row,
                    const uint16_t *scale_row, const uint16_t *bias_row,
                    int64_t K, int bits, int group_size, double *y, double *a)
{
    double acc = 0.0, mag = 0.0;
    for (int64_t k = 0; k < K; ++k) {
        double term = bf16_value(x_row[k]) *
                      weight_at(packed_row, scale_row, bias_row, k, bits, group_size);
        acc += term;
        mag += fabs(term);
    }
    *y = acc;
    *a = mag;
}

/* Unpacked integer codes, q[n*K + k]. */
int agqo_unpack(const uint32_t *w, int64_t N, int64_t K, int bits, uint8_t *q)
{
    if (!w || !q || N <= 0 || !bits_ok(bits) || K <= 0 || (K * bits) % 32)
        return AGQO_EARG;
    int64_t words = K * bits / 32;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k)
            q[n * K + k] = (uint8_t)code_at(w + n * words, k, bits);
    return AGQO_OK;
}

/* Dequantized weights out[n*K + k] = scale*q + bias (double). Returns through
 * *not_f32 how many values are not exactly representable in binary32. */
int agqo_dequantize(const uint32_t *w, const uint16_t *scales, const uint16_t *biases,
                    int64_t N, int64_t K, int bits, int group_size,
                    double *out, int64_t *not_f32)
{
    if (!w || !scales || !biases || !out || N <= 0) return AGQO_EARG;
    if (check_format(K, bits, group_size)) return AGQO_EARG;
    int64_t words = K * bits / 32, groups = K / group_size, bad = 0;
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t k = 0; k < K; ++k) {
            double v = weight_at(w + n * words, scales + n * groups, biases + n * groups,
                                 k, bits, group_size);
            out[n * K + k] = v;
            if ((double)(float)v != v) ++bad;
        }
    }
    if (not_f32) *not_f32 = bad;
    return AGQO_OK;
}

/* y[m, i] = sum_k x[m, k] * w[n_i, k] for M activation rows and the weight rows
 * n_i = rows[i] (or n_i = i when rows is NULL, nrows == N). Output layout
 * [M, nrows]; a[] receives sum_k |x[m,k] * w[n_i,k]| in the same layout. */
int agqo_qmv(const uint16_t *x, int64_t M,
             const uint32_t *w, const uint16_t *scales, const uint16_t *biases,
             int64_t N, int64_t K, int bits, int group_size,
             const int64_t *rows, int64_t nrows, double *y, double *a)
{
    if (!x || !w || !scales || !biases || !y || !a || M <= 0 || N <= 0) return AGQO_EARG;
    if (check_format(K, bits, group_size)) return AGQO_EARG;
    if (!rows) nrows = N;
    if (nrows <= 0) return AGQO_EARG;
    int64_t words = K * bits / 32, groups = K / group_size;
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t i = 0; i < nrows; ++i) {
            int64_t n = rows ? rows[i] : i;
            if (n < 0 || n >= N) return AGQO_EINDEX;
            row_dot(x + m * K, w + n * words, scales + n * groups, biases + n * groups,
                    K, bits, group_size, &y[m * nrows + i], &a[m * nrows + i]);
        }
    }
    return AGQO_OK;
}

/* Expert-gathered product, one output row per (token, expert) pair p:
 * y[p, i] = sum_k x[lhs[p], k] * w[rhs[p]][n_i, k]. W, scales and biases are
 * stacked expert planes [E, N, .]. A NULL lhs (rhs) means lhs[p] = p (rhs[p] = p).
 * Output layout [P, nrows]. */
int agqo_gather_qmv(const uint16_t *x, int64_t R,
                    const uint32_t *w, const uint16_t *scales, const uint16_t *biases,
                    int64_t E, int64_t N, int64_t K, int bits, int group_size,
                    const uint32_t *lhs, const uint32_t *rhs, int64_t P,
                    const int64_t *rows, int64_t nrows, double *y, double *a)
{
    if (!x || !w || !scales || !biases || !y || !a) return AGQO_EARG;
    if (R <= 0 || E <= 0 || N <= 0 || P <= 0) return AGQO_EARG;
    if (check_format(K, bits, group_size)) return AGQO_EARG;
    if (!rows) nrows = N;
    if (nrows <= 0) return AGQO_EARG;
    int64_t words = K * bits / 32, groups = K / group_size;
    for (int64_t p = 0; p < P; ++p) {
        int64_t r = lhs ? (int64_t)lhs[p] : p;
        int64_t e = rhs ? (int64_t)rhs[p] : p;
        if (r < 0 || r >= R || e < 0 || e >= E) return AGQO_EINDEX;
        const uint32_t *we = w + e * N * words;
        const uint16_t *se = scales + e * N * groups;
        const uint16_t *be = biases + e * N * groups;
        for (int64_t i = 0; i < nrows; ++i) {
            int64_t n = rows ? rows[i] : i;
            if (n < 0 || n >= N) return AGQO_EINDEX;
            row_dot(x + r * K, we + n * words, se + n * groups, be + n * groups,
                    K, bits, group_size, &y[p * nrows + i], &a[p * nrows + i]);
        }
    }
    return AGQO_OK;
}

/* silu(z) = z * sigmoid(z) = z / (1 + exp(-z)). */
static double silu(double z)
{
    return z / (1.0 + exp(-z));
}

/* Decode MoE layer with a SwiGLU expert MLP, for T tokens with k experts each:
 *   g  = W_gate[e] x_t      (F values; W_gate planes [E, F, H])
 *   u  = W_up[e]   x_t      (F values; W_up planes   [E, F, H])
 *   h  = silu(g) * u        (elementwise)
 *   o  = W_down[e] h        (H values; W_down planes [E, H, F])
 *   y_t = sum_{j < k} r[t, j] * o   with e = experts[t, j]
 * in float64, summing slot by slot in increasing j and each dot product in
 * increasing column index. x is [T, H] bf16; experts [T, k] uint32; r [T, k]
 * float (router weights, already normalized by the caller); y [T, H].
 * a[t, m] = sum_j |r[t, j]| * sum_n |w_down[e][m, n] * h_n|, the scale of the
 * rounding tolerance of the final projection. */
int agqo_moe_swiglu(const uint16_t *x, int64_t T, int64_t H, int64_t F, int64_t E, int64_t k,
                    const uint32_t *wg, const uint16_t *sg, const uint16_t *bg,
                    const uint32_t *wu, const uint16_t *su, const uint16_t *bu,
                    const uint32_t *wd, const uint16_t *sd, const uint16_t *bd,
                    const uint32_t *experts, const float *r, int bits, int group_size,
                    double *y, double *a)
{
    if (!x || !wg || !sg || !bg || !wu || !su || !bu || !wd || !sd || !bd || !experts || !r || !y || !a)
        return AGQO_EARG;
    if (T <= 0 || H <= 0 || F <= 0 || E <= 0 || k <= 0) return AGQO_EARG;
    if (check_format(H, bits, group_size) || check_format(F, bits, group_size)) return AGQO_EARG;
    int64_t hw = H * bits / 32, hg = H / group_size;   /* gate/up rows: H columns */
    int64_t fw = F * bits / 32, fg = F / group_size;   /* down rows: F columns */
    double *h = (double *)malloc((size_t)F * sizeof(double));
    if (!h) return AGQO_EARG;
    for (int64_t t = 0; t < T; ++t) {
        for (int64_t m = 0; m < H; ++m) {
            y[t * H + m] = 0.0;
            a[t * H + m] = 0.0;
        }
        for (int64_t j = 0; j < k; ++j) {
            int64_t e = (int64_t)experts[t * k + j];
            if (e < 0 || e >= E) {
                free(h);
                return AGQO_EINDEX;
            }
            double rw = (double)r[t * k + j];
            for (int64_t f = 0; f < F; ++f) {
                double g, u, dummy;
                const int64_t row = e * F + f;
                row_dot(x + t * H, wg + row * hw, sg + row * hg, bg + row * hg, H, bits, group_size, &g, &dummy);
                row_dot(x + t * H, wu + row * hw, su + row * hg, bu + row * hg, H, bits, group_size, &u, &dummy);
                h[f] = silu(g) * u;
            }
            for (int64_t m = 0; m < H; ++m) {
                const int64_t row = e * H + m;
                double dot = 0.0, size = 0.0;
                for (int64_t f = 0; f < F; ++f) {
                    double part = weight_at(wd + row * fw, sd + row * fg, bd + row * fg, f, bits, group_size) * h[f];
                    dot += part;
                    size += fabs(part);
                }
                y[t * H + m] += rw * dot;
                a[t * H + m] += fabs(rw) * size;
            }
        }
    }
    free(h);
    return AGQO_OK;
}

/* binary32 -> bfloat16 bit pattern, round to nearest even (NaN stays NaN). */
static uint16_t bf16_rne(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40u);
    uint32_t lsb = (u >> 16) & 1u;
    return (uint16_t)((u + 0x7FFFu + lsb) >> 16);
}

/* Affine group quantizer, the recipe the workloads state: per row and group of
 * group_size consecutive columns, in binary32,
 *   scale = bf16((max - min) / (2^bits - 1)),  bias = bf16(min),
 *   q = clamp(rint((w - bias) / scale), 0, 2^bits - 1)   (q = 0 where scale is 0)
 * with rint rounding half to even, using the rounded scale and bias. Codes are
 * packed into the row's low-first bit stream. w is [N, K] float; wq [N, K*bits/32];
 * scales and biases [N, K/group_size] bf16. */
int agqo_quantize(const float *w, int64_t N, int64_t K, int bits, int group_size,
                  uint32_t *wq, uint16_t *scales, uint16_t *biases)
{
    if (!w || !wq || !scales || !biases || N <= 0) return AGQO_EARG;
    if (check_format(K, bits, group_size)) return AGQO_EARG;
    const int64_t groups = K / group_size, words = K * bits / 32;
    const float levels = (float)((1 << bits) - 1);
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t i = 0; i < words; ++i) wq[n * words + i] = 0;
        for (int64_t g = 0; g < groups; ++g) {
            const float *wg = w + n * K + g * group_size;
            float mx = wg[0], mn = wg[0];
            for (int64_t j = 1; j < group_size; ++j) {
                if (wg[j] > mx) mx = wg[j];
                if (wg[j] < mn) mn = wg[j];
            }
            const float diff = mx - mn;
            const uint16_t s16 = bf16_rne(diff / levels);
            const uint16_t b16 = bf16_rne(mn);
            scales[n * groups + g] = s16;
            biases[n * groups + g] = b16;
            const float s = (float)bf16_value(s16), b = (float)bf16_value(b16);
            for (int64_t j = 0; j < group_size; ++j) {
                uint32_t q = 0;
                if (s != 0.0f) {
                    const float num = wg[j] - b;
                    const float r = rintf(num / s);
                    q = r <= 0.0f ? 0u : r >= levels ? (uint32_t)levels : (uint32_t)r;
                }
                const int64_t first = (int64_t)bits * (g * group_size + j);  /* stream bit */
                wq[n * words + first / 32] |= q << (uint32_t)(first % 32);
                if (first % 32 + bits > 32) wq[n * words + first / 32 + 1] |= q >> (uint32_t)(32 - first % 32);
            }
        }
    }
    return AGQO_OK;
}

/* Nearest bfloat16 value to v (8 significant bits), ties to even; v finite and
 * inside the normal range. */
static double bf16_round(double v)
{
    if (v == 0.0) return v;
    int e;
    double m = frexp(v, &e); /* v = m * 2^e, 0.5 <= |m| < 1 */
    double t = m * 256.0;    /* 8 significant bits above the point */
    double r = floor(t);
    double d = t - r;
    if (d > 0.5 || (d == 0.5 && fmod(r, 2.0) != 0.0)) r += 1.0;
    return ldexp(r, e - 8);
}

/* E2M1 (FP4) element from its 4-bit code: sign, exponent (bias 1), mantissa;
 * exponent 0 is subnormal (m * 2^-1). */
static double e2m1_value(uint32_t c)
{
    const double sign = (c & 8u) ? -1.0 : 1.0;
    const uint32_t e = (c >> 1) & 3u, m = c & 1u;
    const double mag = e == 0 ? 0.5 * (double)m : ldexp(1.0 + 0.5 * (double)m, (int)e - 1);
    return sign * mag;
}

/* E4M3 (FP8) scale from its byte: sign, exponent (bias 7), mantissa; exponent
 * 0 is subnormal (m/8 * 2^-6); S.1111.111 is NaN (no infinities). */
static double e4m3_value(uint32_t b)
{
    const double sign = (b & 0x80u) ? -1.0 : 1.0;
    const uint32_t e = (b >> 3) & 15u, m = b & 7u;
    if (e == 15 && m == 7) return NAN;
    const double mag = e == 0 ? ldexp((double)m / 8.0, -6) : ldexp(1.0 + (double)m / 8.0, (int)e - 7);
    return sign * mag;
}

/* Exported for the pins. */
double agqo_e2m1(uint32_t c) { return e2m1_value(c & 15u); }
double agqo_e4m3(uint32_t b) { return e4m3_value(b & 255u); }

/* NVFP4 product: y[m, i] = sum_k x[m, k] * e2m1(q[n_i, k]) * e4m3(s[n_i, k/16]) * tensor_scale,
 * in the order unpack -> element value -> scaled weight -> dot product (increasing k),
 * with a[m, i] = sum_k |x * w|. x [M, K] bf16; w [N, K/8] U32; scales [N, K/16] bytes;
 * rows: an optional subset of output rows (NULL: all N). Output layout [M, nrows]. */
int agqo_qmv_nvfp4(const uint16_t *x, int64_t M, const uint32_t *w, const uint8_t *scales, double tensor_scale,
                   int64_t N, int64_t K, const int64_t *rows, int64_t nrows, double *y, double *a)
{
    if (!x || !w || !scales || !y || !a || M <= 0 || N <= 0 || K <= 0 || K % 16 != 0) return AGQO_EARG;
    if (!rows) nrows = N;
    if (nrows <= 0) return AGQO_EARG;
    const int64_t words = K / 8, blocks = K / 16;
    for (int64_t m = 0; m < M; ++m)
        for (int64_t i = 0; i < nrows; ++i) {
            const int64_t n = rows ? rows[i] : i;
            if (n < 0 || n >= N) return AGQO_EINDEX;
            double acc = 0.0, mag = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                const uint32_t q = (w[n * words + k / 8] >> (4 * (k % 8))) & 15u;
                const double wk = e2m1_value(q) * e4m3_value(scales[n * blocks + k / 16]) * tensor_scale;
                const double t = bf16_value(x[m * K + k]) * wk;
                acc += t;
                mag += fabs(t);
            }
            y[m * nrows + i] = acc;
            a[m * nrows + i] = mag;
        }
    return AGQO_OK;
}

/* The rounding above, exported so the test suite can pin it on its own. */
double agqo_bf16_round(double v)
{
    return bf16_round(v);
}

/* gelu through tanh: 0.5 z (1 + tanh(sqrt(2/pi) (z + 0.044715 z^3))). */
static double gelu_tanh(double z)
{
    return 0.5 * z * (1.0 + tanh(0.7978845608028654 * (z + 0.044715 * z * z * z)));
}

/* Batch-1 projection with the decode layer's neighbouring stages fused in:
 *  - prologue (gamma != NULL): RMS norm of x, x_n[k] = bf16(x[k] * r * gamma[k])
 *    with r = 1 / sqrt(sum_k x[k]^2 / K + eps), the normalized activation
 *    rounded to bfloat16, the layer's activation type;
 *  - the product v[n] = sum_k x_n[k] * w[n, k];
 *  - epilogue act 0: y[n] = v[n] (+ residual[n] when residual != NULL);
 *    act 1 (SwiGLU) and act 2 (GeGLU, gelu in its tanh form): rows come in
 *    interleaved gate/up pairs, y[j] = act(v[2j]) * v[2j + 1], N/2 outputs.
 * a[] is the scale of the rounding tolerance: sum_k |x_n[k] w[n, k]| for
 * act 0, and 1.13 |v[2j+1]| A[2j] + |act(v[2j])| A[2j+1] for the GLU forms
 * (1.13 bounds the slope of both activations). */
int agqo_qmv_fused(const uint16_t *x, const uint16_t *gamma, double eps,
                   const uint32_t *w, const uint16_t *scales, const uint16_t *biases,
                   int64_t N, int64_t K, int bits, int group_size,
                   const uint16_t *residual, int act, double *y, double *a)
{
    if (!x || !w || !scales || !biases || !y || !a || N <= 0) return AGQO_EARG;
    if (check_format(K, bits, group_size)) return AGQO_EARG;
    if (act < 0 || act > 2 || (act > 0 && (N % 2 != 0 || residual))) return AGQO_EARG;
    double *xn = (double *)malloc((size_t)K * sizeof(double));
    double *v = (double *)malloc((size_t)N * sizeof(double));
    double *m = (double *)malloc((size_t)N * sizeof(double));
    if (!xn || !v || !m) {
        free(xn);
        free(v);
        free(m);
        return AGQO_EARG;
    }
    double r = 1.0;
    if (gamma) {
        double ss = 0.0;
        for (int64_t k = 0; k < K; ++k) ss += bf16_value(x[k]) * bf16_value(x[k]);
        r = 1.0 / sqrt(ss / (double)K + eps);
    }
    for (int64_t k = 0; k < K; ++k)
        xn[k] = gamma ? bf16_round(bf16_value(x[k]) * r * bf16_value(gamma[k])) : bf16_value(x[k]);
    const int64_t words = K * bits / 32, groups = K / group_size;
    for (int64_t n = 0; n < N; ++n) {
        double sum = 0.0, abs_sum = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            const double t = xn[k] * weight_at(w + n * words, scales + n * groups, biases + n * groups, k, bits,
                                               group_size);
            sum += t;
            abs_sum += fabs(t);
        }
        v[n] = sum;
        m[n] = abs_sum;
    }
    if (act == 0) {
        for (int64_t n = 0; n < N; ++n) {
            y[n] = v[n] + (residual ? bf16_value(residual[n]) : 0.0);
            a[n] = m[n];
        }
    } else {
        for (int64_t j = 0; j < N / 2; ++j) {
            const double g = v[2 * j], u = v[2 * j + 1];
            const double f = act == 1 ? silu(g) : gelu_tanh(g);
            y[j] = f * u;
            a[j] = 1.13 * fabs(u) * m[2 * j] + fabs(f) * m[2 * j + 1];
        }
    }
    free(xn);
    free(v);
    free(m);
    return AGQO_OK;
}
