"""Planted-mistake check of the pins.

Each mutant is the oracle's C source with one plausible mistake, compiled to a
private library on the CPU. Every mutant must fail at least one pin. The
original snippet must occur exactly once, which keeps this list in step with
the source.
"""
import os

import pytest

import oracle
from oracle_pins import PINS

MUTANTS = {
    "high_first_unpack": ("return (uint32_t)(pair >> (first % 32)) & mask;",
                          "return (uint32_t)(pair >> ((32 - bits - first % 32) & 63)) & mask;"),
    "wrong_word_index": ("uint64_t pair = packed_row[first / 32];", "uint64_t pair = packed_row[k / 32];"),
    "straddle_dropped": ("if (first % 32 + bits > 32) pair |= (uint64_t)packed_row[first / 32 + 1] << 32;", ""),
    "quant_straddle_dropped": ("if (first % 32 + bits > 32) wq[n * words + first / 32 + 1] |= q >> (uint32_t)(32 - first % 32);", ""),
    # (in bounds: a mutant that writes past a row can crash the test process)
    "quant_stream_offset": ("const int64_t first = (int64_t)bits * (g * group_size + j);",
                            "const int64_t first = (int64_t)bits * (g * group_size + (j ^ 1));"),
    "short_mask": ("uint32_t mask = (1u << bits) - 1u;", "uint32_t mask = (1u << (bits - 1)) - 1u;"),
    "dropped_bias": ("return bf16_value(scale_row[g]) * q + bf16_value(bias_row[g]);",
                     "return bf16_value(scale_row[g]) * q;"),
    "swapped_scale_bias": ("return bf16_value(scale_row[g]) * q + bf16_value(bias_row[g]);",
                           "return bf16_value(bias_row[g]) * q + bf16_value(scale_row[g]);"),
    "bias_sign": ("return bf16_value(scale_row[g]) * q + bf16_value(bias_row[g]);",
                  "return bf16_value(scale_row[g]) * q - bf16_value(bias_row[g]);"),
    "group_of_128": ("int64_t g = k / group_size;", "int64_t g = k / (2 * group_size);"),
    "dropped_last_term": ("for (int64_t k = 0; k < K; ++k) {\n        double term",
                          "for (int64_t k = 0; k < K - 1; ++k) {\n        double term"),
    "signed_magnitude": ("mag += fabs(term);", "mag += term;"),
    "bf16_shift": ("uint32_t u = ((uint32_t)h) << 16;", "uint32_t u = ((uint32_t)h) << 15;"),
    "x_row_ignored": ("row_dot(x + m * K,", "row_dot(x,"),
    "scale_row_offset": ("row_dot(x + m * K, w + n * words, scales + n * groups,",
                         "row_dot(x + m * K, w + n * words, scales,"),
    "expert_plane_ignored": ("const uint32_t *we = w + e * N * words;", "const uint32_t *we = w;"),
    "lhs_ignored": ("int64_t r = lhs ? (int64_t)lhs[p] : p;", "int64_t r = p % R;"),
    "not_f32_never_counted": ("if ((double)(float)v != v) ++bad;", "if ((float)v != (float)v) ++bad;"),
    "not_f32_inverted": ("if ((double)(float)v != v) ++bad;", "if ((double)(float)v == v) ++bad;"),
    "moe_gate_up_swapped": ("h[f] = silu(g) * u;", "h[f] = silu(u) * g;"),
    "moe_no_silu": ("h[f] = silu(g) * u;", "h[f] = g * u;"),
    "moe_sigmoid_sign": ("return z / (1.0 + exp(-z));", "return z / (1.0 + exp(z));"),
    "moe_router_weight_dropped": ("y[t * H + m] += rw * dot;", "y[t * H + m] += dot;"),
    "moe_magnitude_signed": ("size += fabs(part);", "size += part;"),
    "moe_down_expert_ignored": ("const int64_t row = e * H + m;", "const int64_t row = m;"),
    "moe_token_row_ignored": ("row_dot(x + t * H, wg", "row_dot(x, wg"),
    "quant_levels_off_by_one": ("const float levels = (float)((1 << bits) - 1);",
                                "const float levels = (float)(1 << bits);"),
    "quant_bias_is_max": ("const uint16_t b16 = bf16_rne(mn);", "const uint16_t b16 = bf16_rne(mx);"),
    "quant_truncates": ("const float r = rintf(num / s);", "const float r = floorf(num / s);"),
    "quant_unrounded_scale": ("const float s = (float)bf16_value(s16), b = (float)bf16_value(b16);",
                              "const float s = diff / levels, b = (float)bf16_value(b16);"),
    "quant_no_clamp": ("q = r <= 0.0f ? 0u : r >= levels ? (uint32_t)levels : (uint32_t)r;",
                       "q = (uint32_t)r & ((1u << bits) - 1u);"),
    "quant_bf16_truncates": ("return (uint16_t)((u + 0x7FFFu + lsb) >> 16);", "return (uint16_t)(u >> 16);"),
    "fused_sum_not_mean": ("r = 1.0 / sqrt(ss / (double)K + eps);", "r = 1.0 / sqrt(ss + eps);"),
    "fused_gamma_ignored": ("xn[k] = gamma ? bf16_round(bf16_value(x[k]) * r * bf16_value(gamma[k])) : bf16_value(x[k]);",
                            "xn[k] = gamma ? bf16_round(bf16_value(x[k]) * r) : bf16_value(x[k]);"),
    "fused_norm_not_rounded": ("xn[k] = gamma ? bf16_round(bf16_value(x[k]) * r * bf16_value(gamma[k])) : bf16_value(x[k]);",
                               "xn[k] = gamma ? bf16_value(x[k]) * r * bf16_value(gamma[k]) : bf16_value(x[k]);"),
    "fused_round_truncates": ("if (d > 0.5 || (d == 0.5 && fmod(r, 2.0) != 0.0)) r += 1.0;", "if (d > 1.0) r += 1.0;"),
    "fused_ties_away": ("if (d > 0.5 || (d == 0.5 && fmod(r, 2.0) != 0.0)) r += 1.0;", "if (d >= 0.5) r += 1.0;"),
    "fused_glu_swapped": ("const double g = v[2 * j], u = v[2 * j + 1];", "const double u = v[2 * j], g = v[2 * j + 1];"),
    "fused_acts_swapped": ("const double f = act == 1 ? silu(g) : gelu_tanh(g);",
                           "const double f = act == 2 ? silu(g) : gelu_tanh(g);"),
    "fused_gelu_cubic": ("(z + 0.044715 * z * z * z)", "(z + 0.044715 * z * z)"),
    "fused_magnitude_signed": ("abs_sum += fabs(t);", "abs_sum += t;"),
    "fused_residual_dropped": ("y[n] = v[n] + (residual ? bf16_value(residual[n]) : 0.0);", "y[n] = v[n];"),
    "e2m1_bias_2": ("ldexp(1.0 + 0.5 * (double)m, (int)e - 1)", "ldexp(1.0 + 0.5 * (double)m, (int)e - 2)"),
    "e2m1_no_subnormal": ("e == 0 ? 0.5 * (double)m :", "e == 0 ? 1.0 * (double)m :"),
    "e2m1_sign_ignored": ("const double sign = (c & 8u) ? -1.0 : 1.0;", "const double sign = 1.0;"),
    "e4m3_bias_8": ("ldexp(1.0 + (double)m / 8.0, (int)e - 7)", "ldexp(1.0 + (double)m / 8.0, (int)e - 8)"),
    "e4m3_subnormal_scale": ("ldexp((double)m / 8.0, -6)", "ldexp((double)m / 8.0, -7)"),
    "nvfp4_block_32": ("e4m3_value(scales[n * blocks + k / 16])", "e4m3_value(scales[n * blocks + k / 32])"),
    "nvfp4_high_first": ("(w[n * words + k / 8] >> (4 * (k % 8))) & 15u", "(w[n * words + k / 8] >> (4 * (7 - k % 8))) & 15u"),
    "nvfp4_magnitude_signed": ("mag += fabs(t);", "mag += t;"),
    "nvfp4_tensor_scale_dropped": ("* e4m3_value(scales[n * blocks + k / 16]) * tensor_scale;", "* e4m3_value(scales[n * blocks + k / 16]);"),
    "moe_up_with_gate_scales": ("row_dot(x + t * H, wu + row * hw, su + row * hg,",
                                "row_dot(x + t * H, wu + row * hw, sg + row * hg,"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    with open(oracle.SRC) as f:
        src = f.read()
    assert src.count(old) == 1, f"snippet for {name} not found exactly once"
    path = tmp_path / f"{name}.c"
    path.write_text(src.replace(old, new))
    lib = oracle.load(oracle.build(str(path), str(tmp_path / f"lib{name}.so"), strict=False))
    failed = []
    for pin in PINS:
        try:
            pin(lib)
        except (AssertionError, oracle.OracleError):
            failed.append(pin.__name__)
    assert failed, f"mutant {name} passed every pin"
