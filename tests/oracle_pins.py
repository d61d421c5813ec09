"""Pins that tie the CPU oracle to facts outside itself.

Each ``pin_*`` takes a loaded oracle library and raises ``AssertionError`` on
a mismatch. ``test_oracle_pins.py`` runs them against the real oracle.
``test_oracle_mutants.py`` runs them against copies of the oracle with one
planted mistake each, and requires every mutant to fail at least one pin.

Anchors used:
  * known-answer packed words (the low-first bit layout, written out by hand);
  * the hand-worked closed forms in ``golden/worked_k64.json``;
  * the producer-side quantizer (scale = (max-min)/(2^bits-1), bias = min):
    quantizing the oracle's dequantized weights must give back the original
    codes, scales and biases;
  * exact rational brute force (``fractions.Fraction``) on tiny shapes, with
    codes taken from before packing;
  * a float64 BLAS product on a densely built weight matrix;
  * an integer-valued special case, which must come out exact;
  * the constant-code closed form sum_g (s_g*c + b_g) * sum_{k in g} x_k;
  * for the decode MoE layer: the odd part of silu (silu(z) - silu(-z) = z, so
    negated gate planes with router weights +1 and -1 leave an exp-free
    polynomial), saturation (silu(64) = 64 and silu(-64) ~ 0 in float64), and
    exact-rational projections with silu written through tanh.
"""
from __future__ import annotations

import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from seeded_inputs import bf16_bits, bf16_to_f32, pack_codes, quantize_rows, draw_quantized_weight

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "worked_k64.json")
U53 = 2.0 ** -53


def _frac_bf16(h):
    return Fraction(float(bf16_to_f32(np.array([h], dtype=np.uint16))[0]))


def _random_problem(seed, M, N, K, bits, E=None):
    g = np.random.default_rng(seed)
    shape = (N, K) if E is None else (E, N, K)
    codes = g.integers(0, 2 ** bits, size=shape, dtype=np.uint8)
    gshape = shape[:-1] + (K // 64,)
    scales = bf16_bits((0.01 + 0.02 * g.random(gshape)).astype(np.float32))
    biases = bf16_bits((-0.05 + 0.03 * g.standard_normal(gshape)).astype(np.float32))
    x = bf16_bits(g.standard_normal((M, K)).astype(np.float32))
    return x, codes, scales, biases


def _exact_row(xrow, qrow, srow, brow, gs=64):
    y = Fraction(0)
    a = Fraction(0)
    for k in range(len(qrow)):
        w = _frac_bf16(srow[k // gs]) * int(qrow[k]) + _frac_bf16(brow[k // gs])
        t = _frac_bf16(xrow[k]) * w
        y += t
        a += abs(t)
    return y, a


def pin_unpack_known_words(lib):
    words4 = np.array([[0x76543210, 0xFEDCBA98, 0x00000000, 0x80000000,
                        0xFFFFFFFF, 0x11111111, 0x01234567, 0x0000000F]], dtype=np.uint32)
    want4 = ([0, 1, 2, 3, 4, 5, 6, 7] + [8, 9, 10, 11, 12, 13, 14, 15] + [0] * 8 +
             [0] * 7 + [8] + [15] * 8 + [1] * 8 + [7, 6, 5, 4, 3, 2, 1, 0] + [15] + [0] * 7)
    got4 = oracle.unpack(words4, 64, 4, lib=lib)
    assert got4.tolist() == [want4], got4
    words8 = np.array([[0x03020100, 0xFFFEFDFC, 0x80000000, 0xFFFFFFFF,
                        0x000000FF, 0x7F00807F, 0x00000001, 0x01000000]], dtype=np.uint32)
    want8 = ([0, 1, 2, 3] + [252, 253, 254, 255] + [0, 0, 0, 128] + [255] * 4 +
             [255, 0, 0, 0] + [127, 128, 0, 127] + [1, 0, 0, 0] + [0, 0, 0, 1])
    got8 = oracle.unpack(words8, 32, 8, lib=lib)
    assert got8.tolist() == [want8], got8
    # The other widths: codes c_k = (3k + 1) mod 2^bits, k < 32, placed by hand at stream bits
    # bits*k .. bits*k + bits - 1 (word 0 of the 3-bit row: bits 0, 5-8, 10, 12, 14, 18, 19,
    # 22-24, 29-31 set, the last two from code 10 = 7, which runs into word 1).
    words = {2: [0xB1B1B1B1, 0xB1B1B1B1],
             3: [0xE1CC55E1, 0x55E1CC55, 0xCC55E1CC],
             5: [0xE0D51C81, 0x517F99B4, 0x5E9172D0, 0x8930C1DD, 0xF6F1593D],
             6: [0x0D287101, 0xF7195934, 0xBABA2589, 0x3DEB7D31, 0xF3091830, 0x79B61548]}
    for bits, ws in words.items():
        got = oracle.unpack(np.array([ws], np.uint32), 32, bits, lib=lib)
        assert got.tolist() == [[(3 * k + 1) % 2 ** bits for k in range(32)]], (bits, got)


def pin_unpack_roundtrip(lib):
    for bits in (2, 3, 4, 5, 6, 8):
        q = np.random.default_rng(bits).integers(0, 2 ** bits, size=(5, 192), dtype=np.uint8)
        got = oracle.unpack(pack_codes(q, bits), 192, bits, lib=lib)
        assert np.array_equal(got, q)


def pin_golden_worked(lib):
    with open(GOLDEN) as f:
        doc = json.load(f)
    for case in doc["cases"]:
        y, a = oracle.qmv(np.array(case["x_bf16"], dtype=np.uint16),
                          np.array(case["w_u32"], dtype=np.uint32),
                          np.array(case["scales_bf16"], dtype=np.uint16),
                          np.array(case["biases_bf16"], dtype=np.uint16),
                          case["K"], case["bits"], case["group_size"], lib=lib)
        assert y.tolist() == case["y"], (case["bits"], y)
        assert a.tolist() == case["A"], (case["bits"], a)


def pin_dequant_quantizer_roundtrip(lib):
    for bits in (3, 4, 5, 6, 8):
        d = draw_quantized_weight(99, bits, 64, 256, bits, keep_codes=True)
        what, not_f32 = oracle.dequantize(d["w"], d["scales"], d["biases"], 256, bits, lib=lib)
        assert not_f32 == 0
        q2, s2, b2 = quantize_rows(what.astype(np.float32), bits)
        # Groups whose codes span the full range re-quantize to themselves exactly:
        # max - min = scale*(2^bits-1) and min = bias. (8-bit groups whose top code
        # rounded to 2^bits-2 are excluded; they are a minority.)
        qg = d["codes"].reshape(64, 4, 64)
        full = (qg.min(-1) == 0) & (qg.max(-1) == 2 ** bits - 1)
        assert full.mean() > 0.5
        assert np.array_equal(s2[full], d["scales"][full])
        assert np.array_equal(b2[full], d["biases"][full])
        assert np.array_equal(q2.reshape(64, 4, 64)[full], qg[full])


def _fits_binary32(v: Fraction) -> bool:
    """Whether an exact dyadic rational is a binary32 value: its odd significand has at
    most 24 bits (the values here are far inside the normal exponent range)."""
    if v == 0:
        return True
    num, den = abs(v.numerator), v.denominator
    assert den & (den - 1) == 0, "dyadic rationals only"
    while num % 2 == 0:
        num //= 2
    return num < (1 << 24)


def pin_dequant_not_f32_count(lib):
    """The count of dequantized weights that binary32 cannot hold, against an exact count.

    Groups: s = 129*2^-17 with b = 2^15 (every nonzero code needs more than 24 bits),
    the same s with b = 2^8 (codes that are multiples of 4 fit, others do not), and
    s = 1, b = 1/2 (everything fits). The expected count comes from integer reasoning
    on the exact rational s*q + b, not from a floating-point round trip."""
    for bits in (4, 8):
        K = 192
        g = np.random.default_rng(60 + bits)
        q = g.integers(0, 2 ** bits, size=(3, K), dtype=np.uint8)
        q[0, :5] = 0
        s = np.array([[0x3A81, 0x3A81, 0x3F80]] * 3, np.uint16)
        b = np.array([[0x4700, 0x4380, 0x3F00]] * 3, np.uint16)
        want = 0
        for n in range(3):
            for k in range(K):
                v = _frac_bf16(s[n, k // 64]) * int(q[n, k]) + _frac_bf16(b[n, k // 64])
                want += not _fits_binary32(v)
        assert 0 < want < 3 * K
        _, got = oracle.dequantize(pack_codes(q, bits), s, b, K, bits, lib=lib)
        assert got == want, (bits, got, want)


def pin_dot_exact_bruteforce(lib):
    for bits in (2, 3, 4, 5, 6, 8):
        for seed, (M, N, K) in enumerate([(2, 3, 64), (1, 2, 128), (3, 4, 192)]):
            x, q, s, b = _random_problem(100 + seed + bits, M, N, K, bits)
            y, a = oracle.qmv(x, pack_codes(q, bits), s, b, K, bits, lib=lib)
            for m in range(M):
                for n in range(N):
                    ye, ae = _exact_row(x[m], q[n], s[n], b[n])
                    bound = 2 * K * U53 * float(ae)
                    assert abs(y[m, n] - float(ye)) <= bound, (bits, M, N, K, m, n)
                    assert abs(a[m, n] - float(ae)) <= bound, (bits, M, N, K, m, n)


def pin_other_group_sizes_bruteforce(lib):
    """Groups of 32 and 128 columns: exact rationals over codes from before packing."""
    for bits in (3, 4, 5, 8):
        for gs, K in ((32, 96), (128, 256)):
            g = np.random.default_rng([70, bits, gs])
            M, N = 2, 3
            q = g.integers(0, 2 ** bits, size=(N, K), dtype=np.uint8)
            sc = bf16_bits((0.01 + 0.02 * g.random((N, K // gs))).astype(np.float32))
            bi = bf16_bits((-0.05 + 0.03 * g.standard_normal((N, K // gs))).astype(np.float32))
            x = bf16_bits(g.standard_normal((M, K)).astype(np.float32))
            y, a = oracle.qmv(x, pack_codes(q, bits), sc, bi, K, bits, group_size=gs, lib=lib)
            for m in range(M):
                for n in range(N):
                    ye, ae = _exact_row(x[m], q[n], sc[n], bi[n], gs)
                    assert abs(y[m, n] - float(ye)) <= 2 * K * U53 * float(ae), (bits, gs, m, n)
            deq, _ = oracle.dequantize(pack_codes(q, bits), sc, bi, K, bits, group_size=gs, lib=lib)
            want = np.repeat(bf16_to_f32(sc).astype(np.float64), gs, axis=1) * q + \
                np.repeat(bf16_to_f32(bi).astype(np.float64), gs, axis=1)
            assert np.array_equal(deq, want), (bits, gs)


def pin_numpy_blas(lib):
    for bits in (3, 4, 6, 8):
        x, q, s, b = _random_problem(7 + bits, 3, 96, 1024, bits)
        y, a = oracle.qmv(x, pack_codes(q, bits), s, b, 1024, bits, lib=lib)
        sf = np.repeat(bf16_to_f32(s).astype(np.float64), 64, axis=1)
        bf = np.repeat(bf16_to_f32(b).astype(np.float64), 64, axis=1)
        wd = sf * q.astype(np.float64) + bf
        xd = bf16_to_f32(x).astype(np.float64)
        yb = xd @ wd.T
        ab = np.abs(xd) @ np.abs(wd).T
        assert np.all(np.abs(y - yb) <= 1e-12 * ab)
        assert np.allclose(a, ab, rtol=1e-12, atol=0)


def pin_integer_special_case(lib):
    g = np.random.default_rng(5)
    N, K = 7, 320
    q = g.integers(0, 256, size=(N, K), dtype=np.uint8)
    xi = g.integers(-8, 9, size=(2, K))
    x = bf16_bits(xi.astype(np.float32))
    ones = np.full((N, K // 64), 0x3F80, dtype=np.uint16)
    zeros = np.zeros((N, K // 64), dtype=np.uint16)
    y, a = oracle.qmv(x, pack_codes(q, 8), ones, zeros, K, 8, lib=lib)
    want = xi.astype(np.int64) @ q.astype(np.int64).T
    assert np.array_equal(y, want.astype(np.float64))
    assert np.array_equal(a, (np.abs(xi) @ q.astype(np.int64).T).astype(np.float64))


def pin_constant_code_closed_form(lib):
    for bits, c in ((4, 11), (8, 200)):
        g = np.random.default_rng(bits)
        N, K = 3, 256
        q = np.full((N, K), c, dtype=np.uint8)
        s = bf16_bits((0.01 + 0.02 * g.random((N, K // 64))).astype(np.float32))
        b = bf16_bits((-0.1 * g.random((N, K // 64))).astype(np.float32))
        x = bf16_bits(g.standard_normal((1, K)).astype(np.float32))
        y, a = oracle.qmv(x, pack_codes(q, bits), s, b, K, bits, lib=lib)
        for n in range(N):
            want = Fraction(0)
            for gi in range(K // 64):
                xs = sum((_frac_bf16(x[0, k]) for k in range(64 * gi, 64 * gi + 64)), Fraction(0))
                want += (_frac_bf16(s[n, gi]) * c + _frac_bf16(b[n, gi])) * xs
            assert abs(y[0, n] - float(want)) <= 2 * K * U53 * a[0, n]
    # a single group value everywhere: (s*c + b) * sum(x)
    K = 128
    x = bf16_bits(np.linspace(-1, 1, K).astype(np.float32))[None]
    y, _ = oracle.qmv(x, pack_codes(np.full((1, K), 3, np.uint8), 4),
                      np.full((1, 2), 0x3F00, np.uint16), np.full((1, 2), 0xBF80, np.uint16), K, 4, lib=lib)
    assert y[0, 0] == 0.5 * float(bf16_to_f32(x).astype(np.float64).sum())


def pin_gather_bruteforce(lib):
    bits, E, N, K, R = 4, 3, 5, 128, 4
    x, q, s, b = _random_problem(31, R, N, K, bits, E=E)
    lhs = np.array([0, 0, 1, 2, 3, 3], dtype=np.uint32)
    rhs = np.array([2, 0, 1, 1, 0, 2], dtype=np.uint32)
    y, a = oracle.gather_qmv(x, pack_codes(q, bits), s, b, lhs, rhs, K, bits, lib=lib)
    for p in range(len(lhs)):
        for n in range(N):
            ye, ae = _exact_row(x[lhs[p]], q[rhs[p], n], s[rhs[p], n], b[rhs[p], n])
            assert abs(y[p, n] - float(ye)) <= 2 * K * U53 * float(ae), (p, n)
    # NULL indices mean the identity map
    w = pack_codes(q, bits)
    y1, _ = oracle.gather_qmv(x[:3], w, s, b, None, np.array([2, 0, 1], np.uint32), K, bits, lib=lib)
    y2, _ = oracle.gather_qmv(x[:3], w, s, b, np.arange(3, dtype=np.uint32), np.array([2, 0, 1], np.uint32),
                              K, bits, lib=lib)
    assert np.array_equal(y1, y2)
    y3, _ = oracle.gather_qmv(x, w, s, b, np.array([3, 1, 0], np.uint32), None, K, bits, lib=lib)
    y4, _ = oracle.gather_qmv(x, w, s, b, np.array([3, 1, 0], np.uint32), np.arange(3, dtype=np.uint32),
                              K, bits, lib=lib)
    assert np.array_equal(y3, y4)


def pin_row_subset(lib):
    x, q, s, b = _random_problem(3, 2, 9, 128, 8)
    w = pack_codes(q, 8)
    yf, af = oracle.qmv(x, w, s, b, 128, 8, lib=lib)
    rows = np.array([8, 0, 4, 4], dtype=np.int64)
    ys, as_ = oracle.qmv(x, w, s, b, 128, 8, rows=rows, lib=lib)
    assert np.array_equal(ys, yf[:, rows]) and np.array_equal(as_, af[:, rows])
    for bits in (4, 8):
        x, q, s, b = _random_problem(40 + bits, 1, 6, 192, bits)
        ye = [_exact_row(x[0], q[n], s[n], b[n])[0] for n in range(6)]
        ys, as_ = oracle.qmv(x, pack_codes(q, bits), s, b, 192, bits, rows=np.array([5, 1]), lib=lib)
        for i, n in enumerate([5, 1]):
            assert abs(ys[0, i] - float(ye[n])) <= 2 * 192 * U53 * as_[0, i]


def _moe_planes(seed, E, F, H, bits, codes=False):
    """Random gate/up/down planes: dicts of packed w, scales, biases (and the codes)."""
    out = []
    for i, (n, kdim) in enumerate(((F, H), (F, H), (H, F))):
        g = np.random.default_rng([seed, i])
        q = g.integers(0, 2 ** bits, size=(E, n, kdim), dtype=np.uint8)
        sc = bf16_bits((0.01 + 0.02 * g.random((E, n, kdim // 64))).astype(np.float32))
        bi = bf16_bits((-0.05 + 0.03 * g.standard_normal((E, n, kdim // 64))).astype(np.float32))
        d = {"w": pack_codes(q, bits), "scales": sc, "biases": bi}
        if codes:
            d["codes"] = q
        out.append(d)
    return out


def _dense(d, bits):
    """float64 dequantized planes from the codes (independent of the oracle's unpack)."""
    s = bf16_to_f32(d["scales"]).astype(np.float64)
    b = bf16_to_f32(d["biases"]).astype(np.float64)
    return np.repeat(s, 64, axis=-1) * d["codes"].astype(np.float64) + np.repeat(b, 64, axis=-1)


def pin_moe_odd_part_of_silu(lib):
    """Expert 1 is expert 0 with its gate plane negated (bf16 sign flips), the same up and
    down planes; with router weights +1 and -1 the silu terms cancel to the polynomial
    W_down (g * u), computed here from the codes."""
    bits, H, F = 4, 128, 192
    gate, up, down = _moe_planes(50, 1, F, H, bits, codes=True)
    neg = {k: v.copy() for k, v in gate.items()}
    neg["scales"] = neg["scales"] ^ np.uint16(0x8000)
    neg["biases"] = neg["biases"] ^ np.uint16(0x8000)
    g2 = {k: np.concatenate([gate[k], neg[k]]) for k in ("w", "scales", "biases")}
    u2 = {k: np.concatenate([up[k], up[k]]) for k in ("w", "scales", "biases")}
    d2 = {k: np.concatenate([down[k], down[k]]) for k in ("w", "scales", "biases")}
    x = bf16_bits(np.random.default_rng(51).standard_normal((2, H)).astype(np.float32))
    ex = np.array([[0, 1], [1, 0]], np.uint32)
    r = np.array([[1.0, -1.0], [-1.0, 1.0]], np.float32)
    y, a = oracle.moe_swiglu(x, g2, u2, d2, ex, r, bits, lib=lib)
    xd = bf16_to_f32(x).astype(np.float64)
    g = xd @ _dense(gate, bits)[0].T
    u = xd @ _dense(up, bits)[0].T
    want = (g * u) @ _dense(down, bits)[0].T
    assert np.all(np.abs(y - want) <= 1e-12 * a), np.max(np.abs(y - want) / a)


def pin_moe_silu_saturation(lib):
    """Gate planes of constant weight +1 (or -1) against x with 64 ones: every gate value is
    +64 (or -64), silu(64) = 64 and silu(-64) ~ -1e-26 in float64, so h = 64 * u (or ~0)."""
    bits, H, F, E = 4, 128, 64, 2
    _, up, down = _moe_planes(52, E, F, H, bits, codes=True)
    zero = np.zeros((E, F, H // 64), np.uint16)
    x = np.zeros((1, H), np.uint16)
    x[0, 5:69] = 0x3F80
    ex = np.array([[1, 0]], np.uint32)
    r = np.array([[0.75, 0.25]], np.float32)
    xd = bf16_to_f32(x).astype(np.float64)
    for sign, bias in ((1, 0x3F80), (-1, 0xBF80)):
        gate = {"w": np.zeros((E, F, H * bits // 32), np.uint32), "scales": zero,
                "biases": np.full((E, F, H // 64), bias, np.uint16)}
        y, a = oracle.moe_swiglu(x, gate, up, down, ex, r, bits, lib=lib)
        if sign > 0:
            want = np.zeros(H)
            for j in range(2):
                e = int(ex[0, j])
                u = xd[0] @ _dense(up, bits)[e].T
                want += float(r[0, j]) * (_dense(down, bits)[e] @ (64.0 * u))
            assert np.all(np.abs(y[0] - want) <= 1e-12 * a[0]), np.max(np.abs(y[0] - want) / np.maximum(a[0], 1e-300))
        else:
            assert np.all(np.abs(y) <= 1e-20), np.max(np.abs(y))


def pin_moe_bruteforce_tanh_form(lib):
    """Tiny layers in exact rationals for the projections, silu written through tanh
    (sigmoid(z) = (1 + tanh(z/2)) / 2), the down projection and the router sum in float64."""
    for bits in (4, 8):
        T, H, F, E, k = 2, 64, 64, 3, 2
        gate, up, down = _moe_planes(53 + bits, E, F, H, bits, codes=True)
        x = bf16_bits(np.random.default_rng(54 + bits).standard_normal((T, H)).astype(np.float32))
        ex = np.array([[2, 0], [1, 2]], np.uint32)
        r = np.array([[0.625, 0.375], [0.5, 0.5]], np.float32)
        y, a = oracle.moe_swiglu(x, gate, up, down, ex, r, bits, lib=lib)
        for t in range(T):
            want = np.zeros(H)
            for j in range(k):
                e = int(ex[t, j])
                h = np.empty(F)
                for f in range(F):
                    g = float(_exact_row(x[t], gate["codes"][e, f], gate["scales"][e, f], gate["biases"][e, f])[0])
                    u = float(_exact_row(x[t], up["codes"][e, f], up["scales"][e, f], up["biases"][e, f])[0])
                    h[f] = g * 0.5 * (1.0 + math.tanh(0.5 * g)) * u
                want += float(r[t, j]) * (_dense(down, bits)[e] @ h)
            assert np.all(np.abs(y[t] - want) <= 1e-12 * a[t]), (bits, t, np.max(np.abs(y[t] - want) / np.maximum(a[t], 1e-300)))
            # the tolerance scale: sum_j |r| * sum_n |w_down * h|
            assert np.all(a[t] > 0)


def pin_quantize_known_groups(lib):
    """Hand-worked groups: a ramp 1 + 0.5*c over codes c spanning 0 .. 2^bits - 1 gives
    scale 0.5, bias 1 and codes c; a constant group gives scale 0, bias the constant, codes 0; ties round
    to even codes; values beyond the ramp clamp."""
    for bits in (3, 4, 5, 6, 8):
        lv = 2 ** bits - 1
        K = 64
        codes = np.concatenate([[0, lv], np.arange(1, K - 1) % (lv + 1)])  # spans 0 .. 2^bits - 1
        ramp = (1.0 + 0.5 * codes).astype(np.float32)
        const = np.full(K, -0.375, np.float32)
        ties = np.zeros(K, np.float32)
        ties[0], ties[1] = 0.0, float(lv)       # scale 1, bias 0
        ties[2:6] = [0.5, 1.5, 2.5, 3.5]        # half-way values -> even codes 0, 2, 2, 4
        w = np.stack([ramp, const, ties])
        wq, sc, bi = oracle.quantize(w, bits, lib=lib)
        q = oracle.unpack(wq, K, bits, lib=lib)
        assert sc[0, 0] == 0x3F00 and bi[0, 0] == 0x3F80, (bits, hex(sc[0, 0]), hex(bi[0, 0]))
        assert np.array_equal(q[0], codes)
        assert sc[1, 0] == 0 and bi[1, 0] == 0xBEC0 and not q[1].any()
        assert sc[2, 0] == 0x3F80 and bi[2, 0] == 0
        assert q[2, :6].tolist() == [0, lv, 0, 2, 2, 4]


def pin_quantize_properties(lib):
    """On random groups: every code is in range; the scale and bias are the bf16 roundings
    of (max - min)/(2^bits - 1) and min; values strictly inside the code range land within
    half a scale (plus the float32 rounding of (w - b)/s) of their dequantized weight; the
    dequantized weights re-quantize to the same codes, scales and biases wherever the codes
    span the full range (then max and min are exactly representable on the grid)."""
    for bits in (2, 3, 4, 5, 6, 8):
        for gs in (32, 64, 128):
            g = np.random.default_rng([71, bits, gs])
            N, K = 6, 256
            w = (0.02 * g.standard_normal((N, K))).astype(np.float32)
            wq, sc, bi = oracle.quantize(w, bits, gs, lib=lib)
            q = oracle.unpack(wq, K, bits, lib=lib)
            lv = 2 ** bits - 1
            wg = w.reshape(N, K // gs, gs).astype(np.float64)
            s = bf16_to_f32(sc).astype(np.float64)
            b = bf16_to_f32(bi).astype(np.float64)
            assert np.array_equal(sc, bf16_bits(((wg.max(-1) - wg.min(-1)).astype(np.float32) /
                                                 np.float32(lv)).astype(np.float32)))
            assert np.array_equal(bi, bf16_bits(wg.min(-1).astype(np.float32)))
            qg = q.reshape(N, K // gs, gs).astype(np.float64)
            what = s[..., None] * qg + b[..., None]
            inner = ((wg - b[..., None]) / s[..., None] > 0.5) & ((wg - b[..., None]) / s[..., None] < lv - 0.5)
            err = np.abs(wg - what)
            assert np.all(err[inner] <= (0.5 + 1e-5) * np.broadcast_to(s[..., None], err.shape)[inner])
            deq, _ = oracle.dequantize(wq, sc, bi, K, bits, gs, lib=lib)
            wq2, sc2, bi2 = oracle.quantize(deq.astype(np.float32), bits, gs, lib=lib)
            full = (qg.min(-1) == 0) & (qg.max(-1) == lv)
            assert full.any()
            q2 = oracle.unpack(wq2, K, bits, lib=lib).reshape(N, K // gs, gs)
            assert np.array_equal(sc2[full], sc[full]) and np.array_equal(bi2[full], bi[full])
            assert np.array_equal(q2[full], qg[full].astype(np.uint8))


def pin_quantize_packs_like_the_producer(lib):
    """The oracle quantizer's packed words, scales and biases equal the producer's (quantize_rows,
    then pack_codes: the same recipe and bit stream written independently), at every width."""
    for bits in (2, 3, 4, 5, 6, 8):
        g = np.random.default_rng([72, bits])
        w = (0.02 * g.standard_normal((5, 320))).astype(np.float32)
        wq, sc, bi = oracle.quantize(w, bits, lib=lib)
        q, s2, b2 = quantize_rows(w, bits)
        assert np.array_equal(sc, s2) and np.array_equal(bi, b2), bits
        assert np.array_equal(wq, pack_codes(q, bits)), bits


def pin_quantize_codes_are_nearest(lib):
    """Each code is the grid point s*q + b (q in 0 .. 2^bits - 1) nearest to its weight, up to
    the float32 rounding of (w - b)/s. Groups offset far from zero (8-bit) make rounding the
    scale and bias push some weights past either end of the grid, which only a clamp fixes."""
    for bits in (4, 8):
        lv = 2 ** bits - 1
        g = np.random.default_rng([72, bits])
        N, K = 64, 64
        w = (0.02 * g.standard_normal((N, K))).astype(np.float32)
        w[N // 2:] += (100 * g.random((N // 2, 1)) + 1).astype(np.float32)  # offset groups
        wq, sc, bi = oracle.quantize(w, bits, lib=lib)
        q = oracle.unpack(wq, K, bits, lib=lib).astype(np.int64)
        s = bf16_to_f32(sc).astype(np.float64)[:, :1]
        b = bf16_to_f32(bi).astype(np.float64)[:, :1]
        grid = s[:, :, None] * np.arange(lv + 1)[None, None, :] + b[:, :, None]  # [N, 1, levels]
        dist = np.abs(w.astype(np.float64)[:, :, None] - grid)
        best = dist.min(-1)
        got = np.take_along_axis(dist, q[:, :, None], -1)[..., 0]
        assert np.all(got <= best + 1e-4 * s), np.max((got - best) / s)
        outside = (w < b - 0.5 * s) | (w > b + (lv + 0.5) * s)
        if bits == 8:
            assert outside.any()  # the case needs clamping


def pin_bf16_round_known_values(lib):
    """Ties go to the even neighbour, everything else to the nearest: 1 + 2^-8 -> 1,
    1 + 3*2^-8 -> 1 + 2^-6, 1 + 2^-8 + 2^-20 -> 1 + 2^-7, and the mirror images; on
    doubles that are binary32 values the result is the bf16 RNE of that binary32 value."""
    f = lib.agqo_bf16_round
    for v, want in ((1 + 2 ** -8, 1.0), (1 + 3 * 2 ** -8, 1 + 2 ** -6), (1 + 2 ** -8 + 2 ** -20, 1 + 2 ** -7),
                    (3.0, 3.0), (0.0, 0.0), (2 ** -130 * 1.5, 2 ** -130 * 1.5)):
        assert f(v) == want and f(-v) == -want, (v, f(v), want)
    vals = np.random.default_rng(90).standard_normal(2000).astype(np.float32)
    want = bf16_to_f32(bf16_bits(vals)).astype(np.float64)
    assert all(f(float(v)) == w for v, w in zip(vals, want))


def _fused_problem(seed, N, K, bits=4):
    g = np.random.default_rng([91, seed])
    q = g.integers(0, 2 ** bits, size=(N, K), dtype=np.uint8)
    sc = bf16_bits((0.01 + 0.02 * g.random((N, K // 64))).astype(np.float32))
    bi = bf16_bits((-0.05 + 0.03 * g.standard_normal((N, K // 64))).astype(np.float32))
    return q, sc, bi, g


def pin_fused_reduces_to_qmv(lib):
    """Without a norm and with no epilogue the fused projection is the plain product."""
    q, sc, bi, g = _fused_problem(1, 9, 192)
    x = bf16_bits(g.standard_normal((1, 192)).astype(np.float32))
    w = pack_codes(q, 4)
    y, a = oracle.qmv_fused(x, w, sc, bi, 192, 4, lib=lib)
    y0, a0 = oracle.qmv(x, w, sc, bi, 192, 4, lib=lib)
    assert np.array_equal(y, y0[0]) and np.array_equal(a, a0[0])


def pin_fused_norm_closed_forms(lib):
    """x of constant magnitude c with eps = 0 normalizes to the sign vector exactly; a norm
    weight of 2 doubles the product exactly; scaling x by a power of two changes nothing;
    a zero norm weight gives zero; with identity-like weights (8-bit, scale 1, bias 0, one
    code 1 per row) every output is one normalized activation, hence a bf16 value."""
    K, N = 256, 7
    q, sc, bi, g = _fused_problem(2, N, K)
    w = pack_codes(q, 4)
    sign = np.where(g.random(K) < 0.5, -1.0, 1.0)
    x = bf16_bits((0.09375 * sign).astype(np.float32))[None]
    ones = np.full(K, 0x3F80, np.uint16)
    y, _ = oracle.qmv_fused(x, w, sc, bi, K, 4, gamma=ones, eps=0.0, lib=lib)
    ys, _ = oracle.qmv(bf16_bits(sign.astype(np.float32))[None], w, sc, bi, K, 4, lib=lib)
    assert np.array_equal(y, ys[0])
    xr = bf16_bits(g.standard_normal(K).astype(np.float32))[None]
    gam = bf16_bits((0.5 + g.random(K)).astype(np.float32))
    y1, _ = oracle.qmv_fused(xr, w, sc, bi, K, 4, gamma=gam, eps=0.0, lib=lib)
    y8, _ = oracle.qmv_fused(bf16_bits(8 * bf16_to_f32(xr)), w, sc, bi, K, 4, gamma=gam, eps=0.0, lib=lib)
    assert np.array_equal(y1, y8)
    yo, _ = oracle.qmv_fused(xr, w, sc, bi, K, 4, gamma=ones, eps=1e-3, lib=lib)
    y2, _ = oracle.qmv_fused(xr, w, sc, bi, K, 4, gamma=np.full(K, 0x4000, np.uint16), eps=1e-3, lib=lib)
    assert np.array_equal(y2, 2 * yo)
    yz, _ = oracle.qmv_fused(xr, w, sc, bi, K, 4, gamma=np.zeros(K, np.uint16), lib=lib)
    assert not yz.any()
    eye = np.zeros((64, 64), np.uint8)
    eye[np.arange(64), np.arange(64)] = 1
    yi, _ = oracle.qmv_fused(xr[:, :64], pack_codes(eye, 8), np.full((64, 1), 0x3F80, np.uint16),
                             np.zeros((64, 1), np.uint16), 64, 8, gamma=gam[:64], eps=0.5, lib=lib)
    assert np.array_equal(yi, bf16_to_f32(bf16_bits(yi.astype(np.float32))).astype(np.float64))
    assert np.array_equal(yi.astype(np.float32).astype(np.float64), yi)


def pin_fused_residual(lib):
    q, sc, bi, g = _fused_problem(3, 11, 128)
    w = pack_codes(q, 4)
    x = bf16_bits(g.standard_normal((1, 128)).astype(np.float32))
    res = bf16_bits(g.standard_normal(11).astype(np.float32))
    y0, _ = oracle.qmv_fused(x, w, sc, bi, 128, 4, lib=lib)
    y1, _ = oracle.qmv_fused(x, w, sc, bi, 128, 4, residual=res, lib=lib)
    assert np.all(np.abs((y1 - y0) - bf16_to_f32(res)) <= 4e-16 * (np.abs(y1) + 1))


def pin_fused_glu_odd_part(lib):
    """Gate rows g and -g (bf16 sign flips) with the same up row: the outputs differ by
    exactly g * u for SwiGLU and GeGLU alike (both activations have odd part z / 2)."""
    K = 192
    q, sc, bi, g = _fused_problem(4, 2, K)  # row 0: gate, row 1: up
    x = bf16_bits(g.standard_normal((1, K)).astype(np.float32))
    plain, _ = oracle.qmv(x, pack_codes(q, 4), sc, bi, K, 4, lib=lib)
    gv, uv = plain[0]
    q4 = np.stack([q[0], q[1], q[0], q[1]])
    sc4 = np.stack([sc[0], sc[1], sc[0] ^ np.uint16(0x8000), sc[1]])
    bi4 = np.stack([bi[0], bi[1], bi[0] ^ np.uint16(0x8000), bi[1]])
    for act in (oracle.ACT_SWIGLU, oracle.ACT_GEGLU):
        y, a = oracle.qmv_fused(x, pack_codes(q4, 4), sc4, bi4, K, 4, act=act, lib=lib)
        assert abs((y[0] - y[1]) - gv * uv) <= 1e-13 * (abs(y[0]) + abs(y[1])), (act, y, gv * uv)


def pin_fused_glu_values(lib):
    """Gate rows of constant weight w_g against x of 64 ones give gate value 64*w_g: at 64
    both activations return 64, at -64 about 0, at 1 silu(1) = e/(1 + e) = 0.7310585786300049
    and the tanh form of gelu 0.5*(1 + tanh(sqrt(2/pi)*1.044715)) = 0.8411919906082768.
    The up row has constant weight 1/2 (up value 32)."""
    K = 64
    x = np.full((1, K), 0x3F80, np.uint16)
    zero = np.zeros((2, 1), np.uint16)
    for gate_bias, want in ((0x3F80, {1: 64.0, 2: 64.0}), (0xBF80, {1: 0.0, 2: 0.0}),
                            (0x3C80, {1: 0.7310585786300049, 2: 0.8411919906082768})):
        b = np.array([[gate_bias], [0x3F00]], np.uint16)
        for act in (1, 2):
            y, _ = oracle.qmv_fused(x, np.zeros((2, K // 8), np.uint32), zero, b, K, 4, act=act, lib=lib)
            assert abs(y[0] - 32.0 * want[act]) <= 1e-12 * 32.0, (hex(gate_bias), act, y[0])


def pin_e2m1_values(lib):
    """The E2M1 value set of the NVFP4 format: magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6 for codes
    0..7, and the sign bit (code | 8) negates."""
    want = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    for c in range(8):
        assert lib.agqo_e2m1(c) == want[c], (c, lib.agqo_e2m1(c))
        assert lib.agqo_e2m1(c | 8) == -want[c]
        assert math.copysign(1.0, lib.agqo_e2m1(c | 8)) == -1.0


def pin_e4m3_matches_torch(lib):
    """Every E4M3 byte decodes as torch's float8_e4m3fn does (an independent decoder), NaN
    for S.1111.111; spot values 0x38 = 1, 0x7E = 448, 0x08 = 2^-6, 0x01 = 2^-9."""
    torch = pytest.importorskip("torch")
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = np.array([lib.agqo_e4m3(b) for b in range(256)])
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])
    assert (lib.agqo_e4m3(0x38), lib.agqo_e4m3(0x7E), lib.agqo_e4m3(0x08), lib.agqo_e4m3(0x01)) == \
        (1.0, 448.0, 2.0 ** -6, 2.0 ** -9)


def _nvfp4_problem(seed, N, K):
    g = np.random.default_rng([95, seed])
    q = g.integers(0, 16, size=(N, K), dtype=np.uint8)
    sc = g.integers(0x20, 0x50, size=(N, K // 16), dtype=np.uint8)  # E4M3 scales 2^-4 .. 2^2
    x = bf16_bits(g.standard_normal((2, K)).astype(np.float32))
    return q, sc, x


def pin_nvfp4_bruteforce(lib):
    """Exact rational brute force from the codes before packing (values from the E2M1 and
    E4M3 tables written out here), at two tensor scales."""
    e2m1 = [Fraction(v) for v in (0, 0.5, 1, 1.5, 2, 3, 4, 6)]

    def e4m3(b):
        e, m = (b >> 3) & 15, b & 7
        mag = Fraction(m, 8) * Fraction(1, 64) if e == 0 else (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7)
        return -mag if b & 0x80 else mag

    N, K = 5, 48
    q, sc, x = _nvfp4_problem(1, N, K)
    w = pack_codes(q, 4)
    for ts in (1.0, 0.375):
        y, a = oracle.qmv_nvfp4(x, w, sc, ts, K, lib=lib)
        xf = bf16_to_f32(x).astype(np.float64)
        for m in range(2):
            for n in range(N):
                exact = sum(Fraction(float(xf[m, k])) * (e2m1[q[n, k] & 7] * (-1 if q[n, k] & 8 else 1)) *
                            e4m3(int(sc[n, k // 16])) * Fraction(ts) for k in range(K))
                assert abs(Fraction(y[m, n]) - exact) <= Fraction(1, 2 ** 40) * (abs(exact) + 1), (m, n)


def pin_nvfp4_closed_forms(lib):
    """A constant code c and scale byte b give e2m1(c) * e4m3(b) * ts * sum(x); doubling the
    tensor scale doubles y exactly; the row subset selects rows."""
    K, N = 64, 3
    x = bf16_bits(np.random.default_rng(96).standard_normal((1, K)).astype(np.float32))
    sx = float(np.sum(bf16_to_f32(x).astype(np.float64)))
    for c, b, v in ((3, 0x38, 1.5), (15, 0x40, -12.0), (9, 0x30, -0.25)):
        w = pack_codes(np.full((N, K), c, np.uint8), 4)
        sc = np.full((N, K // 16), b, np.uint8)
        y, a = oracle.qmv_nvfp4(x, w, sc, 0.5, K, lib=lib)
        assert np.allclose(y, v * 0.5 * sx, rtol=1e-14, atol=1e-14), (c, b, y, v * sx)
        ax = float(np.sum(np.abs(bf16_to_f32(x).astype(np.float64))))
        assert np.allclose(a, abs(v) * 0.5 * ax, rtol=1e-14), (c, b, a)
    q, sc, xx = _nvfp4_problem(2, 7, 128)
    w = pack_codes(q, 4)
    y1, _ = oracle.qmv_nvfp4(xx, w, sc, 1.0, 128, lib=lib)
    y2, _ = oracle.qmv_nvfp4(xx, w, sc, 2.0, 128, lib=lib)
    assert np.array_equal(y2, 2 * y1)
    ys, _ = oracle.qmv_nvfp4(xx, w, sc, 1.0, 128, rows=np.array([6, 0, 3]), lib=lib)
    assert np.array_equal(ys, y1[:, [6, 0, 3]])


PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
