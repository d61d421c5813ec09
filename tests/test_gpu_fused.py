"""GPU parity of the fused batch-1 projection (RMS-norm prologue, residual / SwiGLU / GeGLU
epilogue) against the oracle's agqo_qmv_fused.

Tolerances:
 * act 0: |y - y_ref| <= 2e-3 * (A + |residual|) + half a bf16 ulp of y_ref, A = sum_k |x_n,k w_k|;
 * acts 1, 2: |y - y_ref| <= 2e-3 * a + half a bf16 ulp, a = 1.13 |u| A_gate + |act(g)| A_up
   (the oracle's bound for the gated forms: 1.13 bounds the slope of both activations).
The normalized activation is rounded to bf16 on both sides, from an fp32 value here and an
exact one in the oracle; the two roundings can differ by one bf16 ulp where the exact value
lies within fp32 error of a rounding midpoint. The one-hot tests check that directly: each
GPU x_n equals the oracle's except in that band, where either neighbour is accepted.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import seeded_inputs as si
from gpu_util import REL_TOL, bf16_bits_host, bf16_dev, bf16_host, half_ulp_bf16, progress, u32_dev

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("no GPU", allow_module_level=True)

import affine_group_quantized_amd as agq  # noqa: E402


def check(y_gpu, y_ref, a, what, res=None):
    y = bf16_host(y_gpu).reshape(y_ref.shape)
    tol = REL_TOL * (a + (0 if res is None else np.abs(res))) + half_ulp_bf16(y_ref)
    err = np.abs(y - y_ref)
    bad = ~(err <= tol)
    if bad.any():
        i = int(np.argmax(np.where(bad, err / np.maximum(tol, 1e-300), 0)))
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} outside tolerance; worst at {i}: "
                             f"gpu={y[i]!r} ref={y_ref[i]!r} a={a[i]!r}")


def rows_of(d, rows):
    return d["w"][rows], d["scales"][rows], d["biases"][rows]


def sample_rows(N, act, count, seed):
    """Sorted sample of weight rows (act 0) or of interleaved gate/up pairs (acts 1, 2),
    always including the first and last."""
    g = np.random.default_rng(seed)
    units = N if act == 0 else N // 2
    pick = np.unique(np.concatenate([[0, units - 1], g.choice(units, min(count, units), replace=False)]))
    if act == 0:
        return pick, pick
    return pick, np.stack([2 * pick, 2 * pick + 1], axis=1).reshape(-1)


def run_case(d, x, bits, gs, act, gamma=None, eps=1e-5, res=None, sample=None, what="", seed=0, inplace=False):
    N, K = d["w"].shape[0], x.shape[-1]
    wd, sd, bd = u32_dev(d["w"]), bf16_dev(d["scales"]), bf16_dev(d["biases"])
    gd = None if gamma is None else bf16_dev(gamma)
    rd = None if res is None else bf16_dev(res)
    progress(f"fused {what} N={N} K={K} bits={bits} gs={gs} act={act} norm={gamma is not None} "
             f"res={res is not None}{' in-place' if inplace else ''}")
    out = rd if inplace else None
    y = agq.qmv_fused(bf16_dev(x), wd, sd, bd, bits=bits, group_size=gs, norm_weight=gd, eps=eps, residual=rd,
                      act=act, out=out)
    torch.cuda.synchronize()
    outs, rows = (np.arange(N if act == 0 else N // 2), np.arange(N)) if sample is None else \
        sample_rows(N, act, sample, seed)
    w, s, b = rows_of(d, rows)
    r = None if res is None else res[rows]
    y_ref, a = oracle.qmv_fused(x, w, s, b, K, bits, group_size=gs, gamma=gamma, eps=eps, residual=r, act=act)
    check(y[torch.as_tensor(outs, device=y.device)], y_ref, a, what,
          None if r is None else si.bf16_to_f32(r).astype(np.float64))
    return y


def quantized(seed, N, K, bits, gs=64):
    w = (0.02 * np.random.default_rng([90, seed]).standard_normal((N, K))).astype(np.float32)
    q, sc, bi = si.quantize_rows(w, bits, group_size=gs)
    return {"w": si.pack_codes(q, bits), "scales": sc, "biases": bi}


def norm_weight(seed, K):
    return si.bf16_bits((1 + 0.1 * np.random.default_rng([91, seed]).standard_normal(K)).astype(np.float32))


# ----------------------------------------------------------------------------
# The Llama-shaped decode layer (workload 1's projections, the decode_layer inputs).

@pytest.fixture(scope="module")
def layer():
    return si.workload(1), si.decode_layer()


def test_decode_layer_attention_side(layer):
    wl, dl = layer
    x = dl["h"][None]
    # norm -> concatenated q/k/v (6144 rows), every row checked
    run_case(wl["qkv"], x, 4, 64, 0, gamma=dl["gamma_attn"], eps=dl["eps"], what="qkv")
    # o projection with the residual added in place (y is the residual buffer)
    xo = wl["x4096"]
    run_case(wl["o"], xo, 4, 64, 0, res=dl["h"], what="o+residual", inplace=True)


def test_decode_layer_mlp_side(layer):
    wl, dl = layer
    # norm -> interleaved gate/up (28672 rows) -> SwiGLU, every pair checked
    run_case(wl["gate_up"], dl["h"][None], 4, 64, 1, gamma=dl["gamma_mlp"], eps=dl["eps"], what="gate_up swiglu")
    # down projection (K = 14336: two K segments) with the residual
    run_case(wl["down"], wl["x14336"], 4, 64, 0, res=dl["h"], what="down+residual")
    # the same projection with a norm in front (sum of squares across the K split)
    run_case(wl["down"], wl["x14336"], 4, 64, 0, gamma=norm_weight(1, 14336), res=dl["h"], what="norm+down")


def test_decode_layer_final_norm_and_logits(layer):
    wl, dl = layer
    # 128256 rows: the deep plan, x staged by each wave; sampled rows
    run_case(wl["lm_head"], dl["h"][None], 4, 64, 0, gamma=dl["gamma_final"], eps=dl["eps"], sample=4096,
             what="final norm + lm_head", seed=3)


# ----------------------------------------------------------------------------
# Plans and shapes: every instantiated form, ragged rows and edge cases.

@pytest.mark.parametrize("N,K,bits,gs,act", [
    (2, 64, 4, 64, 1), (6, 64, 8, 32, 2), (14, 192, 4, 64, 0), (1000, 1024, 4, 128, 1),
    (999, 4160, 4, 64, 0), (2050, 8192, 4, 64, 2), (513, 2048, 8, 64, 0), (1538, 4096, 8, 128, 1),
    (4864 * 2, 896, 8, 64, 2), (896, 4864, 8, 64, 0), (300, 14336, 8, 64, 1), (64, 65536, 4, 64, 0),
    (130, 32768, 8, 32, 2), (4096, 12288, 4, 64, 1),
    # large 4-bit grids with one chunk of K (ragged rows, a partial chunk, one group)
    (8194, 1088, 4, 64, 1), (8202, 64, 4, 64, 0), (16390, 4096, 4, 64, 2), (8210, 4096, 4, 64, 0),
])
def test_fused_shapes(N, K, bits, gs, act):
    d = quantized(N * 7 + K + bits, N, K, bits, gs)
    x = si.draw_activations(90, N + K, 1, K)
    res = si.draw_activations(92, N, 1, N)[0] if act == 0 and N % 2 == 0 else None
    run_case(d, x, bits, gs, act, gamma=norm_weight(N + K, K), eps=1e-5, res=res, what="shape")
    # the same weights without the norm (and for act 0 without the residual)
    run_case(d, x, bits, gs, act, what="no norm")


@pytest.mark.parametrize("act", [0, 1, 2])
def test_fused_gated_deep_plan(act):
    """A row walk long enough for the deep plan (per-wave norm), gated rows in pairs."""
    N, K = 65536, 4096
    d = {"w": np.random.default_rng(93).integers(0, 2 ** 32, size=(N, K // 8), dtype=np.uint32),
         "scales": si.bf16_bits((0.001 + 0.002 * np.random.default_rng(94).random((N, K // 64))).astype(np.float32)),
         "biases": si.bf16_bits((-0.015 * np.random.default_rng(95).random((N, K // 64))).astype(np.float32))}
    x = si.draw_activations(93, 1, 1, K)
    res = si.draw_activations(94, 1, 1, N)[0] if act == 0 else None
    run_case(d, x, 4, 64, act, gamma=norm_weight(7, K), eps=1e-6, res=res, sample=2048, what="deep", seed=act)


def test_fused_large_grid_inplace_residual():
    """A large 4-bit grid with the residual buffer as y (the in-place residual add)."""
    N, K = 8200, 4096
    d = quantized(13, N, K, 4)
    x = si.draw_activations(99, 0, 1, K)
    res = si.draw_activations(100, 0, 1, N)[0]
    run_case(d, x, 4, 64, 0, gamma=norm_weight(5, K), eps=1e-5, res=res, what="large grid in-place", inplace=True)


def test_fused_eps_and_scale():
    """A large eps dominates the mean square; x scaled by 2^20 with eps = 0 normalizes to the
    same activation as x (exact in both implementations up to the rounding band)."""
    N, K = 512, 4096
    d = quantized(11, N, K, 4)
    x = si.draw_activations(95, 0, 1, K)
    run_case(d, x, 4, 64, 0, gamma=norm_weight(3, K), eps=100.0, what="eps=100")
    xs = si.bf16_bits(si.bf16_to_f32(x) * np.float32(2 ** 20))
    y1 = run_case(d, x, 4, 64, 1, gamma=norm_weight(3, K), eps=0.0, what="eps=0")
    y2 = run_case(d, xs, 4, 64, 1, gamma=norm_weight(3, K), eps=0.0, what="eps=0, x * 2^20")
    # rs scales by exactly 2^-20 in fp32 too, so the two normalized rows match bit for bit
    assert torch.equal(y1, y2)


def test_fused_is_deterministic():
    N, K = 6144, 4096
    d = quantized(12, N, K, 4)
    x = bf16_dev(si.draw_activations(96, 0, 1, K))
    args = (u32_dev(d["w"]), bf16_dev(d["scales"]), bf16_dev(d["biases"]))
    g = bf16_dev(norm_weight(4, K))
    progress("fused determinism")
    a = agq.qmv_fused(x, *args, norm_weight=g, act=1)
    b = agq.qmv_fused(x, *args, norm_weight=g, act=1)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


# ----------------------------------------------------------------------------
# The normalized activation itself, through one-hot rows: y[n] = x_n[c_n] exactly.
# 8-bit codes: their products are exact fp32 FMAs (code 0 or 1, scale 1, bias 0), while
# the 4-bit form cancels a 128 offset in fp32 and is exact only up to rounding noise. The
# norm is applied to the raw activation words before the code-width-specific staging.

def one_hot_rows(cols, K):
    """8-bit rows with code 1 at column cols[n] and 0 elsewhere, scale 1, bias 0."""
    N = len(cols)
    w = np.zeros((N, K // 4), np.uint32)
    w[np.arange(N), cols // 4] = np.left_shift(np.uint32(1), (8 * (cols % 4)).astype(np.uint32))
    G = K // 64
    return {"w": w, "scales": np.full((N, G), 0x3F80, np.uint16), "biases": np.zeros((N, G), np.uint16)}


@pytest.mark.parametrize("K,N", [
    (64, 64),        # one chunk per lane
    (4096, 1600),    # one K segment, the block's LDS copy
    (8192, 1600),    # two K segments sharing the LDS copy
    (14336, 1600),   # four K segments, x staged per wave
    (32768, 1600),   # eight K segments
    (4096, 65536),   # the deep plan: one segment, x staged per wave
])
def test_norm_rounding_on_one_hot_rows(K, N):
    g = np.random.default_rng([97, K, N])
    cols = (np.arange(N) % K) if N >= K else np.sort(g.choice(K, N, replace=False))
    d = one_hot_rows(cols, K)
    x = si.draw_activations(97, K, 1, K)
    gamma = norm_weight(K, K)
    eps = 1e-5
    progress(f"fused one-hot norm K={K} N={N}")
    y = agq.qmv_fused(bf16_dev(x), u32_dev(d["w"]), bf16_dev(d["scales"]), bf16_dev(d["biases"]), bits=8,
                      norm_weight=bf16_dev(gamma), eps=eps)
    torch.cuda.synchronize()
    got = bf16_bits_host(y)
    # the oracle's x_n for every column (one identity row per column)
    ident = one_hot_rows(np.arange(K), K)
    ref_all, _ = oracle.qmv_fused(x, ident["w"], ident["scales"], ident["biases"], K, 8, gamma=gamma, eps=eps)
    ref = ref_all[cols]
    want = si.bf16_bits(ref.astype(np.float32))
    assert np.array_equal(si.bf16_to_f32(want).astype(np.float64), ref)  # the oracle's x_n are bf16
    # exact value x * rs * gamma, and its distance to the nearest bf16 rounding midpoint
    xf = si.bf16_to_f32(x[0]).astype(np.float64)
    rs = 1.0 / np.sqrt(np.sum(xf * xf) / K + eps)
    v = xf[cols] * rs * si.bf16_to_f32(gamma[cols]).astype(np.float64)
    ulp = 2 * half_ulp_bf16(v)
    frac = np.abs(v) / ulp - np.floor(np.abs(v) / ulp)
    near_mid = np.abs(frac - 0.5) * ulp <= 2.0 ** -16 * np.abs(v)  # fp32 error band of x * rs * gamma
    diff = got != want
    assert not (diff & ~near_mid).any(), np.flatnonzero(diff & ~near_mid)[:8]
    assert (np.abs(si.bf16_to_f32(got).astype(np.float64) - ref) <= ulp).all()
    # and with a residual: y = x_n + r, one fp32 add and one rounding
    if N == 1600:
        r = si.draw_activations(98, K, 1, N)[0]
        y2 = agq.qmv_fused(bf16_dev(x), u32_dev(d["w"]), bf16_dev(d["scales"]), bf16_dev(d["biases"]), bits=8,
                           norm_weight=bf16_dev(gamma), eps=eps, residual=bf16_dev(r))
        torch.cuda.synchronize()
        xn = si.bf16_to_f32(got)
        assert np.array_equal(bf16_bits_host(y2), si.bf16_bits(xn + si.bf16_to_f32(r)))
