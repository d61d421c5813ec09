"""GPU parity: libagq through its C ABI against the CPU oracle, element by element.

Tolerance: |y_gpu - y_ref| <= 2e-3 * sum_k |x_k * w_hat_k| per output element,
with w_hat the dequantized weight. The adversarial closed-form cases, where
|y| equals that sum, also allow half a bf16 ulp for the output rounding.
Dequantization is compared bit for bit.

Full-size workloads run in the launch configuration the benchmark uses, and
the oracle checks every output row of every one of them (it streams about
0.2 GB/s, so the largest, lm_head, takes under two seconds).
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import seeded_inputs as si
from gpu_util import bf16_bits_host, bf16_dev, bf16_host, check_close, progress, u32_dev

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("no GPU", allow_module_level=True)

import affine_group_quantized_amd as agq  # noqa: E402  (loads libagq.so; fails loudly if missing)


def dev_weight(d):
    return u32_dev(d["w"]), bf16_dev(d["scales"]), bf16_dev(d["biases"])


@pytest.fixture(scope="module")
def wl():
    cache = {}

    def get(cfg):
        if cfg not in cache:
            progress(f"generating workload {cfg}")
            cache[cfg] = si.workload(cfg)
        return cache[cfg]
    return get


def run_qmv_case(name, x, d, K, bits, rows=None, M=None):
    w, s, b = dev_weight(d)
    xd = bf16_dev(x)
    N = d["w"].shape[0]
    progress(f"{name}: N={N} K={K} bits={bits} M={x.shape[0]}")
    if x.shape[0] == 1 and M is None:
        y = agq.qmv(xd[0], w, s, b, bits=bits)[None]
    else:
        y = agq.qmv_wide(xd, w, s, b, bits=bits)
    torch.cuda.synchronize()
    y_ref, A = oracle.qmv(x, d["w"], d["scales"], d["biases"], K, bits, rows=rows)
    yg = y if rows is None else y[:, torch.as_tensor(rows, device=y.device)]
    worst = check_close(yg, y_ref, A, name)
    progress(f"{name}: ok, worst |err|/A = {worst:.3e}")
    return y


# ---------------------------------------------------------------- dequantize


@pytest.mark.parametrize("bits,N,K", [(4, 4096, 4096), (8, 4864, 896), (8, 896, 4864), (4, 7, 64), (4, 33, 1088)])
def test_dequantize_bit_exact(bits, N, K):
    d = si.draw_quantized_weight(5, bits, N, K, bits)
    w, s, b = dev_weight(d)
    progress(f"dequantize bits={bits} N={N} K={K}")
    out = agq.dequantize(w, s, b, bits=bits)
    torch.cuda.synchronize()
    ref, not_f32 = oracle.dequantize(d["w"], d["scales"], d["biases"], K, bits)
    assert not_f32 == 0
    got = out.cpu().numpy()
    assert np.array_equal(got.view(np.uint32), ref.astype(np.float32).view(np.uint32))


def test_dequantize_expert_planes(wl):
    d = si.draw_quantized_weight(6, 1, 3 * 96, 256, 4)
    w = u32_dev(d["w"].reshape(3, 96, -1))
    s = bf16_dev(d["scales"].reshape(3, 96, -1))
    b = bf16_dev(d["biases"].reshape(3, 96, -1))
    progress("dequantize planes [3,96,256]")
    out = agq.dequantize(w, s, b, bits=4)
    torch.cuda.synchronize()
    ref, _ = oracle.dequantize(d["w"], d["scales"], d["biases"], 256, 4)
    assert out.shape == (3, 96, 256)
    assert np.array_equal(out.cpu().numpy().reshape(-1, 256), ref.astype(np.float32))


# ---------------------------------------------------------------- workloads


def test_workload0_qmv_4096(wl):
    d = wl(0)
    run_qmv_case("w0 qmv 4096x4096", d["x"], d["w"], 4096, 4)


@pytest.mark.parametrize("name", ["qkv", "o", "gate_up", "down", "lm_head"])
def test_workload1_llama_gemv_set(wl, name):
    d = wl(1)
    m = d[name]
    run_qmv_case(f"w1 {name}", d[m["x"]], m, m["K"], 4)


@pytest.mark.parametrize("M", [2, 4, 8])
@pytest.mark.parametrize("name", ["w_a", "w_b"])
def test_workload2_qmv_wide(wl, name, M):
    d = wl(2)
    m = d[name]
    run_qmv_case(f"w2 {name} M={M}", d[m["x"]][:M], m, m["K"], 4, M=M)


@pytest.mark.parametrize("name", ["gate_up", "down", "qkv", "lm_head"])
def test_workload3_8bit(wl, name):
    d = wl(3)
    m = d[name]
    run_qmv_case(f"w3 {name}", d[m["x"]], m, m["K"], 8)


@pytest.fixture(scope="module")
def moe():
    progress("generating workload 4 (MoE)")
    return si.workload(4)


@pytest.mark.parametrize("which", ["w1", "w2"])
def test_workload4_gather(moe, which):
    m = moe[which]
    K, N, E = m["K"], m["N"], m["E"]
    if which == "w1":
        x, lhs = moe["x"], moe["lhs1"]
    else:
        x, lhs = moe["h"], None
    rhs = moe["rhs"]
    w = u32_dev(m["w"])
    s = bf16_dev(m["scales"])
    b = bf16_dev(m["biases"])
    progress(f"w4 gather {which}: E={E} N={N} K={K} P={len(rhs)}")
    y = agq.gather_qmv(bf16_dev(x), w, s, b, rhs_indices=u32_dev(rhs),
                       lhs_indices=None if lhs is None else u32_dev(lhs), bits=4)
    torch.cuda.synchronize()
    y_ref, A = oracle.gather_qmv(x, m["w"], m["scales"], m["biases"], lhs, rhs, K, 4)
    worst = check_close(y, y_ref, A, f"w4 {which}")
    progress(f"w4 gather {which}: ok, worst |err|/A = {worst:.3e}")


# ---------------------------------------------------------------- shapes and edges


@pytest.mark.parametrize("bits,M,N,K", [
    (4, 1, 1, 64), (8, 1, 1, 64), (4, 1, 7, 192), (8, 3, 7, 192), (4, 1, 33, 4160), (8, 1, 33, 4160),
    (4, 1, 1001, 896), (8, 1, 1001, 896), (4, 1, 300, 32768), (4, 1, 17, 114688), (8, 1, 9, 57344),
    (4, 5, 129, 1088), (4, 6, 77, 8192), (4, 7, 64, 16384), (8, 7, 64, 8192), (4, 3, 513, 12288),
    (8, 2, 257, 4864), (4, 8, 4099, 4096), (8, 8, 1000, 896), (4, 1, 4097, 4096), (8, 4, 3, 16384),
])
def test_shapes_and_ragged_tails(bits, M, N, K):
    d = si.draw_quantized_weight(7, 100 * bits + M, N, K, bits)
    x = si.draw_activations(7, 1000 + M, M, K)
    run_qmv_case(f"shape M={M}", x, d, K, bits, M=None if M == 1 else M)


@pytest.mark.parametrize("M,N,K", [
    (5, 31, 512), (6, 17, 1536), (8, 1, 2560), (5, 100, 3584), (6, 1000, 4096), (7, 33, 14336),
    (5, 2049, 6144), (7, 4111, 4096), (8, 4097, 2048), (6, 16400, 2048), (8, 16401, 1024),
    (4, 31, 512), (4, 100, 3584), (4, 4111, 4096), (4, 16401, 1024),
])
def test_matrix_core_shapes(M, N, K):
    """4-bit products of several rows on the matrix cores: K splits of 1, 3 and 4 waves,
    bands of one and two tiles, ragged last tiles (rows past N in a load's 8-row half of a
    tile read zeros), and M = 4, whose kernel loads each activation segment once per lane
    group and rotates the words into place."""
    plan = agq.launch_plan(M, N, K, 4)
    assert plan["engine"] == 1
    d = si.draw_quantized_weight(23, M, N, K, 4)
    x = si.draw_activations(23, 100 + M, M, K)
    run_qmv_case(f"mfma M={M} N={N} K={K} S={plan['waves_per_group']} band={plan['rows_per_iter']} "
                 f"xlds={plan['x_lds_bytes']}",
                 x, d, K, 4, M=M)


def test_gather_matrix_core_passes_of_sixteen():
    """33 pairs on one expert (passes of 16, 16 and 1) and 3 on another, repeated x rows."""
    E, N, K, R = 4, 70, 1024, 9
    assert agq.launch_plan(8, N, K, 4, experts=E)["engine"] == 1
    planes = [si.draw_quantized_weight(24, e, N, K, 4) for e in range(E)]
    st = {k: np.stack([p[k] for p in planes]) for k in ("w", "scales", "biases")}
    x = si.draw_activations(24, 99, R, K)
    rhs = np.array([2] * 33 + [0] * 3, np.uint32)
    np.random.default_rng([24, 1]).shuffle(rhs)
    lhs = (np.arange(len(rhs)) * 5 % R).astype(np.uint32)
    progress("gather, passes of 16 on the matrix cores")
    y = agq.gather_qmv(bf16_dev(x), u32_dev(st["w"]), bf16_dev(st["scales"]), bf16_dev(st["biases"]),
                       rhs_indices=u32_dev(rhs), lhs_indices=u32_dev(lhs))
    torch.cuda.synchronize()
    y_ref, A = oracle.gather_qmv(x, st["w"], st["scales"], st["biases"], lhs, rhs, K, 4)
    check_close(y, y_ref, A, "gather passes of 16")


def test_gather_matrix_core_activation_load_forms():
    """Planes with 4, 5, 8, 9 and 16 pairs in one call: each side of the pass sizes at
    which the kernel switches its activation load (one rotated load up to 4 rows, staged
    through LDS up to 8, four loads beyond), over ragged tiles and K split over 2 waves."""
    E, N, K, R = 6, 45, 2048, 13
    assert agq.launch_plan(8, N, K, 4, experts=E)["engine"] == 1
    planes = [si.draw_quantized_weight(25, e, N, K, 4) for e in range(E)]
    st = {k: np.stack([p[k] for p in planes]) for k in ("w", "scales", "biases")}
    x = si.draw_activations(25, 98, R, K)
    rhs = np.array([0] * 4 + [1] * 5 + [2] * 8 + [3] * 9 + [5] * 16, np.uint32)
    np.random.default_rng([25, 1]).shuffle(rhs)
    lhs = (np.arange(len(rhs)) * 7 % R).astype(np.uint32)
    progress("gather, activation load forms on the matrix cores")
    y = agq.gather_qmv(bf16_dev(x), u32_dev(st["w"]), bf16_dev(st["scales"]), bf16_dev(st["biases"]),
                       rhs_indices=u32_dev(rhs), lhs_indices=u32_dev(lhs))
    torch.cuda.synchronize()
    y_ref, A = oracle.gather_qmv(x, st["w"], st["scales"], st["biases"], lhs, rhs, K, 4)
    check_close(y, y_ref, A, "gather activation load forms")


@pytest.mark.parametrize("bits", [4, 8])
def test_constant_code_closed_form_adversarial(bits):
    """|y| equals sum|x*w| here, so the bf16 output rounding alone can approach 4e-3*A."""
    N, K = 64, 4096
    g = np.random.default_rng(bits)
    q = np.full((N, K), 2 ** bits - 1, np.uint8)
    s = si.bf16_bits((0.01 + 0.01 * g.random((N, K // 64))).astype(np.float32))
    b = si.bf16_bits((0.001 * g.random((N, K // 64))).astype(np.float32))
    x = si.bf16_bits(np.abs(g.standard_normal((1, K))).astype(np.float32))
    wq = si.pack_codes(q, bits)
    progress(f"adversarial bits={bits}")
    y = agq.qmv(bf16_dev(x)[0], u32_dev(wq), bf16_dev(s), bf16_dev(b), bits=bits)
    torch.cuda.synchronize()
    y_ref, A = oracle.qmv(x, wq, s, b, K, bits)
    check_close(y[None], y_ref, A, "adversarial", extra_half_ulp=True)


# ---------------------------------------------------------------- invariants


@pytest.mark.parametrize("bits", [4, 8])
def test_one_hot_columns_are_bitwise_weights(bits):
    """x = e_k gives y[n] = bf16(w_hat[n, k]) exactly: one exact product per output."""
    N, K = 515, 1024
    d = si.draw_quantized_weight(8, bits, N, K, bits)
    w, s, b = dev_weight(d)
    ref, _ = oracle.dequantize(d["w"], d["scales"], d["biases"], K, bits)
    want = si.bf16_bits(ref.astype(np.float32))
    cols = list(range(0, 8)) + list(range(56, 72)) + [K - 9, K - 1] + list(np.random.default_rng(1).integers(0, K, 14))
    for c0 in range(0, len(cols), 8):
        cs = cols[c0:c0 + 8]
        x = np.zeros((len(cs), K), np.uint16)
        for i, c in enumerate(cs):
            x[i, c] = 0x3F80
        progress(f"one-hot bits={bits} cols={cs}")
        y = agq.qmv_wide(bf16_dev(x), w, s, b, bits=bits)
        torch.cuda.synchronize()
        got = bf16_bits_host(y)
        for i, c in enumerate(cs):
            assert np.array_equal(got[i], want[:, c]), (bits, c)


def dequantized_bf16_columns(d, K, bits, cols, block=8192):
    """bf16 RNE of the oracle's exact dequantized weights w_hat[:, cols], computed in row
    blocks (the full dequantized lm_head would take 4 GB of float64)."""
    N = d["w"].shape[0]
    want = np.empty((N, len(cols)), np.uint16)
    for r0 in range(0, N, block):
        ref, bad = oracle.dequantize(d["w"][r0:r0 + block], d["scales"][r0:r0 + block],
                                     d["biases"][r0:r0 + block], K, bits)
        assert bad == 0  # each w_hat is a binary32 value, so bf16(fp32(w_hat)) is unique
        want[r0:r0 + block] = si.bf16_bits(ref[:, cols].astype(np.float32))
    return want


def seam_columns(K, bits):
    """Every column of the first 64-column group, both sides of every 64-chunk seam (where
    a lane's next chunk starts, and where a K split hands over to the next wave), and the
    last group's edges and the last column."""
    per_chunk = 128 // bits  # columns per 16-byte chunk
    cols = set(range(64)) | {64, 65, K - 64, K - 33, K - 32, K - 2, K - 1}
    for c in range(64, K // per_chunk, 64):
        cols |= {c * per_chunk - 1, c * per_chunk}
    return sorted(c for c in cols if 0 <= c < K)


def one_hot_sweep(w, s, b, d, K, bits, M, cols, what):
    """x rows e_c for c in cols, M per call: y[m, n] must equal bf16(w_hat[n, c]) bit for bit."""
    want = dequantized_bf16_columns(d, K, bits, cols)
    for c0 in range(0, len(cols), M):
        cs = cols[c0:c0 + M]
        x = np.zeros((len(cs), K), np.uint16)
        for i, c in enumerate(cs):
            x[i, c] = 0x3F80
        xd = bf16_dev(x)
        y = agq.qmv(xd[0], w, s, b, bits=bits)[None] if M == 1 else agq.qmv_wide(xd, w, s, b, bits=bits)
        torch.cuda.synchronize()
        got = bf16_bits_host(y)
        for i, c in enumerate(cs):
            j = c0 + i
            if not np.array_equal(got[i], want[:, j]):
                bad = np.nonzero(got[i] != want[:, j])[0]
                raise AssertionError(f"{what}: column {c}: {bad.size} rows differ, first row {bad[0]}: "
                                     f"gpu {got[i][bad[0]]:#06x} want {want[bad[0], j]:#06x}")
    progress(f"{what}: {len(cols)} one-hot columns bitwise equal")


@pytest.mark.parametrize("bits,M,N,K", [
    (4, 1, 515, 4096), (4, 2, 515, 4096), (4, 3, 515, 4096),      # one wave per row, block copy of x
    (4, 1, 300, 14336), (4, 2, 300, 14336), (4, 3, 300, 14336),   # K split over waves
    (8, 1, 515, 896), (8, 1, 300, 4864),
])
def test_one_hot_columns_bitwise_on_the_vector_path(bits, M, N, K):
    """The VALU product (batch 1 and M <= 3, every 8-bit product): x = e_k gives
    y[n] = bf16(w_hat[n, k]) exactly, over every column of a group and the chunk, lane
    and wave seams."""
    plan = agq.launch_plan(M, N, K, bits)
    assert plan["engine"] == 0
    d = si.draw_quantized_weight(26, 10 * bits + M, N, K, bits)
    one_hot_sweep(*dev_weight(d), d, K, bits, M, seam_columns(K, bits),
                  f"one-hot VALU bits={bits} M={M} {N}x{K} S={plan['waves_per_group']} cpt={plan['cpt']}")


def test_one_hot_columns_bitwise_on_lm_head(wl):
    """The launch that runs lm_head (128256x4096, 4-bit) in the benchmark, the bit-stream
    kernel (engine 2), one-hot bitwise on the real weights: every column of the first group
    (each position of the 4-bit pair plan) and the chunk and row ends."""
    m = wl(1)["lm_head"]
    plan = agq.launch_plan(1, m["N"], m["K"], 4)
    assert plan["engine"] == 2
    cols = list(range(64)) + [2047, 2048, 4031, 4032, 4095]
    one_hot_sweep(*dev_weight(m), m, m["K"], 4, 1, cols, "one-hot lm_head (bit-stream kernel)")


@pytest.mark.parametrize("bits", [4, 8])
def test_zero_x_gives_positive_zero(bits):
    d = si.draw_quantized_weight(9, bits, 300, 2048, bits)
    w, s, b = dev_weight(d)
    progress(f"zero x bits={bits}")
    y = agq.qmv(torch.zeros(2048, dtype=torch.bfloat16, device="cuda"), w, s, b, bits=bits)
    torch.cuda.synchronize()
    assert np.all(bf16_bits_host(y) == 0)


@pytest.mark.parametrize("bits,M", [(4, 1), (8, 1), (4, 4), (4, 8)])
def test_deterministic_and_power_of_two_scaling(bits, M):
    N, K = 2000, 4096
    d = si.draw_quantized_weight(10, bits, N, K, bits)
    w, s, b = dev_weight(d)
    x = si.draw_activations(10, 100 + M, M, K)
    xd = bf16_dev(x)
    progress(f"determinism bits={bits} M={M}")
    f = (lambda t: agq.qmv(t[0], w, s, b, bits=bits)[None]) if M == 1 else (lambda t: agq.qmv_wide(t, w, s, b, bits=bits))
    y1 = bf16_bits_host(f(xd))
    y2 = bf16_bits_host(f(xd))
    assert np.array_equal(y1, y2)
    y4 = bf16_bits_host(f(xd * 4))        # exact: multiplying bf16 by 4 only shifts the exponent
    assert np.array_equal(bf16_host(f(xd * 4)), 4 * bf16_host(f(xd)))
    assert y4.shape == y1.shape


@pytest.mark.parametrize("M", [1, 8])   # VALU and matrix cores
def test_row_permutation_equivariance(M):
    N, K = 1000, 4096
    d = si.draw_quantized_weight(11, 4, N, K, 4)
    x = bf16_dev(si.draw_activations(11, M, M, K))
    perm = np.random.default_rng(2).permutation(N)
    w, s, b = dev_weight(d)
    wp, sp, bp = dev_weight({k: v[perm] for k, v in d.items()})
    progress(f"row permutation M={M}")
    f = (lambda *a: agq.qmv(x[0], *a)[None]) if M == 1 else (lambda *a: agq.qmv_wide(x, *a))
    y = bf16_bits_host(f(w, s, b))
    yp = bf16_bits_host(f(wp, sp, bp))
    assert np.array_equal(yp, y[:, perm])


@pytest.mark.parametrize("M", [3, 6])   # VALU and matrix cores
def test_output_guard_region_untouched(M):
    N, K = 1003, 4096
    d = si.draw_quantized_weight(12, 4, N, K, 4)
    w, s, b = dev_weight(d)
    x = bf16_dev(si.draw_activations(12, 1, M, K))
    buf = torch.full((M * N + 4096,), float("nan"), dtype=torch.bfloat16, device="cuda")
    sentinel = bf16_bits_host(buf[M * N:]).copy()
    progress(f"guard region M={M}")
    agq.qmv_wide(x, w, s, b, out=buf[:M * N].view(M, N))
    torch.cuda.synchronize()
    assert np.array_equal(bf16_bits_host(buf[M * N:]), sentinel)
    assert not np.any(np.isnan(bf16_host(buf[:M * N])))


def test_gather_matches_per_pair_qmv_and_identity_forms():
    E, N, K, R = 4, 700, 4096, 5
    planes = [si.draw_quantized_weight(13, e, N, K, 4) for e in range(E)]
    st = {k: np.stack([p[k] for p in planes]) for k in ("w", "scales", "biases")}
    x = si.draw_activations(13, 99, R, K)
    lhs = np.array([0, 1, 1, 4, 2, 3, 0, 4, 2], np.uint32)
    rhs = np.array([3, 0, 2, 2, 2, 1, 0, 3, 2], np.uint32)
    w, s, b = u32_dev(st["w"]), bf16_dev(st["scales"]), bf16_dev(st["biases"])
    xd = bf16_dev(x)
    progress("gather vs per-pair qmv")
    y = agq.gather_qmv(xd, w, s, b, rhs_indices=u32_dev(rhs), lhs_indices=u32_dev(lhs))
    torch.cuda.synchronize()
    y_ref, A = oracle.gather_qmv(x, st["w"], st["scales"], st["biases"], lhs, rhs, K, 4)
    check_close(y, y_ref, A, "gather small")
    for p in range(len(lhs)):
        yp = agq.qmv(xd[lhs[p]], w[rhs[p]], s[rhs[p]], b[rhs[p]])
        check_close(yp[None], y_ref[p:p + 1], A[p:p + 1], f"qmv pair {p}")
    # NULL indices are the identity
    y_id = agq.gather_qmv(xd[:4], w, s, b, rhs_indices=None, lhs_indices=None)
    y_ex = agq.gather_qmv(xd[:4], w, s, b, rhs_indices=u32_dev(np.arange(4, dtype=np.uint32)),
                          lhs_indices=u32_dev(np.arange(4, dtype=np.uint32)))
    torch.cuda.synchronize()
    assert np.array_equal(bf16_bits_host(y_id), bf16_bits_host(y_ex))


def test_gather_many_pairs_one_expert_and_unused_experts():
    """17 pairs on one expert (three passes of up to 8), other experts unused."""
    E, N, K = 6, 300, 14336
    planes = [si.draw_quantized_weight(14, e, N, K, 4) for e in range(E)]
    st = {k: np.stack([p[k] for p in planes]) for k in ("w", "scales", "biases")}
    x = si.draw_activations(14, 99, 20, K)
    lhs = np.arange(19, dtype=np.uint32) % 20
    rhs = np.array([4] * 17 + [1, 4], np.uint32)
    progress("gather 17 pairs on one expert")
    y = agq.gather_qmv(bf16_dev(x), u32_dev(st["w"]), bf16_dev(st["scales"]), bf16_dev(st["biases"]),
                       rhs_indices=u32_dev(rhs), lhs_indices=u32_dev(lhs))
    torch.cuda.synchronize()
    y_ref, A = oracle.gather_qmv(x, st["w"], st["scales"], st["biases"], lhs, rhs, K, 4)
    check_close(y, y_ref, A, "gather one expert")


def test_gather_passes_through_the_block_copy_of_x():
    """VALU gather (8-bit codes): several passes per plane (21 pairs on one expert: 8, 8
    and 5) through the block's LDS copy of x with two K segments, with repeated and
    scattered x rows."""
    E, N, K, R, bits = 3, 1030, 2048, 24, 8
    plan = agq.launch_plan(8, N, K, bits, experts=E)
    assert plan["engine"] == 0 and plan["x_lds_bytes"] > 0 and plan["waves_per_group"] == 2
    planes = [si.draw_quantized_weight(21, e, N, K, bits) for e in range(E)]
    st = {k: np.stack([p[k] for p in planes]) for k in ("w", "scales", "biases")}
    x = si.draw_activations(21, 99, R, K)
    rng = np.random.default_rng([21, 1])
    rhs = np.array([1] * 21 + [0] * 5 + [2] * 4, np.uint32)
    rng.shuffle(rhs)
    lhs = rng.integers(0, R, len(rhs)).astype(np.uint32)
    progress("gather, several passes through the LDS copy of x")
    y = agq.gather_qmv(bf16_dev(x), u32_dev(st["w"]), bf16_dev(st["scales"]), bf16_dev(st["biases"]),
                       rhs_indices=u32_dev(rhs), lhs_indices=u32_dev(lhs), bits=bits)
    torch.cuda.synchronize()
    y_ref, A = oracle.gather_qmv(x, st["w"], st["scales"], st["biases"], lhs, rhs, K, bits)
    check_close(y, y_ref, A, "gather passes")


@pytest.mark.parametrize("N", [1, 5, 9])
def test_gather_tiny_planes_with_wide_passes(N):
    """Planes of a few rows (one ragged 16-row tile on the matrix cores) with six pairs
    on one plane and one on the other."""
    E, K, R = 2, 1024, 8
    planes = [si.draw_quantized_weight(22, 10 * N + e, N, K, 4) for e in range(E)]
    st = {k: np.stack([p[k] for p in planes]) for k in ("w", "scales", "biases")}
    x = si.draw_activations(22, N, R, K)
    rhs = np.array([1, 1, 0, 1, 1, 1, 1], np.uint32)
    lhs = np.array([0, 3, 7, 1, 5, 2, 6], np.uint32)
    progress(f"gather tiny plane N={N}")
    y = agq.gather_qmv(bf16_dev(x), u32_dev(st["w"]), bf16_dev(st["scales"]), bf16_dev(st["biases"]),
                       rhs_indices=u32_dev(rhs), lhs_indices=u32_dev(lhs))
    torch.cuda.synchronize()
    y_ref, A = oracle.gather_qmv(x, st["w"], st["scales"], st["biases"], lhs, rhs, K, 4)
    check_close(y, y_ref, A, f"gather N={N}")


@pytest.mark.parametrize("bits", [8, 4])   # VALU and matrix-core gathers
def test_gather_out_of_range_indices_give_nan_rows(bits):
    E, N, K, R = 3, 130, 1024, 4
    planes = [si.draw_quantized_weight(15, e, N, K, bits) for e in range(E)]
    st = {k: np.stack([p[k] for p in planes]) for k in ("w", "scales", "biases")}
    x = si.draw_activations(15, 99, R, K)
    lhs = np.array([0, 9, 2, 3], np.uint32)     # 9 >= R
    rhs = np.array([1, 0, 7, 2], np.uint32)     # 7 >= E
    progress("gather invalid indices")
    y = agq.gather_qmv(bf16_dev(x), u32_dev(st["w"]), bf16_dev(st["scales"]), bf16_dev(st["biases"]),
                       rhs_indices=u32_dev(rhs), lhs_indices=u32_dev(lhs), bits=bits)
    torch.cuda.synchronize()
    yh = bf16_host(y)
    assert np.all(np.isnan(yh[1])) and np.all(np.isnan(yh[2]))
    ok = np.array([0, 3])
    y_ref, A = oracle.gather_qmv(x, st["w"], st["scales"], st["biases"], lhs[ok], rhs[ok], K, bits)
    check_close(y[torch.as_tensor(ok, device=y.device)], y_ref, A, "valid pairs")


def test_wide_rows_equal_single_row_results():
    """Row m of qmv_wide and qmv on x[m] both meet the tolerance against the same oracle."""
    N, K = 4096, 14336
    d = si.draw_quantized_weight(16, 4, N, K, 4)
    w, s, b = dev_weight(d)
    x = si.draw_activations(16, 1, 3, K)
    progress("wide vs single rows")
    yw = agq.qmv_wide(bf16_dev(x), w, s, b)
    y_ref, A = oracle.qmv(x, d["w"], d["scales"], d["biases"], K, 4, rows=np.arange(0, N, 7))
    cols = torch.arange(0, N, 7, device="cuda")
    check_close(yw[:, cols], y_ref, A, "wide")
    for m in range(3):
        y1 = agq.qmv(bf16_dev(x[m]), w, s, b)
        check_close(y1[cols][None], y_ref[m:m + 1], A[m:m + 1], f"single {m}")


def test_launch_plans_size_each_block_size_separately():
    """One kernel (8 activation rows, one chunk per lane, x staged per wave) runs with
    256-thread blocks at K=2048 (four single-wave row groups, two blocks per compute
    unit) and 448-thread blocks at K=14336 (one row group of 7 waves, one block). The
    residency the grid is sized from must be that of the block size in use, whatever was
    planned before: bigger blocks of the same kernel can never hold more waves."""
    shapes = {256: (8, 65536, 1024), 448: (8, 4096, 7168)}  # 8-bit: the VALU form
    for order in ((256, 448), (448, 256), (256, 448)):
        plans = {t: agq.launch_plan(*shapes[t], 8) for t in order}
        small, big = plans[256], plans[448]
        for p, threads in ((small, 256), (big, 448)):
            assert p["threads_per_block"] == threads and p["cpt"] == 1 and p["mw"] == 8
            assert p["x_lds_bytes"] == 0
            assert p["resident_waves"] % (threads // 64) == 0
            assert p["blocks"] * threads // 64 <= p["resident_waves"]  # one round of resident blocks
        assert big["resident_waves"] <= small["resident_waves"]


def test_graph_replays_match_eager():
    """The three products captured in one HIP graph: every replay, with eager work and
    synchronizations in between, reproduces the eager outputs bit for bit."""
    N, K, E, P = 1500, 4096, 3, 5
    d = si.draw_quantized_weight(17, 1, N, K, 4)
    planes = [si.draw_quantized_weight(17, 2 + e, N, K, 4) for e in range(E)]
    st = {k: np.stack([p[k] for p in planes]) for k in ("w", "scales", "biases")}
    x = si.draw_activations(17, 9, 8, K)
    w, s, b = dev_weight(d)
    ws, ss, bs = u32_dev(st["w"]), bf16_dev(st["scales"]), bf16_dev(st["biases"])
    xd = bf16_dev(x)
    x4 = xd[:4].contiguous()
    rhs = u32_dev(np.array([2, 0, 2, 1, 0], np.uint32))
    lhs = u32_dev(np.array([0, 3, 1, 1, 2], np.uint32))
    y1 = torch.empty(N, dtype=torch.bfloat16, device="cuda")
    y4 = torch.empty((4, N), dtype=torch.bfloat16, device="cuda")
    y8 = torch.empty((8, N), dtype=torch.bfloat16, device="cuda")
    yg = torch.empty((P, N), dtype=torch.bfloat16, device="cuda")
    outs = (y1, y4, y8, yg)

    def run():
        agq.qmv(xd[0], w, s, b, out=y1)
        agq.qmv_wide(x4, w, s, b, out=y4)     # VALU
        agq.qmv_wide(xd, w, s, b, out=y8)     # matrix cores
        agq.gather_qmv(xd, ws, ss, bs, rhs_indices=rhs, lhs_indices=lhs, out=yg)

    progress("graph capture of qmv, qmv_wide (M = 4 and 8), gather_qmv")
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        run()  # eager, also primes the launch-plan caches outside capture
    torch.cuda.synchronize()
    eager = [bf16_bits_host(t).copy() for t in outs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        run()
    torch.cuda.synchronize()
    for rep in range(4):
        for t in outs:
            t.zero_()
        agq.qmv(xd[1], w, s, b)  # unrelated eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for got, want in zip(outs, eager):
            assert np.array_equal(bf16_bits_host(got), want), f"replay {rep}"
    y_ref, A = oracle.qmv(x[:1], d["w"], d["scales"], d["biases"], K, 4, rows=np.arange(0, N, 11))
    check_close(y1[None][:, torch.arange(0, N, 11, device="cuda")], y_ref, A, "graph qmv")


@pytest.mark.parametrize("K", [128, 512])   # VALU and matrix-core gathers
def test_gather_at_the_pair_limit(K):
    """4096 pairs (the most one call takes) over 3 planes, with repeated x rows."""
    E, N, R, P = 3, 96, 64, 4096
    planes = [si.draw_quantized_weight(18, e, N, K, 4) for e in range(E)]
    st = {k: np.stack([p[k] for p in planes]) for k in ("w", "scales", "biases")}
    x = si.draw_activations(18, 99, R, K)
    rng = np.random.default_rng([18, 1])
    lhs = rng.integers(0, R, P).astype(np.uint32)
    rhs = rng.integers(0, E, P).astype(np.uint32)
    progress("gather with 4096 pairs")
    y = agq.gather_qmv(bf16_dev(x), u32_dev(st["w"]), bf16_dev(st["scales"]), bf16_dev(st["biases"]),
                       rhs_indices=u32_dev(rhs), lhs_indices=u32_dev(lhs))
    torch.cuda.synchronize()
    y_ref, A = oracle.gather_qmv(x, st["w"], st["scales"], st["biases"], lhs, rhs, K, 4)
    check_close(y, y_ref, A, "gather 4096 pairs")


def test_calls_on_a_side_stream():
    """Work is queued on the stream handed in (or current at preparation), not the null stream."""
    N, K = 777, 2048
    d = si.draw_quantized_weight(19, 1, N, K, 8)
    w, s, b = dev_weight(d)
    x = si.draw_activations(19, 2, 2, K)
    xd = bf16_dev(x)
    y = torch.empty((2, N), dtype=torch.bfloat16, device="cuda")
    side = torch.cuda.Stream()
    call = agq.prepare_qmv(xd, w, s, b, y, bits=8, stream=side)
    progress("prepared qmv_wide on a side stream")
    torch.cuda.synchronize()
    with torch.cuda.stream(side):
        y.fill_(float("nan"))
        call()
    side.synchronize()
    y_ref, A = oracle.qmv(x, d["w"], d["scales"], d["biases"], K, 8)
    check_close(y, y_ref, A, "side stream")


@pytest.mark.parametrize("bits,M,K", [(4, 2, 65536), (8, 2, 32768), (4, 8, 16384), (4, 6, 65536)])
def test_k_limits_of_the_wide_form(bits, M, K):
    """The largest K per M on the VALU (eight waves split each row); the matrix cores
    (four waves) have no such limit."""
    p = agq.plan(M, 5, K, bits, 64, 256, 0)
    assert p["waves_per_group"] == (4 if p["engine"] == 1 else 8) or M == 8
    d = si.draw_quantized_weight(20, 100 * bits + M, 5, K, bits)
    x = si.draw_activations(20, M, M, K)
    run_qmv_case(f"K limit M={M} bits={bits}", x, d, K, bits, M=M)
