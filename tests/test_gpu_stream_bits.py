"""GPU parity of the bit-stream widths: 2-, 3-, 5- and 6-bit affine codes (group size 64),
whose codes fill each row's low-first bit stream (a 3-, 5- or 6-bit code can run into the
next word). The products (agq_qmv, agq_qmv_wide, and agq_qmm in passes of 8 rows) meet the
usual tolerance against the oracle on every row, |y_gpu - y_ref| <= 2e-3 * sum_k |x_k w_k|
(plus half a bf16 ulp where K <= 128); one-hot columns give bf16(w_hat) bit for bit (each
weight fma(s, q, b) is exact in fp32 for the quantizer's recipe); dequantization is bitwise.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import seeded_inputs as si
from gpu_util import bf16_bits_host, bf16_dev, check_close, progress, u32_dev

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("no GPU", allow_module_level=True)

import affine_group_quantized_amd as agq  # noqa: E402

BITS = [2, 3, 5, 6]


def dev_weight(d):
    return u32_dev(d["w"]), bf16_dev(d["scales"]), bf16_dev(d["biases"])


@pytest.mark.parametrize("bits", BITS)
@pytest.mark.parametrize("M,N,K", [
    (1, 4096, 4096), (1, 1000, 14336), (3, 777, 4160), (8, 300, 2048), (5, 17, 64), (2, 33, 128),
    (4, 2048, 8192), (7, 130, 4096 + 64 * 3), (2, 1000, 4160), (2, 4096, 14336),
    (1, 999, 12288), (2, 300, 8192 + 64),   # the K split: an odd chunk count, a chunk of one group
])
def test_stream_bits_products(bits, M, N, K):
    """Several 64-group chunks of K, partial last chunks, weight rows past the last full
    block, and every activation-row count form (1, 2, 4, 8 and between)."""
    d = si.draw_quantized_weight(50, 10 * bits + M, N, K, bits)
    x = si.draw_activations(50, 100 + M, M, K)
    w, s, b = dev_weight(d)
    progress(f"stream bits={bits} M={M} N={N} K={K}")
    xd = bf16_dev(x)
    y = agq.qmv(xd[0], w, s, b, bits=bits)[None] if M == 1 else agq.qmv_wide(xd, w, s, b, bits=bits)
    torch.cuda.synchronize()
    y_ref, A = oracle.qmv(x, d["w"], d["scales"], d["biases"], K, bits)
    worst = check_close(y, y_ref, A, f"bits={bits} M={M} N={N} K={K}", extra_half_ulp=K <= 128)
    progress(f"stream bits: ok, worst |err|/A = {worst:.3e}")


@pytest.mark.parametrize("bits", BITS)
@pytest.mark.parametrize("route", ["passes", "widened"])
def test_stream_bits_one_hot_columns_are_bitwise_weights(bits, route):
    """x = e_k for every column of 5 groups (all 64 positions of a code in its group, so
    every straddling position): y[n] = bf16(w_hat[n, k]) bit for bit, through qmm's passes
    of 8 rows (no workspace) and through the codes widened to 8 bits and the 8-bit GEMM."""
    N, K = 300, 320
    d = si.draw_quantized_weight(51, bits, N, K, bits)
    w, s, b = dev_weight(d)
    ref, bad = oracle.dequantize(d["w"], d["scales"], d["biases"], K, bits)
    assert bad == 0
    want = si.bf16_bits(ref.astype(np.float32))
    x = np.zeros((K, K), np.uint16)
    x[np.arange(K), np.arange(K)] = 0x3F80
    progress(f"stream bits one-hot bits={bits} route={route}")
    got = bf16_bits_host(agq.qmm(bf16_dev(x), w, s, b, bits=bits, workspace=False if route == "passes" else None))
    assert np.array_equal(got, want.T)


@pytest.mark.parametrize("bits", BITS)
def test_stream_bits_one_hot_columns_matvec(bits):
    """The one- and two-row matvec forms: x = e_k (and 2 e_k as a second activation row) for
    every column of five groups, so every position of a code in its group, including the
    codes decoded as pairs k, k + d from one stream window and the adjacent pairs at the end
    of a 3- or 5-bit group: y = bf16(w_hat[:, k]) and bf16(2 w_hat[:, k]) bit for bit."""
    N, K = 300, 320
    d = si.draw_quantized_weight(53, bits, N, K, bits)
    w, s, b = dev_weight(d)
    ref, bad = oracle.dequantize(d["w"], d["scales"], d["biases"], K, bits)
    assert bad == 0
    want1 = si.bf16_bits(ref.astype(np.float32))
    want2 = si.bf16_bits((2 * ref).astype(np.float32))
    eye = np.zeros((K, K), np.uint16)
    eye[np.arange(K), np.arange(K)] = 0x3F80
    pair = np.zeros((K, 2, K), np.uint16)
    pair[np.arange(K), 0, np.arange(K)] = 0x3F80
    pair[np.arange(K), 1, np.arange(K)] = 0x4000
    xe, xp = bf16_dev(eye), bf16_dev(pair.reshape(2 * K, K))
    progress(f"stream bits one-hot matvec bits={bits}")
    y1 = torch.stack([agq.qmv(xe[k], w, s, b, bits=bits) for k in range(K)])
    y2 = torch.stack([agq.qmv_wide(xp[2 * k:2 * k + 2], w, s, b, bits=bits) for k in range(K)])
    torch.cuda.synchronize()
    g1, g2 = bf16_bits_host(y1), bf16_bits_host(y2)
    assert np.array_equal(g1, want1.T)
    assert np.array_equal(g2[:, 0], want1.T)
    assert np.array_equal(g2[:, 1], want2.T)


@pytest.mark.parametrize("bits", BITS)
@pytest.mark.parametrize("gs", [32, 64, 128])
def test_stream_bits_dequantize_bit_exact(bits, gs):
    N, K = 97, 1024
    g = np.random.default_rng([52, bits, gs])
    q = g.integers(0, 2 ** bits, size=(N, K), dtype=np.uint8)
    sc = si.bf16_bits((0.01 + 0.02 * g.random((N, K // gs))).astype(np.float32))
    bi = si.bf16_bits((-0.05 + 0.03 * g.standard_normal((N, K // gs))).astype(np.float32))
    wq = si.pack_codes(q, bits)
    progress(f"stream bits dequantize bits={bits} gs={gs}")
    out = agq.dequantize(u32_dev(wq), bf16_dev(sc), bf16_dev(bi), bits=bits, group_size=gs)
    torch.cuda.synchronize()
    ref, bad = oracle.dequantize(wq, sc, bi, K, bits, gs)
    assert bad == 0
    assert np.array_equal(out.cpu().numpy().astype(np.float64), ref)


@pytest.mark.parametrize("bits", BITS)
def test_stream_bits_qmm_passes_and_device_quantizer(bits):
    """Weights quantized on the device (the oracle's codes bit for bit) feed a 20-row qmm
    (passes of 8, 8 and 4 rows) that meets the oracle bound on every row."""
    N, K, M = 500, 1024, 20
    wf = (0.02 * np.random.default_rng([53, bits]).standard_normal((N, K))).astype(np.float32)
    x = si.draw_activations(53, bits, M, K)
    progress(f"stream bits quantize -> qmm bits={bits}")
    codes, sc, bi = agq.quantize(torch.as_tensor(wf, device="cuda"), bits=bits)
    y = agq.qmm(bf16_dev(x), codes, sc, bi, bits=bits)
    torch.cuda.synchronize()
    wq, s_ref, b_ref = oracle.quantize(wf, bits)
    assert np.array_equal(codes.cpu().numpy().view(np.uint32), wq)
    y_ref, A = oracle.qmv(x, wq, s_ref, b_ref, K, bits)
    check_close(y, y_ref, A, f"quantize -> qmm bits={bits}")


def test_stream_bits_refused_where_not_supported():
    """The fused projection takes 4- or 8-bit codes; other group sizes (32, 128) are
    refused for the bit-stream products; every refusal precedes any launch."""
    N, K = 64, 256
    d = si.draw_quantized_weight(54, 0, N, K, 3)
    w, s, b = dev_weight(d)
    x = bf16_dev(si.draw_activations(54, 1, 2, K))
    for call in (lambda: agq.qmv_fused(x[0], w, s, b, bits=3),):
        with pytest.raises(agq.AgqError) as e:
            call()
        assert e.value.status == agq.AGQ_ENOTSUP
    d32 = si.pack_codes(np.zeros((N, K), np.uint8), 3)
    with pytest.raises(agq.AgqError) as e:
        agq.qmv(x[0], u32_dev(d32), bf16_dev(np.zeros((N, K // 32), np.uint16)),
                bf16_dev(np.zeros((N, K // 32), np.uint16)), bits=3, group_size=32)
    assert e.value.status == agq.AGQ_ENOTSUP


def stacked_planes(cfg, E, N, K, bits):
    planes = [si.draw_quantized_weight(cfg, 10 * bits + e, N, K, bits) for e in range(E)]
    return {k: np.stack([p[k] for p in planes]) for k in ("w", "scales", "biases")}


def dev_planes(st):
    return u32_dev(st["w"]), bf16_dev(st["scales"]), bf16_dev(st["biases"])


@pytest.mark.parametrize("bits", BITS)
def test_stream_bits_gather(bits):
    """Expert gather at the bit-stream widths: pairs with repeated and unused experts,
    planes of a ragged number of rows, two chunks of K (the second partial), and the NULL
    index forms (identity lhs with R == P, identity rhs with E == P)."""
    E, N, K, R = 6, 300, 4160, 5
    st = stacked_planes(55, E, N, K, bits)
    w, s, b = dev_planes(st)
    x = si.draw_activations(55, bits, R, K)
    rng = np.random.default_rng([55, bits])
    rhs = np.array([3, 0, 3, 5, 3, 1, 0, 5, 3], np.uint32)
    lhs = rng.integers(0, R, len(rhs)).astype(np.uint32)
    progress(f"stream gather bits={bits} P={len(rhs)}")
    y = agq.gather_qmv(bf16_dev(x), w, s, b, rhs_indices=u32_dev(rhs), lhs_indices=u32_dev(lhs), bits=bits)
    torch.cuda.synchronize()
    y_ref, A = oracle.gather_qmv(x, st["w"], st["scales"], st["biases"], lhs, rhs, K, bits)
    check_close(y, y_ref, A, f"stream gather bits={bits}")
    # Identity lhs (R == P) and identity rhs (E == P).
    xp = si.draw_activations(55, 20 + bits, E, K)
    progress(f"stream gather bits={bits} NULL indices")
    y1 = agq.gather_qmv(bf16_dev(xp[:len(rhs[:E])]), w, s, b, rhs_indices=u32_dev(rhs[:E]), bits=bits)
    y2 = agq.gather_qmv(bf16_dev(x), w, s, b, lhs_indices=u32_dev(lhs[:E]), bits=bits)
    torch.cuda.synchronize()
    r1, A1 = oracle.gather_qmv(xp, st["w"], st["scales"], st["biases"], None, rhs[:E], K, bits)
    r2, A2 = oracle.gather_qmv(x, st["w"], st["scales"], st["biases"], lhs[:E], None, K, bits)
    check_close(y1, r1, A1, "identity lhs")
    check_close(y2, r2, A2, "identity rhs")


@pytest.mark.parametrize("bits", BITS)
def test_stream_bits_gather_out_of_range_indices_give_nan_rows(bits):
    E, N, K, R = 3, 130, 1024, 4
    st = stacked_planes(56, E, N, K, bits)
    w, s, b = dev_planes(st)
    x = si.draw_activations(56, 99, R, K)
    lhs = np.array([0, 9, 2, 3], np.uint32)     # 9 >= R
    rhs = np.array([1, 0, 7, 2], np.uint32)     # 7 >= E
    progress(f"stream gather invalid indices bits={bits}")
    y = agq.gather_qmv(bf16_dev(x), w, s, b, rhs_indices=u32_dev(rhs), lhs_indices=u32_dev(lhs), bits=bits)
    torch.cuda.synchronize()
    yh = bf16_bits_host(y)
    assert np.all(yh[1] == 0x7FC0) and np.all(yh[2] == 0x7FC0)
    ok = np.array([0, 3])
    y_ref, A = oracle.gather_qmv(x, st["w"], st["scales"], st["biases"], lhs[ok], rhs[ok], K, bits)
    check_close(y[torch.as_tensor(ok, device=y.device)], y_ref, A, "valid pairs")


@pytest.mark.parametrize("bits", [3, 6])
def test_stream_bits_gather_qmm(bits):
    """gather_qmm at the bit-stream widths: many pairs per expert (a prefill gather)."""
    E, N, K, R = 4, 200, 2048, 48
    st = stacked_planes(57, E, N, K, bits)
    w, s, b = dev_planes(st)
    x = si.draw_activations(57, bits, R, K)
    rng = np.random.default_rng([57, bits])
    rhs = rng.integers(0, E - 1, 96).astype(np.uint32)   # plane E - 1 unused
    lhs = rng.integers(0, R, 96).astype(np.uint32)
    progress(f"stream gather_qmm bits={bits} P={len(rhs)}")
    y = agq.gather_qmm(bf16_dev(x), w, s, b, rhs_indices=u32_dev(rhs), lhs_indices=u32_dev(lhs), bits=bits)
    torch.cuda.synchronize()
    y_ref, A = oracle.gather_qmv(x, st["w"], st["scales"], st["biases"], lhs, rhs, K, bits)
    check_close(y, y_ref, A, f"stream gather_qmm bits={bits}")


@pytest.mark.parametrize("bits", BITS)
@pytest.mark.parametrize("M", [64, 300])
def test_stream_bits_qmm_widened_to_8_bits(bits, M):
    """From 64 rows with a workspace, qmm widens the codes to the 8-bit layout and runs
    the 8-bit GEMM: every row meets the oracle bound, the workspace query covers the
    widened codes (N*K bytes), and a smaller workspace is refused before any launch."""
    N, K = 200, 1024
    d = si.draw_quantized_weight(58, bits, N, K, bits)
    w, s, b = dev_weight(d)
    x = si.draw_activations(58, M, M, K)
    need = agq.lib.agq_qmm_workspace(M, N, K, bits, 64)
    assert need >= N * K
    assert agq.lib.agq_qmm_workspace(63, N, K, bits, 64) == 0   # passes below 64 rows
    progress(f"stream qmm widened bits={bits} M={M}")
    y = agq.qmm(bf16_dev(x), w, s, b, bits=bits)
    torch.cuda.synchronize()
    y_ref, A = oracle.qmv(x, d["w"], d["scales"], d["biases"], K, bits)
    check_close(y, y_ref, A, f"widened qmm bits={bits} M={M}")
    small = torch.empty(N * K - 256, dtype=torch.uint8, device="cuda")
    with pytest.raises(agq.AgqError) as e:
        agq.qmm(bf16_dev(x), w, s, b, bits=bits, workspace=small)
    assert e.value.status == agq.AGQ_EINVAL


def test_stream_bits_gather_at_the_pair_limit():
    """4096 pairs (the pair list's capacity) over two small planes: passes of 8 pairs, about
    256 per plane, every pair's row against the oracle."""
    E, N, K, R, bits = 2, 24, 128, 64, 3
    st = stacked_planes(59, E, N, K, bits)
    w, s, b = dev_planes(st)
    x = si.draw_activations(59, 0, R, K)
    rng = np.random.default_rng(59)
    rhs = rng.integers(0, E, 4096).astype(np.uint32)
    lhs = rng.integers(0, R, 4096).astype(np.uint32)
    progress("stream gather at the pair limit")
    y = agq.gather_qmv(bf16_dev(x), w, s, b, rhs_indices=u32_dev(rhs), lhs_indices=u32_dev(lhs), bits=bits)
    torch.cuda.synchronize()
    y_ref, A = oracle.gather_qmv(x, st["w"], st["scales"], st["biases"], lhs, rhs, K, bits)
    check_close(y, y_ref, A, "stream gather, 4096 pairs", extra_half_ulp=True)
