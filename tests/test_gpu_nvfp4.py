"""GPU parity of the NVFP4 product (agq_qmv_nvfp4) against the oracle's agqo_qmv_nvfp4.

Tolerance as for the affine products: |y_gpu - y_ref| <= 2e-3 * sum_k |x_k * w_k| per element
(plus half a bf16 ulp of y for short rows, where |y| can approach that sum). Every element
value e2m1 * e4m3 is exact in fp32 and the products with bf16 x are exact, so the kernel's
error is its fp32 summation and the one rounding to bf16. One-hot columns with a tensor scale
of 1 give bf16(e2m1(q) * e4m3(s)) bit for bit.
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

import affine_group_quantized_amd as agq  # noqa: E402


def u8_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).to("cuda")


def run(d, x, what, ts=None):
    K = x.shape[-1]
    ts = d["tensor_scale"] if ts is None else ts
    progress(f"nvfp4 {what} M={x.shape[0]} N={d['w'].shape[0]} K={K}")
    xd = bf16_dev(x)
    y = agq.qmv_nvfp4(xd if x.shape[0] > 1 else xd[0], u32_dev(d["w"]), u8_dev(d["scales"]), ts)
    torch.cuda.synchronize()
    y_ref, a = oracle.qmv_nvfp4(x, d["w"], d["scales"], ts, K)
    return check_close(y.reshape(y_ref.shape), y_ref, a, what, extra_half_ulp=K <= 128)


@pytest.mark.parametrize("M,N,K", [
    (1, 4096, 4096), (1, 14336, 4096), (1, 4096, 14336), (1, 6144, 4096),
    (2, 14336, 4096), (3, 4096, 14336), (4, 4096, 4096), (4, 1000, 8192),
    (1, 128256 // 4, 4096),
])
def test_nvfp4_decode_shapes(M, N, K):
    """Llama-shaped NVFP4 weights (every row checked)."""
    d = si.nvfp4_weight(7, N + K, N, K)
    x = si.draw_activations(7, 100 + M, M, K)
    worst = run(d, x, "decode shape")
    progress(f"nvfp4: ok, worst |err|/A = {worst:.3e}")


@pytest.mark.parametrize("M,N,K", [
    (1, 1, 32), (1, 5, 64), (2, 7, 96), (1, 33, 2048 + 32), (3, 130, 32 * 65), (1, 999, 114688),
    (4, 64, 32768), (2, 17, 65536), (1, 300, 14336 + 32 * 3),
])
def test_nvfp4_ragged_and_limits(M, N, K):
    """Random codes and scale bytes (both signs, subnormal scales), ragged rows and chunk
    counts, and the largest K per M."""
    g = np.random.default_rng([8, M, N, K])
    codes = g.integers(0, 16, size=(N, K), dtype=np.uint8)
    scales = g.integers(0, 0x7F, size=(N, K // 16), dtype=np.uint8)  # never 0x7F / 0xFF (NaN)
    scales |= (g.random((N, K // 16)) < 0.3).astype(np.uint8) << 7
    d = {"w": si.pack_codes(codes, 4), "scales": scales, "tensor_scale": 0.75}
    x = si.draw_activations(8, M + N, M, K)
    run(d, x, "ragged")


def test_nvfp4_large_grid_batch1():
    """Batch-1 products whose 16-row grid gives every compute unit two blocks run on the
    bit-stream kernel's NVFP4 form: random codes and scale bytes (both signs, subnormal
    scales) over a ragged row count and two 4096-column chunks, every row against the
    oracle, and one-hot columns bit for bit (code 8, -0, gives +0)."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    N, K = 2 * cus * 16 + 5, 4096 + 64 * 5
    g = np.random.default_rng([10, N, K])
    codes = g.integers(0, 16, size=(N, K), dtype=np.uint8)
    scales = g.integers(0, 0x7F, size=(N, K // 16), dtype=np.uint8)
    scales |= (g.random((N, K // 16)) < 0.3).astype(np.uint8) << 7
    d = {"w": si.pack_codes(codes, 4), "scales": scales, "tensor_scale": 0.75}
    x = si.draw_activations(10, 1, 1, K)
    run(d, x, "large grid")
    w, s = u32_dev(d["w"]), u8_dev(scales)
    e2m1 = np.array([oracle.load().agqo_e2m1(c) for c in range(16)])
    e4m3 = np.array([oracle.load().agqo_e4m3(b) for b in range(256)])
    for c in (0, 1, 15, 16, 17, 63, 4095, 4096, K - 1):
        e = np.zeros((1, K), np.uint16)
        e[0, c] = 0x3F80
        got = bf16_bits_host(agq.qmv_nvfp4(bf16_dev(e)[0], w, s, 1.0))
        prod = (e2m1[codes[:, c]] * e4m3[scales[:, c // 16]]).astype(np.float32) + np.float32(0)
        assert np.array_equal(got, si.bf16_bits(prod)), c


def test_nvfp4_one_hot_columns_are_bitwise_weights():
    N, K = 300, 256
    g = np.random.default_rng(9)
    codes = g.integers(0, 16, size=(N, K), dtype=np.uint8)
    scales = g.integers(0x01, 0x7F, size=(N, K // 16), dtype=np.uint8)
    w, s = u32_dev(si.pack_codes(codes, 4)), u8_dev(scales)
    e2m1 = np.array([oracle.load().agqo_e2m1(c) for c in range(16)])
    e4m3 = np.array([oracle.load().agqo_e4m3(b) for b in range(256)])
    progress("nvfp4 one-hot columns")
    for c in list(range(0, 40)) + [127, 128, K - 1]:
        x = np.zeros((1, K), np.uint16)
        x[0, c] = 0x3F80
        y = agq.qmv_nvfp4(bf16_dev(x)[0], w, s, 1.0)
        torch.cuda.synchronize()
        # code 8 is -0: the kernel's sum starts at +0 and +0 + -0 is +0, so compare with +0
        prod = (e2m1[codes[:, c]] * e4m3[scales[:, c // 16]]).astype(np.float32) + np.float32(0)
        got, want = bf16_bits_host(y), si.bf16_bits(prod)
        bad = np.flatnonzero(got != want)
        assert bad.size == 0, (c, bad[:8], got[bad[:8]], want[bad[:8]])


def test_nvfp4_nan_scale_and_tensor_scale():
    """A NaN scale byte (S.1111.111) gives NaN in its row only; doubling the tensor scale
    doubles every output (one more exact factor of two before the rounding)."""
    N, K = 40, 512
    d = si.nvfp4_weight(10, 0, N, K)
    sc = d["scales"].copy()
    sc[3, 5] = 0x7F
    sc[17, 0] = 0xFF
    x = si.draw_activations(10, 1, 1, K)
    w, s = u32_dev(d["w"]), u8_dev(sc)
    progress("nvfp4 NaN scale and tensor scale")
    y1 = agq.qmv_nvfp4(bf16_dev(x)[0], w, s, 0.5)
    y2 = agq.qmv_nvfp4(bf16_dev(x)[0], w, s, 1.0)
    torch.cuda.synchronize()
    f1, f2 = y1.float().cpu().numpy(), y2.float().cpu().numpy()
    nan = np.isnan(f1)
    assert np.array_equal(np.flatnonzero(nan), [3, 17]) and np.array_equal(np.isnan(f2), nan)
    assert np.array_equal(f2[~nan], 2 * f1[~nan])
    y_ref, a = oracle.qmv_nvfp4(x, d["w"], sc, 1.0, K)
    check_close(y2[~torch.as_tensor(nan, device="cuda")].cpu().float().numpy().astype(np.float64)[None],
                y_ref[:, ~nan], a[:, ~nan], "non-NaN rows")


def test_nvfp4_is_deterministic():
    d = si.nvfp4_weight(11, 0, 4096, 14336)
    x = bf16_dev(si.draw_activations(11, 1, 2, 14336))
    w, s = u32_dev(d["w"]), u8_dev(d["scales"])
    progress("nvfp4 determinism")
    a = agq.qmv_nvfp4(x, w, s, d["tensor_scale"])
    b = agq.qmv_nvfp4(x, w, s, d["tensor_scale"])
    torch.cuda.synchronize()
    assert torch.equal(a, b)


# --------------------------------------------------------------------------- any M (agq_qmm_nvfp4)

def seam_rows(N):
    n = np.arange(N)
    keep = np.isin(n % 128, [0, 15, 16, 31, 32, 63, 64, 127]) | (n % 13 == 0) | (n == N - 1)
    return n[keep]


@pytest.mark.parametrize("M,N,K,sample", [
    (5, 300, 64, False), (8, 1000, 512, False), (17, 129, 1024, False), (64, 4096, 4096, True),
    (100, 333, 2048, False), (300, 2000, 4096, True), (255, 128, 192, False),
    # few rows on a large matrix (a K split of the 64-row tiles), K % 64 != 0 (passes of 4 rows)
    (16, 4096, 4096, True), (6, 500, 96, False), (13, 200, 2080, False),
    # K splits of the 256-row tiles
    (256, 4096, 4096, True), (300, 1000, 14336, True),
    # grids of 256-row tiles that fill the device
    (1024, 8192, 512, True), (2048, 4096, 1024, True), (1100, 33000, 256, True),
])
def test_qmm_nvfp4_shapes(M, N, K, sample):
    """The matrix-core NVFP4 GEMM (64- and 256-row tiles) against the oracle, with ragged
    activation and weight rows; seam rows and every 13th where the oracle would be slow."""
    d = si.nvfp4_weight(13, M + N, N, K)
    x = si.draw_activations(13, 100 + M, M, K)
    progress(f"qmm_nvfp4 M={M} N={N} K={K}")
    y = agq.qmm_nvfp4(bf16_dev(x), u32_dev(d["w"]), u8_dev(d["scales"]), d["tensor_scale"])
    torch.cuda.synchronize()
    rows = seam_rows(N) if sample else None
    y_ref, a = oracle.qmv_nvfp4(x, d["w"], d["scales"], d["tensor_scale"], K, rows=rows)
    yg = y if rows is None else y[:, torch.as_tensor(rows, device=y.device)]
    worst = check_close(yg, y_ref, a, f"qmm_nvfp4 M={M} N={N} K={K}", extra_half_ulp=K <= 128)
    progress(f"qmm_nvfp4: ok, worst |err|/A = {worst:.3e}")


@pytest.mark.parametrize("M,N", [(256, 300), (1024, 8192)])
def test_qmm_nvfp4_one_hot_columns_are_bitwise_weights(M, N):
    """x = e_k gives y[n] = bf16(e2m1(q[n, k]) * e4m3(s[n, k/16])) bit for bit on both tile
    sizes: the weight goes to the matrix cores exactly (code 8, -0, compared as +0)."""
    K = M
    g = np.random.default_rng([14, N])
    codes = g.integers(0, 16, size=(N, K), dtype=np.uint8)
    scales = g.integers(0x01, 0x7F, size=(N, K // 16), dtype=np.uint8)
    e2m1 = np.array([oracle.load().agqo_e2m1(c) for c in range(16)])
    e4m3 = np.array([oracle.load().agqo_e4m3(b) for b in range(256)])
    want = si.bf16_bits((e2m1[codes] * e4m3[np.repeat(scales, 16, axis=1)]).astype(np.float32) + np.float32(0))
    cols = np.arange(K)
    x = np.zeros((K, K), np.uint16)
    x[cols, cols] = 0x3F80
    progress(f"qmm_nvfp4 one-hot M={M} N={N}")
    got = bf16_bits_host(agq.qmm_nvfp4(bf16_dev(x), u32_dev(si.pack_codes(codes, 4)), u8_dev(scales), 1.0))
    bad = np.argwhere(got != want.T)
    assert bad.size == 0, (bad[:8], got[tuple(bad[:8].T)], want.T[tuple(bad[:8].T)])


def test_qmm_nvfp4_nan_scale_and_small_m_route():
    """A NaN scale byte makes NaN exactly the outputs of its weight row, in every activation
    row; up to 4 rows the call is the matvec product, bit for bit."""
    M, N, K = 64, 200, 512
    d = si.nvfp4_weight(15, 0, N, K)
    sc = d["scales"].copy()
    sc[7, 3] = 0xFF
    x = si.draw_activations(15, 1, M, K)
    w, s = u32_dev(d["w"]), u8_dev(sc)
    progress("qmm_nvfp4 NaN scale, small-M route")
    y = bf16_host(agq.qmm_nvfp4(bf16_dev(x), w, s, d["tensor_scale"]))
    nan = np.isnan(y)
    assert np.array_equal(np.flatnonzero(nan.any(axis=0)), [7]) and nan[:, 7].all()
    for m in (1, 3, 4):
        a = agq.qmm_nvfp4(bf16_dev(x[:m]), w, s, d["tensor_scale"])
        b = agq.qmv_nvfp4(bf16_dev(x[:m]), w, s, d["tensor_scale"])
        torch.cuda.synchronize()
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    # K % 64 != 0: passes of 4 rows for any M, bit for bit the matvec kernel's rows
    d2 = si.nvfp4_weight(15, 1, N, 96)
    x2 = si.draw_activations(15, 2, 11, 96)
    w2, s2 = u32_dev(d2["w"]), u8_dev(d2["scales"])
    a = bf16_bits_host(agq.qmm_nvfp4(bf16_dev(x2), w2, s2, 0.5))
    b = np.concatenate([bf16_bits_host(agq.qmv_nvfp4(bf16_dev(x2[r:r + 4]), w2, s2, 0.5)) for r in (0, 4, 8)])
    assert np.array_equal(a, b)


@pytest.mark.parametrize("M,N,K", [(16, 4096, 4096), (64, 1000, 8192), (256, 4096, 4096)])
def test_qmm_nvfp4_k_split_matches_unsplit_and_is_deterministic(M, N, K):
    """The K split (workspace from the binding) against the same call without one: within
    the oracle bound of each other, and bitwise repeatable; the tensor scale multiplies the
    sum of the splits."""
    need = agq.lib.agq_qmm_nvfp4_workspace(M, N, K)
    assert need > 0
    d = si.nvfp4_weight(16, M + N, N, K)
    x = si.draw_activations(16, 200 + M, M, K)
    xd, w, s = bf16_dev(x), u32_dev(d["w"]), u8_dev(d["scales"])
    progress(f"qmm_nvfp4 K split M={M} N={N} K={K}: {need // (4 * M * N)} splits")
    a = agq.qmm_nvfp4(xd, w, s, d["tensor_scale"])
    b = agq.qmm_nvfp4(xd, w, s, d["tensor_scale"])
    c = agq.qmm_nvfp4(xd, w, s, d["tensor_scale"], workspace=False)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    rows = seam_rows(N)
    y_ref, A = oracle.qmv_nvfp4(x, d["w"], d["scales"], d["tensor_scale"], K, rows=rows)
    ri = torch.as_tensor(rows, device=a.device)
    check_close(a[:, ri], y_ref, A, "split")
    check_close(c[:, ri], y_ref, A, "unsplit")
