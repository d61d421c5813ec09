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
from gpu_util import bf16_bits_host, bf16_dev, check_close, progress, u32_dev

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
