"""GPU parity of the format breadth: the device quantizer (every width) and group sizes 32 and 128.

The quantizer's codes, scales and biases must equal the oracle's bit for bit (every step
is one IEEE binary32 operation on both sides, so each code is decided in the same
precision). Products at group sizes 32 and 128 run on the VALU kernels and meet the usual
tolerance, |y_gpu - y_ref| <= 2e-3 * sum_k |x_k * w_hat_k|; their dequantization is
bitwise, and one-hot columns give bf16(w_hat) exactly.
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


def weights(seed, N, K):
    """N(0, 0.02) rows, a quarter of them offset far from zero (rounding the scale and the
    bias then pushes values past the grid ends: the clamp), one constant group."""
    g = np.random.default_rng([80, seed])
    w = (0.02 * g.standard_normal((N, K))).astype(np.float32)
    w[: N // 4] += (50 * g.random((N // 4, 1)) + 1).astype(np.float32)
    w[N // 2, :128] = np.float32(0.375)
    return w


@pytest.mark.parametrize("bits", [2, 3, 4, 5, 6, 8])
@pytest.mark.parametrize("gs", [32, 64, 128])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_quantize_bit_exact(bits, gs, dtype):
    N, K = 301, 1024
    w = weights(100 * bits + gs, N, K)
    if dtype == "bf16":
        wh = si.bf16_bits(w)
        w = si.bf16_to_f32(wh)
        wd = bf16_dev(wh)
    else:
        wd = torch.as_tensor(w, device="cuda")
    progress(f"quantize bits={bits} gs={gs} {dtype}")
    codes, sc, bi = agq.quantize(wd, bits=bits, group_size=gs)
    torch.cuda.synchronize()
    wq_ref, sc_ref, bi_ref = oracle.quantize(w, bits, gs)
    assert np.array_equal(codes.cpu().numpy().view(np.uint32), wq_ref)
    assert np.array_equal(bf16_bits_host(sc), sc_ref)
    assert np.array_equal(bf16_bits_host(bi), bi_ref)


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("gs,M,N,K", [(32, 1, 1000, 4096), (128, 1, 777, 4096), (32, 3, 300, 14336),
                                      (128, 5, 513, 2048), (32, 8, 64, 96), (128, 2, 200, 8192)])
def test_products_at_other_group_sizes(bits, gs, M, N, K):
    w = (0.02 * np.random.default_rng([81, bits, gs, M]).standard_normal((N, K))).astype(np.float32)
    q, sc, bi = si.quantize_rows(w, bits, group_size=gs)
    wq = si.pack_codes(q, bits)
    x = si.draw_activations(81, 100 * gs + M, M, K)
    progress(f"products gs={gs} bits={bits} M={M} N={N} K={K}")
    wd, sd, bd = u32_dev(wq), bf16_dev(sc), bf16_dev(bi)
    xd = bf16_dev(x)
    plan = agq.launch_plan(M, N, K, bits, group_size=gs)
    assert plan["engine"] == 0
    y = agq.qmv(xd[0], wd, sd, bd, bits=bits, group_size=gs)[None] if M == 1 else \
        agq.qmv_wide(xd, wd, sd, bd, bits=bits, group_size=gs)
    torch.cuda.synchronize()
    y_ref, A = oracle.qmv(x, wq, sc, bi, K, bits, group_size=gs)
    check_close(y, y_ref, A, f"gs={gs} M={M}", extra_half_ulp=K <= 128)
    # dequantization, bit for bit
    deq = agq.dequantize(wd, sd, bd, bits=bits, group_size=gs)
    ref, bad = oracle.dequantize(wq, sc, bi, K, bits, group_size=gs)
    assert bad == 0
    assert np.array_equal(deq.cpu().numpy(), ref.astype(np.float32))


def test_large_batch1_4bit_products_take_the_stream_kernel():
    """Batch-1 4-bit gs64 products whose 16-row blocks number at least two per compute
    unit run on the bit-stream kernel (engine 2); short grids stay on the VALU plans."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    for N, K in ((128256, 4096), (28672, 4096), (6144, 4096), (4096, 4096), (4096, 14336)):
        want = 2 if -(-N // 16) >= 2 * cus else 0
        assert agq.launch_plan(1, N, K, 4)["engine"] == want, (N, K)
    assert agq.launch_plan(2, 128256, 4096, 4)["engine"] == 0        # one activation row only
    assert agq.launch_plan(1, 128256, 4096, 4, group_size=128)["engine"] == 0


def test_stream_route_ragged_rows_and_chunk():
    """The batch-1 4-bit route to the bit-stream kernel on a ragged shape: N not a multiple
    of 16 rows (a last block with 3 rows, waves without rows) and K with a partial last
    4096-column chunk; every row against the oracle, and one-hot columns bit for bit."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    N, K = 2 * cus * 16 + 3, 4096 + 64 * 3
    assert agq.launch_plan(1, N, K, 4)["engine"] == 2
    d = si.draw_quantized_weight(83, 0, N, K, 4)
    x = si.draw_activations(83, 1, 1, K)
    w, s, b = u32_dev(d["w"]), bf16_dev(d["scales"]), bf16_dev(d["biases"])
    progress(f"stream route ragged N={N} K={K}")
    y = agq.qmv(bf16_dev(x)[0], w, s, b, bits=4)[None]
    torch.cuda.synchronize()
    y_ref, A = oracle.qmv(x, d["w"], d["scales"], d["biases"], K, 4)
    check_close(y, y_ref, A, "stream route ragged")
    ref, bad = oracle.dequantize(d["w"], d["scales"], d["biases"], K, 4)
    assert bad == 0
    want = si.bf16_bits(ref.astype(np.float32))
    for c in (0, 1, 7, 8, 63, 4095, 4096, 4097, K - 1):
        e = np.zeros((1, K), np.uint16)
        e[0, c] = 0x3F80
        got = bf16_bits_host(agq.qmv(bf16_dev(e)[0], w, s, b, bits=4))
        assert np.array_equal(got, want[:, c]), c


@pytest.mark.parametrize("gs", [32, 128])
def test_deep_plan_at_other_group_sizes(gs):
    """Batch-1 4-bit products over 128256 rows at group sizes 32 and 128 take the VALU deep
    plan (two rows per iteration, x from L2); sampled rows, the last 40 among them, meet the
    oracle bound. (4096 drawn rows tiled down the matrix: every row's address is walked.)"""
    N, K, base = 128256, 4096, 4096
    w = (0.02 * np.random.default_rng([82, gs]).standard_normal((base, K))).astype(np.float32)
    q, sc, bi = si.quantize_rows(w, 4, group_size=gs)
    reps = -(-N // base)
    wq = np.tile(si.pack_codes(q, 4), (reps, 1))[:N]
    sc, bi = np.tile(sc, (reps, 1))[:N], np.tile(bi, (reps, 1))[:N]
    x = si.draw_activations(82, gs, 1, K)
    plan = agq.launch_plan(1, N, K, 4, group_size=gs)
    assert plan["engine"] == 0 and plan["rows_per_iter"] == 2 and plan["x_lds_bytes"] == 0
    progress(f"deep plan gs={gs}")
    y = agq.qmv(bf16_dev(x)[0], u32_dev(wq), bf16_dev(sc), bf16_dev(bi), bits=4, group_size=gs)[None]
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([np.arange(0, N, 997), np.arange(N - 40, N)]))
    y_ref, A = oracle.qmv(x, wq, sc, bi, K, 4, group_size=gs, rows=rows)
    check_close(y[:, torch.as_tensor(rows, device=y.device)], y_ref, A, f"deep plan gs={gs}")


@pytest.mark.parametrize("gs", [32, 128])
def test_one_hot_and_gather_at_other_group_sizes(gs):
    bits, N, K, E = 4, 300, 1024, 3
    planes = []
    for e in range(E):
        w = (0.02 * np.random.default_rng([82, gs, e]).standard_normal((N, K))).astype(np.float32)
        q, sc, bi = si.quantize_rows(w, bits, group_size=gs)
        planes.append({"w": si.pack_codes(q, bits), "scales": sc, "biases": bi})
    st = {k: np.stack([p[k] for p in planes]) for k in ("w", "scales", "biases")}
    wd, sd, bd = u32_dev(st["w"]), bf16_dev(st["scales"]), bf16_dev(st["biases"])
    # one-hot columns through the batch-1 product: bf16(w_hat) bit for bit
    ref, _ = oracle.dequantize(st["w"][0], st["scales"][0], st["biases"][0], K, bits, group_size=gs)
    want = si.bf16_bits(ref.astype(np.float32))
    progress(f"one-hot and gather gs={gs}")
    for c in list(range(0, 70)) + [gs - 1, gs, K - 1]:
        x = np.zeros((1, K), np.uint16)
        x[0, c] = 0x3F80
        y = agq.qmv(bf16_dev(x)[0], wd[0], sd[0], bd[0], bits=bits, group_size=gs)
        torch.cuda.synchronize()
        assert np.array_equal(bf16_bits_host(y), want[:, c]), c
    # the gather (VALU form at group sizes other than 64)
    R = 6
    x = si.draw_activations(82, gs, R, K)
    lhs = np.array([0, 1, 1, 5, 3, 2, 4], np.uint32)
    rhs = np.array([2, 0, 1, 2, 2, 1, 0], np.uint32)
    y = agq.gather_qmv(bf16_dev(x), wd, sd, bd, rhs_indices=u32_dev(rhs), lhs_indices=u32_dev(lhs), bits=bits,
                       group_size=gs)
    torch.cuda.synchronize()
    y_ref, A = oracle.gather_qmv(x, st["w"], st["scales"], st["biases"], lhs, rhs, K, bits, group_size=gs)
    check_close(y, y_ref, A, f"gather gs={gs}")


def test_device_quantized_weights_feed_the_products():
    """Quantize on the device, multiply on the device, compare with the oracle on the same
    codes (which equal its own quantizer's)."""
    N, K = 2048, 4096
    w = (0.02 * np.random.default_rng(83).standard_normal((N, K))).astype(np.float32)
    x = si.draw_activations(83, 1, 1, K)
    progress("device quantize -> qmv")
    codes, sc, bi = agq.quantize(torch.as_tensor(w, device="cuda"), bits=4)
    y = agq.qmv(bf16_dev(x)[0], codes, sc, bi)
    torch.cuda.synchronize()
    wq, s_ref, b_ref = oracle.quantize(w, 4)
    assert np.array_equal(codes.cpu().numpy().view(np.uint32), wq)
    y_ref, A = oracle.qmv(x, wq, s_ref, b_ref, K, 4)
    check_close(y[None], y_ref, A, "quantize -> qmv")
