"""GPU parity of the quantized GEMM forms (agq_qmm, agq_gather_qmm) against the CPU oracle.

Same tolerance as the matvec forms: |y_gpu - y_ref| <= 2e-3 * sum_k |x_k * w_hat_k| per
output element, plus half a bf16 ulp of y_ref where K <= 128 (there |y| can come close to
that sum, and the bf16 output rounding alone can exceed 2e-3 of it). Shapes cover one and several 64-row activation tiles, ragged activation
and weight-row tails, K of one group, and both code widths. Where the oracle would take
minutes, the checked output rows are every row that sits on a tile or sub-tile seam (n
mod 128 in {0, 15, 16, 31, 32, 63, 64, 127}) plus every 13th row.
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


def seam_rows(N):
    n = np.arange(N)
    keep = np.isin(n % 128, [0, 15, 16, 31, 32, 63, 64, 127]) | (n % 13 == 0) | (n == N - 1)
    return n[keep]


def dev_weight(d):
    return u32_dev(d["w"]), bf16_dev(d["scales"]), bf16_dev(d["biases"])


@pytest.mark.parametrize("bits,M,N,K,sample", [
    (4, 9, 100, 512, False), (4, 16, 257, 4096, False), (4, 64, 128, 4096, False), (4, 65, 300, 1088, False),
    (4, 33, 64, 192, False), (4, 1, 5, 64, False), (4, 8, 1000, 4096, False), (4, 200, 131, 64, False),
    (4, 512, 4099, 4096, True), (4, 130, 14336, 4096, True), (4, 96, 4096, 14336, True),
    (8, 9, 100, 896, False), (8, 65, 300, 4864, False), (8, 100, 129, 64, False), (8, 512, 1000, 896, True),
    (4, 17, 129, 512, False), (4, 100, 333, 2048, False), (4, 128, 1000, 14336, True), (4, 300, 200, 4096, False),
    # enough 128x64 tiles for two blocks per compute unit: the large tile
    (4, 1024, 4100, 512, True), (8, 1000, 4096, 576, True),
    # grids of 128-row weight tiles that fill the device: the split-weight tiles
    # (256 x 128 and 128 x 128), with ragged activation rows and weight rows
    (4, 2048, 4096, 1024, True), (4, 1100, 33000, 256, True), (8, 2048, 4096, 512, True),
    (8, 700, 9000, 320, True), (4, 260, 16400, 2048, True),
    # 65-255 rows on the split-weight tiles (most rows of the 256-row tile empty): split
    # along K (65, 200 rows), and a grid that fills the device unsplit (100 rows)
    (4, 65, 4096, 4096, True), (8, 200, 4096, 2048, True), (4, 100, 28672, 1024, True),
    # 33-64 rows on 64-row split-weight tiles: split along K, and a full grid unsplit (49+ rows)
    (4, 48, 4096, 14336, True), (8, 40, 4096, 2048, True), (4, 64, 28672, 512, True), (4, 33, 3000, 4096, True),
    (4, 40, 28672, 512, True),
])
def test_qmm_shapes(bits, M, N, K, sample):
    """Shapes on both tile sizes: the 128x64 tile where it gives at least two blocks per
    compute unit (M > 128), the pipelined 64x64 tile otherwise."""
    d = si.draw_quantized_weight(30, 100 * bits + M, N, K, bits)
    x = si.draw_activations(30, 1000 + M, M, K)
    w, s, b = dev_weight(d)
    progress(f"qmm bits={bits} M={M} N={N} K={K}")
    y = agq.qmm(bf16_dev(x), w, s, b, bits=bits)
    torch.cuda.synchronize()
    rows = seam_rows(N) if sample else None
    y_ref, A = oracle.qmv(x, d["w"], d["scales"], d["biases"], K, bits, rows=rows)
    yg = y if rows is None else y[:, torch.as_tensor(rows, device=y.device)]
    # With one or two groups |y| can approach sum|x*w|, and then half a bf16 ulp of output
    # rounding alone exceeds 2e-3 of it: those shapes also allow that half ulp.
    worst = check_close(yg, y_ref, A, f"qmm M={M} N={N} K={K} bits={bits}", extra_half_ulp=K <= 128)
    progress(f"qmm: ok, worst |err|/A = {worst:.3e}")


@pytest.mark.parametrize("M", [9, 40, 128])
def test_qmm_passes_agree_with_the_tiled_gemm(M):
    """4-bit products of 9-64 rows (and up to 128 where split-weight tiles would leave the
    device idle, as here: 5 weight tiles) run on the matrix-core matvec kernel, one grid row
    per 16-row pass; the same rows through agq_gather_qmm (identity routing onto one plane,
    the tiled GEMM) meet the same tolerance against the oracle."""
    N, K = 520, 2048
    d = si.draw_quantized_weight(35, M, N, K, 4)
    x = si.draw_activations(35, 100 + M, M, K)
    w, s, b = dev_weight(d)
    xd = bf16_dev(x)
    progress(f"qmm passes vs tiled M={M}")
    y1 = agq.qmm(xd, w, s, b)
    zero = u32_dev(np.zeros(M, np.uint32))
    y2 = agq.gather_qmm(xd, w[None], s[None], b[None], rhs_indices=zero,
                        lhs_indices=u32_dev(np.arange(M, dtype=np.uint32)))
    torch.cuda.synchronize()
    y_ref, A = oracle.qmv(x, d["w"], d["scales"], d["biases"], K, 4)
    check_close(y1, y_ref, A, "passes")
    check_close(y2, y_ref, A, "tiled")


def test_qmm_is_deterministic_and_scales_by_powers_of_two():
    N, K, M = 700, 4096, 100
    d = si.draw_quantized_weight(31, 1, N, K, 4)
    w, s, b = dev_weight(d)
    xd = bf16_dev(si.draw_activations(31, 2, M, K))
    progress("qmm determinism")
    y1 = bf16_bits_host(agq.qmm(xd, w, s, b))
    y2 = bf16_bits_host(agq.qmm(xd, w, s, b))
    assert np.array_equal(y1, y2)
    assert np.array_equal(bf16_host(agq.qmm(xd * 8, w, s, b)), 8 * bf16_host(agq.qmm(xd, w, s, b)))


@pytest.mark.parametrize("bits", [4, 8])
def test_qmm_one_hot_columns_are_bitwise_weights(bits):
    """x = e_k gives y[n] = bf16(w_hat[n, k]) exactly on the matrix-core GEMM (one exact
    product per output; the group correction cancels the 128 offset exactly)."""
    N, K = 300, 256
    d = si.draw_quantized_weight(32, bits, N, K, bits)
    w, s, b = dev_weight(d)
    ref, bad = oracle.dequantize(d["w"], d["scales"], d["biases"], K, bits)
    assert bad == 0
    want = si.bf16_bits(ref.astype(np.float32))
    cols = np.arange(K)
    x = np.zeros((K, K), np.uint16)
    x[cols, cols] = 0x3F80
    progress(f"qmm one-hot bits={bits}")
    got = bf16_bits_host(agq.qmm(bf16_dev(x), w, s, b, bits=bits))
    assert np.array_equal(got, want.T)


@pytest.mark.parametrize("bits", [4, 8])
def test_qmm_split_weight_tiles_one_hot_bitwise(bits):
    """On the split-weight tiles (a grid that fills the device), x = e_k gives
    y[n] = bf16(w_hat[n, k]) bit for bit: the weights of the quantizer's recipe need at
    most 16 significant bits, so their bfloat16 parts hi + lo hold them exactly."""
    N, K = 8192, 1024
    d = si.draw_quantized_weight(33, bits, N, K, bits)
    w, s, b = dev_weight(d)
    ref, bad = oracle.dequantize(d["w"], d["scales"], d["biases"], K, bits)
    assert bad == 0
    want = si.bf16_bits(ref.astype(np.float32))
    cols = np.arange(K)
    x = np.zeros((K, K), np.uint16)
    x[cols, cols] = 0x3F80
    progress(f"qmm split-weight one-hot bits={bits}")
    got = bf16_bits_host(agq.qmm(bf16_dev(x), w, s, b, bits=bits))
    assert np.array_equal(got, want.T)


# --------------------------------------------------------------------------- K splits

@pytest.mark.parametrize("bits,M,N,K", [
    (4, 100, 4096, 4096),    # 100 rows: 8 splits of one 256-row tile row; unsplit, the matvec passes
    (4, 256, 4096, 4096),    # 32 split-weight tiles, 8 splits of 8 groups
    (4, 256, 1000, 14336),   # 8 tiles, 32 splits of 7 groups
    (8, 300, 2000, 2048),    # 8-bit, ragged rows, 8 splits of 4 groups
    (4, 257, 3000, 2560),    # one row past a tile, ragged weight rows, 5 splits of 8 groups
])
def test_qmm_k_split_against_oracle_and_unsplit(bits, M, N, K):
    """Where the split-weight tiles alone leave compute units idle, the call splits K
    (workspace from the binding): parity with the oracle on seam rows, agreement with the
    unsplit kernels within the same bound, and bitwise determinism of the split path."""
    need = agq.lib.agq_qmm_workspace(M, N, K, bits, 64)
    assert need > 0 and need % (4 * M * N) == 0, need
    d = si.draw_quantized_weight(36, 100 * bits + M, N, K, bits)
    x = si.draw_activations(36, 1000 + M, M, K)
    w, s, b = dev_weight(d)
    xd = bf16_dev(x)
    progress(f"qmm K split bits={bits} M={M} N={N} K={K}: {need // (4 * M * N)} splits")
    y = agq.qmm(xd, w, s, b, bits=bits)
    y2 = agq.qmm(xd, w, s, b, bits=bits)
    y0 = agq.qmm(xd, w, s, b, bits=bits, workspace=False)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))
    rows = seam_rows(N)
    y_ref, A = oracle.qmv(x, d["w"], d["scales"], d["biases"], K, bits, rows=rows)
    ri = torch.as_tensor(rows, device=y.device)
    worst = check_close(y[:, ri], y_ref, A, f"split M={M} N={N} K={K}")
    check_close(y0[:, ri], y_ref, A, f"unsplit M={M} N={N} K={K}")
    progress(f"qmm K split: ok, worst |err|/A = {worst:.3e}")


def test_qmm_k_split_one_hot_bitwise():
    """x = e_k through a K split: one split holds the exact weight, the others +0, so the
    in-order sum and the one bf16 rounding give bf16(w_hat[n, k]) bit for bit."""
    N, K = 4096, 1024
    assert agq.lib.agq_qmm_workspace(K, N, K, 4, 64) > 0
    d = si.draw_quantized_weight(37, 4, N, K, 4)
    w, s, b = dev_weight(d)
    ref, bad = oracle.dequantize(d["w"], d["scales"], d["biases"], K, 4)
    assert bad == 0
    want = si.bf16_bits(ref.astype(np.float32))
    cols = np.arange(K)
    x = np.zeros((K, K), np.uint16)
    x[cols, cols] = 0x3F80
    progress("qmm K split one-hot")
    got = bf16_bits_host(agq.qmm(bf16_dev(x), w, s, b))
    assert np.array_equal(got, want.T)


def test_qmm_small_split_weight_tile_one_hot_bitwise():
    """64 one-hot rows (x = e_c for 64 columns across chunk, group and K-split seams) on the
    64-row split-weight tile split along K: y[m, n] = bf16(w_hat[n, c_m]) bit for bit."""
    N, K, M = 8192, 1024, 64
    assert agq.lib.agq_qmm_workspace(M, N, K, 4, 64) > 0
    d = si.draw_quantized_weight(39, 4, N, K, 4)
    w, s, b = dev_weight(d)
    ref, bad = oracle.dequantize(d["w"], d["scales"], d["biases"], K, 4)
    assert bad == 0
    want = si.bf16_bits(ref.astype(np.float32))
    cols = np.array(list(range(0, 34)) + [63, 64, 65, 127, 128, 255, 256, 257, 511, 512, 513, 639, 640, 767, 768,
                                          895, 896, 1000, 1020, 1021, 1022, 1023, 300, 400, 700, 800, 900, 950, 960,
                                          970][:M])
    assert len(set(cols.tolist())) == M
    x = np.zeros((M, K), np.uint16)
    x[np.arange(M), cols] = 0x3F80
    progress("qmm 64-row split-weight tile one-hot")
    got = bf16_bits_host(agq.qmm(bf16_dev(x), w, s, b))
    assert np.array_equal(got, want[:, cols].T)


def test_qmm_k_splits_in_a_graph():
    """The split GEMM and its reduction (affine and NVFP4) and an unsplit GEMM captured in one
    HIP graph: every replay, with the workspaces overwritten with NaN bytes, the outputs
    cleared and eager work in between, reproduces the eager outputs bit for bit (no part of
    the split path depends on earlier workspace contents)."""
    M, N, K = 256, 4096, 4096
    d = si.draw_quantized_weight(40, 0, N, K, 4)
    w, s, b = dev_weight(d)
    nv = si.nvfp4_weight(40, 1, N, K)
    wn = u32_dev(nv["w"])
    sn = torch.from_numpy(np.ascontiguousarray(nv["scales"])).to("cuda")
    xd = bf16_dev(si.draw_activations(40, 2, M, K))
    need_a = agq.lib.agq_qmm_workspace(M, N, K, 4, 64)
    need_n = agq.lib.agq_qmm_nvfp4_workspace(64, N, K)
    assert need_a > 0 and need_n > 0
    ws_a = torch.empty(need_a, dtype=torch.uint8, device="cuda")
    ws_n = torch.empty(need_n, dtype=torch.uint8, device="cuda")
    ya = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    yn = torch.empty((64, N), dtype=torch.bfloat16, device="cuda")
    yu = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    outs = (ya, yn, yu)
    x64 = xd[:64].contiguous()

    def run():
        agq.qmm(xd, w, s, b, out=ya, workspace=ws_a)
        agq.qmm_nvfp4(x64, wn, sn, nv["tensor_scale"], out=yn, workspace=ws_n)
        agq.qmm(xd, w, s, b, out=yu, workspace=False)

    progress("graph capture of split and unsplit GEMMs")
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        run()
    torch.cuda.synchronize()
    eager = [bf16_bits_host(t).copy() for t in outs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        run()
    torch.cuda.synchronize()
    for rep in range(4):
        for t in outs:
            t.zero_()
        ws_a.fill_(0xFF)
        ws_n.fill_(0xFF)
        agq.qmm(xd[:100].contiguous(), w, s, b)  # unrelated eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for got, want in zip(outs, eager):
            assert np.array_equal(bf16_bits_host(got), want), f"replay {rep}"


def test_qmm_workspace_checks():
    """A workspace below the queried size or off 16-byte alignment is AGQ_EINVAL before any
    launch; a larger one, and none at all, run; calls that need none ignore it."""
    M, N, K = 256, 4096, 4096
    need = agq.lib.agq_qmm_workspace(M, N, K, 4, 64)
    assert need > 0
    assert agq.lib.agq_qmm_workspace(8, N, K, 4, 64) == 0          # matvec
    assert agq.lib.agq_qmm_workspace(2048, N, K, 4, 64) == 0       # grid fills the device
    assert agq.lib.agq_qmm_workspace(M, N, K, 4, 32) == 0          # not a GEMM format
    d = si.draw_quantized_weight(38, 0, N, K, 4)
    w, s, b = dev_weight(d)
    xd = bf16_dev(si.draw_activations(38, 1, M, K))
    ws = torch.empty(need + 64, dtype=torch.uint8, device="cuda")
    with pytest.raises(agq.AgqError) as e:
        agq.qmm(xd, w, s, b, workspace=ws[:need - 16])
    assert e.value.status == agq.AGQ_EINVAL
    with pytest.raises(agq.AgqError) as e:
        agq.qmm(xd, w, s, b, workspace=ws[8:8 + need])
    assert e.value.status == agq.AGQ_EINVAL
    a = agq.qmm(xd, w, s, b, workspace=ws)
    c = agq.qmm(xd, w, s, b, workspace=ws[16:16 + need])
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), c.view(torch.int16))


@pytest.fixture(scope="module")
def moe_w1():
    progress("generating the Mixtral-shaped W1 planes")
    return si.workload(4, only=("w1",))["w1"]


def test_gather_qmm_mixtral_prefill(moe_w1):
    """512 tokens, top-2 of 8 experts (1024 pairs) through the Mixtral-shaped W1 planes."""
    m = moe_w1
    pre = si.moe_prefill(512)
    E, N, K = m["E"], m["N"], m["K"]
    progress(f"gather_qmm prefill P={len(pre['rhs'])} E={E} N={N} K={K}")
    y = agq.gather_qmm(bf16_dev(pre["x"]), u32_dev(m["w"]), bf16_dev(m["scales"]), bf16_dev(m["biases"]),
                       rhs_indices=u32_dev(pre["rhs"]), lhs_indices=u32_dev(pre["lhs"]))
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([seam_rows(N)[::4], [0, 127, 128, N - 1]]))
    y_ref, A = oracle.gather_qmv(pre["x"], m["w"], m["scales"], m["biases"], pre["lhs"], pre["rhs"], K, 4,
                                 rows=rows)
    worst = check_close(y[:, torch.as_tensor(rows, device=y.device)], y_ref, A, "gather_qmm prefill")
    progress(f"gather_qmm prefill: ok, worst |err|/A = {worst:.3e}")


@pytest.mark.parametrize("bits", [4, 8])
def test_gather_qmm_edges(bits):
    """Experts with 0, 1, 64, 65 and 150 pairs, repeated and scattered x rows, an
    out-of-range pair of each kind (NaN rows), and NULL indices as the identity."""
    E, N, K, R = 5, 200, 1024, 70
    planes = [si.draw_quantized_weight(33, 10 * bits + e, N, K, bits) for e in range(E)]
    st = {k: np.stack([p[k] for p in planes]) for k in ("w", "scales", "biases")}
    x = si.draw_activations(33, bits, R, K)
    rng = np.random.default_rng([33, bits])
    rhs = np.array([1] * 1 + [2] * 64 + [3] * 65 + [4] * 150, np.uint32)
    rng.shuffle(rhs)
    lhs = rng.integers(0, R, len(rhs)).astype(np.uint32)
    lhs_bad, rhs_bad = lhs.copy(), rhs.copy()
    lhs_bad[7], rhs_bad[11] = R + 3, E
    w, s, b = u32_dev(st["w"]), bf16_dev(st["scales"]), bf16_dev(st["biases"])
    xd = bf16_dev(x)
    progress(f"gather_qmm edges bits={bits}")
    y = agq.gather_qmm(xd, w, s, b, rhs_indices=u32_dev(rhs_bad), lhs_indices=u32_dev(lhs_bad), bits=bits)
    torch.cuda.synchronize()
    yh = bf16_host(y)
    assert np.all(np.isnan(yh[7])) and np.all(np.isnan(yh[11]))
    ok = np.array([p for p in range(len(rhs)) if p not in (7, 11)])
    y_ref, A = oracle.gather_qmv(x, st["w"], st["scales"], st["biases"], lhs[ok], rhs[ok], K, bits)
    check_close(y[torch.as_tensor(ok, device=y.device)], y_ref, A, "gather_qmm edges")
    # the matvec gather gives results within the same tolerance
    yv = agq.gather_qmv(xd, w, s, b, rhs_indices=u32_dev(rhs), lhs_indices=u32_dev(lhs), bits=bits)
    check_close(yv[torch.as_tensor(ok, device=y.device)], y_ref, A, "gather_qmv edges")
    # NULL indices: identity
    y_id = agq.gather_qmm(xd[:E], w, s, b, bits=bits)
    y_ex = agq.gather_qmm(xd[:E], w, s, b, rhs_indices=u32_dev(np.arange(E, dtype=np.uint32)),
                          lhs_indices=u32_dev(np.arange(E, dtype=np.uint32)), bits=bits)
    torch.cuda.synchronize()
    assert np.array_equal(bf16_bits_host(y_id), bf16_bits_host(y_ex))


@pytest.mark.parametrize("bits", [4, 8])
def test_gather_qmm_split_weight_tiles(bits):
    """About 512 pairs per plane on planes of 8192 rows: the split-weight tiles (256 x 128),
    with ragged pair counts per plane, an empty plane, repeated x rows and one
    out-of-range pair of each kind (NaN rows). Checked on tile-seam weight rows."""
    E, N, K, R, P = 5, 8192, 256, 300, 2048
    planes = [si.draw_quantized_weight(36, 10 * bits + e, N, K, bits) for e in range(E)]
    st = {k: np.stack([p[k] for p in planes]) for k in ("w", "scales", "biases")}
    x = si.draw_activations(36, bits, R, K)
    rng = np.random.default_rng([36, bits])
    rhs = rng.integers(0, E - 1, P).astype(np.uint32)  # plane E - 1 stays empty
    lhs = rng.integers(0, R, P).astype(np.uint32)
    lhs[5], rhs[9] = R + 1, E + 2
    progress(f"gather_qmm split-weight tiles bits={bits}")
    y = agq.gather_qmm(bf16_dev(x), u32_dev(st["w"]), bf16_dev(st["scales"]), bf16_dev(st["biases"]),
                       rhs_indices=u32_dev(rhs), lhs_indices=u32_dev(lhs), bits=bits)
    torch.cuda.synchronize()
    yh = bf16_host(y)
    assert np.all(np.isnan(yh[5])) and np.all(np.isnan(yh[9]))
    ok = np.array([p for p in range(P) if p not in (5, 9)])
    rows = seam_rows(N)
    y_ref, A = oracle.gather_qmv(x, st["w"], st["scales"], st["biases"], lhs[ok], rhs[ok], K, bits, rows=rows)
    yg = y[torch.as_tensor(ok, device=y.device)][:, torch.as_tensor(rows, device=y.device)]
    check_close(yg, y_ref, A, f"gather_qmm split-weight bits={bits}")


def test_gather_qmm_at_the_pair_limit():
    E, N, K, R, P = 3, 96, 512, 64, 4096
    planes = [si.draw_quantized_weight(34, e, N, K, 4) for e in range(E)]
    st = {k: np.stack([p[k] for p in planes]) for k in ("w", "scales", "biases")}
    x = si.draw_activations(34, 99, R, K)
    rng = np.random.default_rng([34, 1])
    lhs = rng.integers(0, R, P).astype(np.uint32)
    rhs = rng.integers(0, E, P).astype(np.uint32)
    progress("gather_qmm with 4096 pairs")
    y = agq.gather_qmm(bf16_dev(x), u32_dev(st["w"]), bf16_dev(st["scales"]), bf16_dev(st["biases"]),
                       rhs_indices=u32_dev(rhs), lhs_indices=u32_dev(lhs))
    torch.cuda.synchronize()
    y_ref, A = oracle.gather_qmv(x, st["w"], st["scales"], st["biases"], lhs, rhs, K, 4)
    check_close(y, y_ref, A, "gather_qmm 4096 pairs")
