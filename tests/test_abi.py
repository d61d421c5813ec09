"""C-ABI tests that need no GPU: exported symbols, host-side validation, launch plans.

Each validation case is malformed or unsupported, so the library rejects it
before any HIP call; no fake pointer ever reaches a kernel.
"""
import ctypes
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "agq.h")

agq = pytest.importorskip("affine_group_quantized_amd")
lib = agq.lib

EINVAL, ENOTSUP = agq.AGQ_EINVAL, agq.AGQ_ENOTSUP
A = ctypes.c_void_p(0x10000)      # 16-byte aligned stand-in address (never dereferenced)
A2 = ctypes.c_void_p(0x10002)     # 2-byte aligned, not 16
NUL = None


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(agq_[a-z_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for want in ("agq_qmv", "agq_qmv_wide", "agq_gather_qmv", "agq_qmm", "agq_gather_qmm", "agq_dequantize",
                 "agq_status_str", "agq_last_error", "agq_version", "agq_plan_product", "agq_plan_launch"):
        assert want in names


@pytest.mark.parametrize("name", declared_functions())
def test_library_exports_every_declared_symbol(name):
    assert hasattr(lib, name), name


def test_moe_workspace_size():
    lib.agq_moe_decode_workspace.argtypes = [ctypes.c_int64] * 4
    lib.agq_moe_decode_workspace.restype = ctypes.c_int64
    assert lib.agq_moe_decode_workspace(16, 2, 4096, 14336) == 4 * 32 * (14336 + 4096)
    assert lib.agq_moe_decode_workspace(0, 2, 4096, 14336) == 0


def test_gemm_workspace_sizes_of_calls_that_need_none():
    """Calls that are not K-split GEMMs need no workspace (answered on the host)."""
    assert lib.agq_qmm_workspace(0, 4096, 4096, 4, 64) == 0
    assert lib.agq_qmm_workspace(63, 4096, 4096, 3, 64) == 0    # bit-stream widths: passes below 64 rows
    assert lib.agq_qmm_workspace(256, 4096, 4096, 3, 128) == 0
    assert lib.agq_qmm_workspace(256, 4096, 4096, 4, 32) == 0
    assert lib.agq_qmm_workspace(8, 4096, 4096, 4, 64) == 0
    assert lib.agq_qmm_workspace(64, 4096, 4096, 4, 64) == 0    # matrix-core matvec passes
    assert lib.agq_qmm_nvfp4_workspace(4, 4096, 4096) == 0
    assert lib.agq_qmm_nvfp4_workspace(64, 4096, 48) == 0


def test_gemm_workspace_of_the_widened_bit_stream_codes():
    """From 64 rows the bit-stream widths widen their codes to 8 bits in the workspace:
    at least N*K bytes (plus the 8-bit GEMM's split partials where a device is present)."""
    for bits in (2, 3, 5, 6):
        assert lib.agq_qmm_workspace(64, 4096, 4096, bits, 64) >= 4096 * 4096
        assert lib.agq_qmm_workspace(2048, 100, 1024, bits, 64) >= 100 * 1024


def test_status_strings():
    assert lib.agq_status_str(0) == b"AGQ_OK"
    assert lib.agq_status_str(1) == b"AGQ_EINVAL"
    assert lib.agq_status_str(2) == b"AGQ_ENOTSUP"
    assert lib.agq_status_str(3) == b"AGQ_EHIP"
    assert lib.agq_version() >= 100


def qmv(x=A, w=A, s=A, b=A, y=A, N=16, K=64, bits=4, gs=64):
    return lib.agq_qmv(x, w, s, b, y, N, K, bits, gs, None)


def wide(M=2, x=A, N=16, K=64, bits=4, gs=64):
    return lib.agq_qmv_wide(x, A, A, A, A, M, N, K, bits, gs, None)


def gather(P=4, R=4, E=4, N=16, K=64, bits=4, gs=64, lhs=A, rhs=A, x=A):
    return lib.agq_gather_qmv(x, A, A, A, lhs, rhs, A, P, R, E, N, K, bits, gs, None)


def qmm(M=16, x=A, N=16, K=64, bits=4, gs=64, y=A, ws=NUL, wsb=0):
    return lib.agq_qmm(x, A, A, A, y, M, N, K, bits, gs, ws, wsb, None)


def moe(T=4, k=2, E=4, H=512, F=1024, bits=4, gs=64, x=A, ws=A, wsb=1 << 30, ex=A):
    return lib.agq_moe_decode(x, A, A, A, A, A, A, A, A, A, ex, A, A, ws, wsb, T, k, E, H, F, bits, gs, None)


def fused(act=0, g=A, eps=1e-5, res=NUL, N=16, K=64, bits=4, gs=64, x=A, y=A):
    return lib.agq_qmv_fused(x, g, eps, A, A, A, res, act, y, N, K, bits, gs, None)


def nvfp4(M=1, N=16, K=64, ts=1.0, x=A, w=A, s=A, y=A):
    return lib.agq_qmv_nvfp4(x, w, s, ts, y, M, N, K, None)


def nvfp4mm(M=64, N=16, K=64, ts=1.0, x=A, w=A, s=A, y=A, ws=NUL, wsb=0):
    return lib.agq_qmm_nvfp4(x, w, s, ts, y, M, N, K, ws, wsb, None)


def gqmm(P=4, R=4, E=4, N=16, K=64, bits=4, gs=64, lhs=A, rhs=A, x=A):
    return lib.agq_gather_qmm(x, A, A, A, lhs, rhs, A, P, R, E, N, K, bits, gs, None)


@pytest.mark.parametrize("call,status", [
    (lambda: qmv(x=NUL), EINVAL),
    (lambda: qmv(w=NUL), EINVAL),
    (lambda: qmv(y=NUL), EINVAL),
    (lambda: qmv(N=0), EINVAL),
    (lambda: qmv(K=0), EINVAL),
    (lambda: qmv(N=-3), EINVAL),
    (lambda: qmv(K=96), EINVAL),
    (lambda: qmv(bits=7), ENOTSUP),
    (lambda: qmv(bits=9), ENOTSUP),
    (lambda: qmv(bits=1), ENOTSUP),
    (lambda: qmv(bits=3, gs=32, K=128), ENOTSUP),   # the bit-stream widths take group size 64
    (lambda: wide(M=9, bits=5), ENOTSUP),
    (lambda: gather(bits=3, gs=32, K=128), ENOTSUP),  # the bit-stream gathers take group size 64
    (lambda: gqmm(bits=6, gs=128, K=128), ENOTSUP),
    (lambda: qmm(bits=5, gs=128, K=128), ENOTSUP),
    (lambda: qmv(gs=16), ENOTSUP),
    (lambda: qmv(gs=256, K=256), ENOTSUP),
    (lambda: qmv(gs=32, K=48), EINVAL),
    (lambda: qmv(gs=0), EINVAL),
    (lambda: qmv(x=A2), EINVAL),
    (lambda: qmv(w=A2), EINVAL),
    (lambda: qmv(s=ctypes.c_void_p(0x10001)), EINVAL),
    (lambda: qmv(N=1 << 41), EINVAL),
    (lambda: qmv(K=1 << 31), EINVAL),
    (lambda: qmv(K=114688 + 64), ENOTSUP),
    (lambda: qmv(K=57344 + 64, bits=8), ENOTSUP),
    (lambda: wide(M=0), EINVAL),
    (lambda: wide(M=-1), EINVAL),
    (lambda: wide(M=9), ENOTSUP),
    (lambda: wide(M=8, K=16384 + 64), ENOTSUP),
    (lambda: wide(M=8, K=8192 + 64, bits=8), ENOTSUP),
    (lambda: wide(M=2, K=65536 + 64), ENOTSUP),
    (lambda: gather(P=0), EINVAL),
    (lambda: gather(R=0), EINVAL),
    (lambda: gather(E=0), EINVAL),
    (lambda: gather(lhs=NUL, R=3), EINVAL),
    (lambda: gather(rhs=NUL, E=3), EINVAL),
    (lambda: gather(lhs=ctypes.c_void_p(0x10002)), EINVAL),
    (lambda: gather(P=4097, R=4097, E=4), ENOTSUP),
    (lambda: gather(E=70000), ENOTSUP),
    (lambda: gather(K=16384 + 64), ENOTSUP),
    (lambda: qmm(M=0), EINVAL),
    (lambda: qmm(x=NUL), EINVAL),
    (lambda: qmm(y=NUL), EINVAL),
    (lambda: qmm(K=96), EINVAL),
    (lambda: qmm(bits=7), ENOTSUP),
    (lambda: qmm(gs=16, K=128), ENOTSUP),
    (lambda: qmm(gs=128, K=128), ENOTSUP),
    (lambda: qmm(gs=32, K=128), ENOTSUP),
    (lambda: gqmm(gs=32, K=128), ENOTSUP),
    (lambda: moe(gs=32), ENOTSUP),
    (lambda: lib.agq_quantize(A, 2, A, A, A, 4, 64, 4, 64, None), EINVAL),
    (lambda: lib.agq_quantize(A, 0, A, A, A, 4, 64, 7, 64, None), ENOTSUP),
    (lambda: lib.agq_quantize(A, 0, A, A, A, 4, 64, 4, 48, None), ENOTSUP),
    (lambda: lib.agq_quantize(A2, 0, A, A, A, 4, 64, 4, 64, None), EINVAL),
    (lambda: lib.agq_quantize(NUL, 0, A, A, A, 4, 64, 4, 64, None), EINVAL),
    (lambda: qmm(x=A2), EINVAL),
    (lambda: qmm(ws=A2, wsb=1 << 20), EINVAL),
    (lambda: qmm(M=1 << 20, K=1024), ENOTSUP),
    (lambda: fused(act=3), EINVAL),
    (lambda: fused(act=-1), EINVAL),
    (lambda: fused(act=1, N=15), EINVAL),
    (lambda: fused(act=2, res=A), EINVAL),
    (lambda: fused(eps=-1.0), EINVAL),
    (lambda: fused(eps=float("nan")), EINVAL),
    (lambda: fused(eps=float("inf")), EINVAL),
    (lambda: fused(g=A2), EINVAL),
    (lambda: fused(res=ctypes.c_void_p(0x10001)), EINVAL),
    (lambda: fused(x=NUL), EINVAL),
    (lambda: fused(y=NUL), EINVAL),
    (lambda: fused(bits=2), ENOTSUP),
    (lambda: fused(bits=3), ENOTSUP),
    (lambda: fused(K=65536 + 64), ENOTSUP),
    (lambda: fused(K=32768 + 64, bits=8), ENOTSUP),
    (lambda: fused(N=1 << 31), ENOTSUP),
    (lambda: nvfp4(x=NUL), EINVAL),
    (lambda: nvfp4(s=NUL), EINVAL),
    (lambda: nvfp4(M=0), EINVAL),
    (lambda: nvfp4(M=5), ENOTSUP),
    (lambda: nvfp4(K=24), EINVAL),
    (lambda: nvfp4(K=48), ENOTSUP),
    (lambda: nvfp4(ts=float("nan")), EINVAL),
    (lambda: nvfp4(ts=float("inf")), EINVAL),
    (lambda: nvfp4(s=ctypes.c_void_p(0x10001)), EINVAL),
    (lambda: nvfp4(x=A2), EINVAL),
    (lambda: nvfp4(K=114688 + 32), ENOTSUP),
    (lambda: nvfp4(M=4, K=32768 + 32), ENOTSUP),
    (lambda: nvfp4mm(x=NUL), EINVAL),
    (lambda: nvfp4mm(ws=A2, wsb=1 << 20), EINVAL),
    (lambda: nvfp4mm(s=NUL), EINVAL),
    (lambda: nvfp4mm(M=0), EINVAL),
    (lambda: nvfp4mm(M=3, K=48), ENOTSUP),
    (lambda: nvfp4mm(K=24), EINVAL),
    (lambda: nvfp4mm(K=48), ENOTSUP),
    (lambda: nvfp4mm(N=0), EINVAL),
    (lambda: nvfp4mm(ts=float("nan")), EINVAL),
    (lambda: nvfp4mm(s=ctypes.c_void_p(0x10001)), EINVAL),
    (lambda: nvfp4mm(x=A2), EINVAL),
    (lambda: nvfp4mm(M=1 << 20, K=1024), ENOTSUP),
    (lambda: gqmm(P=0), EINVAL),
    (lambda: gqmm(lhs=NUL, R=3), EINVAL),
    (lambda: gqmm(rhs=NUL, E=3), EINVAL),
    (lambda: gqmm(P=4097, R=4097, E=4), ENOTSUP),
    (lambda: gqmm(E=70000), ENOTSUP),
    (lambda: gqmm(R=1 << 20, K=1024), ENOTSUP),
    (lambda: moe(x=NUL), EINVAL),
    (lambda: moe(ws=NUL), EINVAL),
    (lambda: moe(T=0), EINVAL),
    (lambda: moe(k=0), EINVAL),
    (lambda: moe(H=96), EINVAL),
    (lambda: moe(bits=8), ENOTSUP),
    (lambda: moe(H=640), ENOTSUP),
    (lambda: moe(F=1088), ENOTSUP),
    (lambda: moe(T=257), ENOTSUP),
    (lambda: moe(T=256, k=17), ENOTSUP),
    (lambda: moe(wsb=4 * 4 * 2 * (1024 + 512) - 1), EINVAL),
    (lambda: moe(ws=ctypes.c_void_p(0x10008)), EINVAL),
    (lambda: moe(ex=ctypes.c_void_p(0x10002)), EINVAL),
    (lambda: lib.agq_dequantize(A, A, A, ctypes.c_void_p(0x10004), 4, 64, 4, 64, None), EINVAL),
    (lambda: lib.agq_dequantize(A, A, A, A, 4, 64, 7, 64, None), ENOTSUP),
])
def test_host_validation(call, status):
    assert call() == status
    assert lib.agq_last_error() != b""


def visited_rows(p, N):
    """Rows the kernels store, following the plan's row walk (host model of the kernel indexing)."""
    R, TG, RPG = p["rows_per_iter"], p["row_groups"], p["rows_per_group"]
    iters = RPG // R
    g = np.arange(TG)[:, None, None]
    it = np.arange(iters)[None, :, None]
    r = np.arange(R)[None, None, :]
    if p["row_order"] == 0:
        rows = (it * TG + g) * R + r
    else:
        rows = g * RPG + it * R + r
    rows = rows.reshape(-1)
    return rows[rows < N]


SHAPES = [  # (M, N, K, bits, experts)
    (1, 4096, 4096, 4, 0), (1, 6144, 4096, 4, 0), (1, 28672, 4096, 4, 0), (1, 4096, 14336, 4, 0),
    (1, 128256, 4096, 4, 0), (2, 14336, 4096, 4, 0), (4, 14336, 4096, 4, 0), (8, 14336, 4096, 4, 0),
    (2, 4096, 14336, 4, 0), (4, 4096, 14336, 4, 0), (8, 4096, 14336, 4, 0),
    (1, 4864, 896, 8, 0), (1, 896, 4864, 8, 0), (1, 1152, 896, 8, 0), (1, 151936, 896, 8, 0),
    (8, 14336, 4096, 4, 8), (8, 4096, 14336, 4, 8),
    (1, 1, 64, 4, 0), (3, 7, 192, 8, 0), (5, 33, 1088, 4, 0), (7, 100, 8192, 8, 0), (1, 5, 114688, 4, 0),
    (8, 3, 16384, 4, 0), (2, 9, 4096, 4, 3), (1, 2, 64, 8, 1),
]


@pytest.mark.parametrize("M,N,K,bits,experts", SHAPES)
@pytest.mark.parametrize("cus,wpc", [(256, 8), (256, 12), (304, 16), (8, 2), (256, 1)])
def test_plan_covers_the_problem(M, N, K, bits, experts, cus, wpc):
    p = agq.plan(M, N, K, bits, 64, cus, experts, waves_per_cu=wpc)
    C = K * bits // 128
    assert p["chunks_per_row"] == C
    R, TG, RPG = p["rows_per_iter"], p["row_groups"], p["rows_per_group"]
    assert TG == p["blocks"] * p["groups_per_block"]
    assert TG * RPG >= N                                                 # every row is covered
    assert (TG - p["groups_per_block"]) * RPG < N                        # at most one block's groups spare
    if N <= 300000:
        rows = visited_rows(p, N)
        assert rows.size == N and np.array_equal(np.sort(rows), np.arange(N))   # each row exactly once
    mfma = bits == 4 and K % 512 == 0 and (M >= 4 or experts > 0)
    stream = bits == 4 and M == 1 and not experts and -(-N // 16) >= 2 * cus
    assert p["engine"] == (2 if stream else 1 if mfma else 0)
    if stream:
        # The bit-stream kernel: blocks of 4 waves, each 4 consecutive rows staged two at a
        # time, x per 4096-column chunk in LDS.
        assert (R, RPG, p["groups_per_block"], p["threads_per_block"], p["row_order"]) == (4, 4, 4, 256, 1)
        assert p["blocks"] == -(-N // 16) and p["mw"] == 1 and p["cpt"] == 0 and p["stages"] == 2
        assert p["x_lds_bytes"] == 8192 and p["resident_waves"] == cus * wpc
        return
    if mfma:
        # Matrix cores: bands of 16 or 32 rows, up to 4 waves (2 for the gather) splitting
        # K into equal slices of whole 4-segment (512-column) blocks, one band group per block.
        assert R in (16, 32) and p["cpt"] == 0 and p["stages"] == 4
        S, smax = p["waves_per_group"], (2 if experts else 4)
        assert 1 <= S <= smax and (K // 512) % S == 0
        assert all((K // 512) % s for s in range(S + 1, smax + 1))           # the most waves that divide
        # Passes of 16 rows (the gather's pairs), operands from L2 (no LDS copy of x).
        assert p["mw"] == 16 and p["x_lds_bytes"] == 0
        assert p["groups_per_block"] == 1 and p["threads_per_block"] == 64 * S
        assert RPG % R == 0
        return
    assert 1 <= p["cpt"] <= 7 and p["cpt"] * p["mw"] <= 8
    assert 1 <= p["waves_per_group"] <= 8
    assert p["waves_per_group"] * p["cpt"] * 64 >= C                     # every chunk has a lane
    assert (p["waves_per_group"] - 1) * p["cpt"] * 64 < C                 # no wave is idle
    assert p["threads_per_block"] == 64 * p["waves_per_group"] * p["groups_per_block"] <= 512
    assert p["stages"] >= 1 and RPG % (p["stages"] * R) == 0              # whole turns of the load ring
    assert p["rows_per_iter"] * p["mw"] <= 16
    if experts:
        assert p["mw"] == 8 and p["cpt"] == 1   # passes of up to 8 pairs, one chunk per lane
    else:
        assert p["mw"] == M


# The VALU plans of several activation rows, probed with 8-bit codes at half the
# 4-bit K (the same chunks per row, so the same plan): 4-bit products with K a
# multiple of 512 and at least 5 rows, and 4-bit gathers, run on the matrix cores.
@pytest.mark.parametrize("M,K,experts,stages", [
    (2, 2048, 0, 4), (4, 1024, 0, 4), (8, 2048, 0, 4),   # one wave covers a row: four-stage ring
    (2, 4096, 0, 2), (2, 14336, 0, 2), (8, 4096, 0, 2), (4, 14336, 0, 2),  # K split over waves
    (1, 4096, 0, 2), (8, 2048, 3, 2), (8, 4096, 3, 2),   # batch 1 and the gather
])
def test_plan_ring_depth(M, K, experts, stages):
    bits, K = (4, K) if M == 1 and not experts else (8, K // 2)
    p = agq.plan(M, 4096, K, bits, 64, 256, experts, waves_per_cu=8)
    assert p["engine"] == 0
    assert p["stages"] == stages
    if M > 1 and not experts:
        assert (p["waves_per_group"] == 1) == (stages == 4)


@pytest.mark.parametrize("M,K,cpt,waves", [
    (2, 4096, 1, 2), (4, 4096, 1, 2), (2, 14336, 1, 7), (2, 16384, 1, 8),  # one chunk while 8 waves cover K
    (2, 32768, 4, 4), (2, 65536, 4, 8), (4, 32768, 2, 8), (3, 24576, 2, 6),  # past that, up to 8/M chunks
    (1, 14336, 4, 2), (1, 65536, 4, 8), (1, 114688, 7, 8),                   # batch 1: up to 4, then 7
])
def test_plan_chunks_per_lane(M, K, cpt, waves):
    bits, K = (4, K) if M == 1 else (8, K // 2)
    p = agq.plan(M, 4096, K, bits, 64, 256, 0, waves_per_cu=8)
    assert p["engine"] == 0
    assert (p["cpt"], p["waves_per_group"]) == (cpt, waves)


@pytest.mark.parametrize("K,bytes_", [(2048, 8 * 64 * 1 * 1 * 68), (4096, 8 * 64 * 1 * 2 * 68), (14336, 0)])
def test_gather_plan_lds_copy_of_x(K, bytes_):
    """Gather blocks whose row groups share columns (one or two K segments, four groups)
    stage each pass's x rows through one LDS copy; seven-segment groups do not."""
    p = agq.plan(8, 4096, K // 2, 8, 64, 256, 8, waves_per_cu=8)
    assert p["engine"] == 0 and p["x_lds_bytes"] == bytes_
    if bytes_:
        assert p["groups_per_block"] == 4 and p["threads_per_block"] == 256 * p["waves_per_group"]


def test_plain_c_client_builds_and_runs(tmp_path):
    """The header compiles as C99 with warnings as errors, a C program links against
    the library, and its host-only calls behave as from Python."""
    import shutil
    import subprocess
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    src = os.path.join(ROOT, "tests", "c", "abi_client.c")
    lib_dir = os.path.dirname(agq.LIB_PATH)
    exe = str(tmp_path / "abi_client")
    subprocess.run([cc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic", "-I", os.path.join(ROOT, "include"),
                    src, "-L", lib_dir, "-lagq", f"-Wl,-rpath,{lib_dir}", "-o", exe], check=True)
    out = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert out.returncode == 0, out.stdout + out.stderr
    assert "failures 0" in out.stdout
