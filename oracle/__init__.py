"""Python face of the CPU oracle (``agq_oracle.c``), loaded through ctypes.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package. The GPU library
never does.

The oracle is single-threaded C in float64. It unpacks the codes,
dequantizes ``w = scale*q + bias``, and takes dot products in increasing k.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "agq_oracle.c")
LIB = os.path.join(HERE, "libagq_oracle.so")

_CFLAGS = ["-O2", "-std=c99", "-fPIC", "-shared", "-ffp-contract=off", "-Wall", "-Wextra", "-Werror"]


def build(src: str = SRC, out: str = LIB, strict: bool = True) -> str:
    """Compile the oracle with gcc (plain -O2, no FMA contraction, no fast-math)."""
    flags = _CFLAGS if strict else [f for f in _CFLAGS if f != "-Werror"]
    cmd = ["gcc", *flags, src, "-o", out + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


_lib = None


def load(path: str | None = None):
    """Load the compiled oracle, building it first if missing or older than its source."""
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(path))
    if _lib is None:
        if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
            build()
        _lib = _bind(ctypes.CDLL(LIB))
    return _lib


def _bind(lib):
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    I = ctypes.c_int
    lib.agqo_unpack.argtypes = [P, I64, I64, I, P]
    lib.agqo_dequantize.argtypes = [P, P, P, I64, I64, I, I, P, P]
    lib.agqo_qmv.argtypes = [P, I64, P, P, P, I64, I64, I, I, P, I64, P, P]
    lib.agqo_gather_qmv.argtypes = [P, I64, P, P, P, I64, I64, I64, I, I, P, P, I64, P, I64, P, P]
    lib.agqo_moe_swiglu.argtypes = [P, I64, I64, I64, I64, I64, P, P, P, P, P, P, P, P, P, P, P, I, I, P, P]
    lib.agqo_quantize.argtypes = [P, I64, I64, I, I, P, P, P]
    lib.agqo_qmv_fused.argtypes = [P, P, ctypes.c_double, P, P, P, I64, I64, I, I, P, I, P, P]
    lib.agqo_qmv_nvfp4.argtypes = [P, I64, P, P, ctypes.c_double, I64, I64, P, I64, P, P]
    lib.agqo_e2m1.argtypes = [ctypes.c_uint32]
    lib.agqo_e2m1.restype = ctypes.c_double
    lib.agqo_e4m3.argtypes = [ctypes.c_uint32]
    lib.agqo_e4m3.restype = ctypes.c_double
    lib.agqo_bf16_round.argtypes = [ctypes.c_double]
    lib.agqo_bf16_round.restype = ctypes.c_double
    for f in (lib.agqo_unpack, lib.agqo_dequantize, lib.agqo_qmv, lib.agqo_gather_qmv, lib.agqo_moe_swiglu,
              lib.agqo_quantize, lib.agqo_qmv_fused):
        f.restype = I
    return lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


class OracleError(RuntimeError):
    pass


def _check(rc):
    if rc != 0:
        raise OracleError(f"oracle returned {rc}")


def unpack(w, K: int, bits: int, lib=None) -> np.ndarray:
    """Packed uint32 ``[N, K*bits/32]`` -> codes uint8 ``[N, K]``."""
    lib = lib or load()
    w = _c(w, np.uint32)
    w2 = w.reshape(-1, w.shape[-1])
    q = np.empty((w2.shape[0], K), dtype=np.uint8)
    _check(lib.agqo_unpack(_p(w2), w2.shape[0], K, bits, _p(q)))
    return q.reshape(w.shape[:-1] + (K,))


def dequantize(w, scales, biases, K: int, bits: int, group_size: int = 64, lib=None):
    """-> (float64 ``[N, K]`` weights, count of values not exact in binary32)."""
    lib = lib or load()
    w = _c(w, np.uint32)
    s = _c(scales, np.uint16)
    b = _c(biases, np.uint16)
    n = int(np.prod(w.shape[:-1]))
    out = np.empty((n, K), dtype=np.float64)
    bad = np.zeros(1, dtype=np.int64)
    _check(lib.agqo_dequantize(_p(w), _p(s), _p(b), n, K, bits, group_size, _p(out), _p(bad)))
    return out.reshape(w.shape[:-1] + (K,)), int(bad[0])


def qmv(x, w, scales, biases, K: int, bits: int, group_size: int = 64, rows=None, lib=None):
    """-> (y float64 ``[M, nrows]``, A float64 ``[M, nrows]``) with A = sum |x*w|."""
    lib = lib or load()
    x = _c(x, np.uint16).reshape(-1, K)
    w = _c(w, np.uint32)
    s = _c(scales, np.uint16)
    b = _c(biases, np.uint16)
    n = w.shape[0]
    r = None if rows is None else _c(rows, np.int64)
    nrows = n if r is None else r.shape[0]
    y = np.empty((x.shape[0], nrows), dtype=np.float64)
    a = np.empty_like(y)
    _check(lib.agqo_qmv(_p(x), x.shape[0], _p(w), _p(s), _p(b), n, K, bits, group_size,
                        _p(r), nrows, _p(y), _p(a)))
    return y, a


def qmv_nvfp4(x, w, scales, tensor_scale: float, K: int, rows=None, lib=None):
    """NVFP4 product: ``x`` [M, K] bf16 bits, ``w`` [N, K/8] uint32 (E2M1 codes low-first),
    ``scales`` [N, K/16] uint8 (E4M3) -> (y, A) float64 ``[M, nrows]``."""
    lib = lib or load()
    x = _c(x, np.uint16).reshape(-1, K)
    w = _c(w, np.uint32)
    s = _c(scales, np.uint8)
    n = w.shape[0]
    r = None if rows is None else _c(rows, np.int64)
    nrows = n if r is None else r.shape[0]
    y = np.empty((x.shape[0], nrows), dtype=np.float64)
    a = np.empty_like(y)
    _check(lib.agqo_qmv_nvfp4(_p(x), x.shape[0], _p(w), _p(s), float(tensor_scale), n, K, _p(r), nrows,
                              _p(y), _p(a)))
    return y, a


def gather_qmv(x, w, scales, biases, lhs, rhs, K: int, bits: int, group_size: int = 64,
               rows=None, P: int | None = None, lib=None):
    """Expert-gathered product. ``w`` is ``[E, N, K*bits/32]``; returns ``[P, nrows]`` y and A."""
    lib = lib or load()
    x = _c(x, np.uint16).reshape(-1, K)
    w = _c(w, np.uint32)
    s = _c(scales, np.uint16)
    b = _c(biases, np.uint16)
    e, n = w.shape[0], w.shape[1]
    lh = None if lhs is None else _c(lhs, np.uint32)
    rh = None if rhs is None else _c(rhs, np.uint32)
    if P is None:
        P = (lh if lh is not None else rh).shape[0]
    r = None if rows is None else _c(rows, np.int64)
    nrows = n if r is None else r.shape[0]
    y = np.empty((P, nrows), dtype=np.float64)
    a = np.empty_like(y)
    _check(lib.agqo_gather_qmv(_p(x), x.shape[0], _p(w), _p(s), _p(b), e, n, K, bits, group_size,
                               _p(lh), _p(rh), P, _p(r), nrows, _p(y), _p(a)))
    return y, a


def moe_swiglu(x, gate, up, down, experts, weights, bits: int, group_size: int = 64, lib=None):
    """Decode MoE layer with SwiGLU experts (float64, exact dequantization).

    ``x`` [T, H] bf16; ``gate``/``up``: dicts of ``w`` [E, F, H*bits/32], ``scales``/``biases``
    [E, F, H/64]; ``down``: ``w`` [E, H, F*bits/32], ``scales``/``biases`` [E, H, F/64];
    ``experts`` [T, k] uint32; ``weights`` [T, k] float32 router weights.
    Returns (y float64 [T, H], A float64 [T, H])."""
    lib = lib or load()
    x = _c(x, np.uint16)
    T, H = x.shape
    ex = _c(experts, np.uint32)
    r = _c(weights, np.float32)
    k = ex.shape[1]
    E, F = gate["w"].shape[0], gate["w"].shape[1]
    arrs = []
    for d in (gate, up, down):
        arrs += [_c(d["w"], np.uint32), _c(d["scales"], np.uint16), _c(d["biases"], np.uint16)]
    y = np.empty((T, H), dtype=np.float64)
    a = np.empty_like(y)
    _check(lib.agqo_moe_swiglu(_p(x), T, H, F, E, k, *[_p(v) for v in arrs], _p(ex), _p(r), bits, group_size,
                               _p(y), _p(a)))
    return y, a


def quantize(w, bits: int, group_size: int = 64, lib=None):
    """float32 ``[N, K]`` -> (packed uint32 ``[N, K*bits/32]``, scales bf16 ``[N, K/gs]``, biases bf16)."""
    lib = lib or load()
    w = _c(w, np.float32)
    N, K = w.shape
    wq = np.empty((N, K * bits // 32), dtype=np.uint32)
    s = np.empty((N, K // group_size), dtype=np.uint16)
    b = np.empty_like(s)
    _check(lib.agqo_quantize(_p(w), N, K, bits, group_size, _p(wq), _p(s), _p(b)))
    return wq, s, b


ACT_NONE, ACT_SWIGLU, ACT_GEGLU = 0, 1, 2


def qmv_fused(x, w, scales, biases, K: int, bits: int, group_size: int = 64, gamma=None, eps: float = 1e-5,
              residual=None, act: int = ACT_NONE, lib=None):
    """Batch-1 product with a fused RMS-norm prologue (``gamma``) and an epilogue (``residual``
    add, or SwiGLU / GeGLU over row-interleaved gate/up pairs). -> (y float64, A float64)."""
    lib = lib or load()
    x = _c(x, np.uint16).reshape(K)
    w = _c(w, np.uint32)
    s = _c(scales, np.uint16)
    b = _c(biases, np.uint16)
    N = w.shape[0]
    g = None if gamma is None else _c(gamma, np.uint16).reshape(K)
    r = None if residual is None else _c(residual, np.uint16).reshape(N)
    out = N if act == ACT_NONE else N // 2
    y = np.empty(out, dtype=np.float64)
    a = np.empty_like(y)
    _check(lib.agqo_qmv_fused(_p(x), _p(g), float(eps), _p(w), _p(s), _p(b), N, K, bits, group_size, _p(r), act,
                              _p(y), _p(a)))
    return y, a
