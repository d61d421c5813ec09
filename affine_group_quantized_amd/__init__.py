"""Affine group-quantized matrix-vector products on AMD MI355X (gfx950).

Python binding of ``libagq.so`` (ctypes). This module only marshals
arguments. Every step of the computation runs in the library's HIP kernels,
and torch supplies device memory and the current stream. If the library is
not built, importing this module raises ``ImportError``; there is no
fallback path.

Operands follow the accelerator boundary of "MLX CUDA Cleanup Plan", Target
Architecture §1: BF16 activations, U32-packed affine codes (4 or 8 bits,
low-first in each word), and BF16 scales and biases per 64-column group.
Weight n, column k dequantizes to ``scales[n, k//64] * q[n, k] + biases[n, k//64]``.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = ["qmv", "qmv_wide", "qmv_fused", "qmv_nvfp4", "qmm_nvfp4", "ACT_NONE", "ACT_SWIGLU", "ACT_GEGLU", "gather_qmv", "qmm", "gather_qmm", "moe_decode", "moe_decode_workspace", "quantize",
           "dequantize", "plan", "launch_plan", "prepare_qmv", "AgqError",
           "LIB_PATH", "lib"]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libagq.so")

AGQ_OK, AGQ_EINVAL, AGQ_ENOTSUP, AGQ_EHIP = 0, 1, 2, 3


class AgqError(RuntimeError):
    """A non-OK status from libagq, carrying the library's message."""

    def __init__(self, status: int, message: str):
        super().__init__(f"{_STATUS.get(status, status)}: {message}")
        self.status = status


_STATUS = {AGQ_OK: "AGQ_OK", AGQ_EINVAL: "AGQ_EINVAL", AGQ_ENOTSUP: "AGQ_ENOTSUP", AGQ_EHIP: "AGQ_EHIP"}


class Plan(ctypes.Structure):
    _fields_ = [
        ("bits", ctypes.c_int32), ("chunks_per_row", ctypes.c_int32), ("cpt", ctypes.c_int32),
        ("mw", ctypes.c_int32), ("rows_per_iter", ctypes.c_int32), ("waves_per_group", ctypes.c_int32),
        ("groups_per_block", ctypes.c_int32), ("threads_per_block", ctypes.c_int32),
        ("rows_per_group", ctypes.c_int64), ("row_groups", ctypes.c_int64), ("blocks", ctypes.c_int64),
        ("row_order", ctypes.c_int32), ("x_lds_bytes", ctypes.c_int32), ("stages", ctypes.c_int32),
        ("resident_waves", ctypes.c_int32), ("engine", ctypes.c_int32),
    ]


def _load(path: str = LIB_PATH):
    if not os.path.exists(path):
        raise ImportError(f"libagq.so is not built ({path}); run __graft_entry__.build()")
    lib = ctypes.CDLL(path)
    P, I64, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    lib.agq_version.restype = I
    lib.agq_status_str.argtypes = [I]
    lib.agq_status_str.restype = ctypes.c_char_p
    lib.agq_last_error.restype = ctypes.c_char_p
    lib.agq_qmv.argtypes = [P, P, P, P, P, I64, I64, I, I, P]
    lib.agq_qmv_wide.argtypes = [P, P, P, P, P, I64, I64, I64, I, I, P]
    lib.agq_qmv_fused.argtypes = [P, P, ctypes.c_float, P, P, P, P, I, P, I64, I64, I, I, P]
    lib.agq_qmv_nvfp4.argtypes = [P, P, P, ctypes.c_float, P, I64, I64, I64, P]
    lib.agq_qmm_nvfp4.argtypes = [P, P, P, ctypes.c_float, P, I64, I64, I64, P, I64, P]
    lib.agq_qmm_nvfp4_workspace.argtypes = [I64, I64, I64]
    lib.agq_qmm_nvfp4_workspace.restype = I64
    lib.agq_gather_qmv.argtypes = [P, P, P, P, P, P, P, I64, I64, I64, I64, I64, I, I, P]
    lib.agq_qmm.argtypes = [P, P, P, P, P, I64, I64, I64, I, I, P, I64, P]
    lib.agq_qmm_workspace.argtypes = [I64, I64, I64, I, I]
    lib.agq_qmm_workspace.restype = I64
    lib.agq_gather_qmm.argtypes = [P, P, P, P, P, P, P, I64, I64, I64, I64, I64, I, I, P]
    lib.agq_moe_decode_workspace.argtypes = [I64, I64, I64, I64]
    lib.agq_moe_decode_workspace.restype = I64
    lib.agq_moe_decode.argtypes = [P] * 14 + [I64] * 6 + [I, I, P]
    lib.agq_moe_decode.restype = I
    lib.agq_quantize.argtypes = [P, I, P, P, P, I64, I64, I, I, P]
    lib.agq_quantize.restype = I
    lib.agq_dequantize.argtypes = [P, P, P, P, I64, I64, I, I, P]
    lib.agq_plan_product.argtypes = [I64, I64, I64, I, I, I, I, I64, ctypes.POINTER(Plan)]
    lib.agq_plan_launch.argtypes = [I64, I64, I64, I, I, I64, ctypes.POINTER(Plan)]
    for f in (lib.agq_qmv, lib.agq_qmv_wide, lib.agq_qmv_fused, lib.agq_qmv_nvfp4, lib.agq_qmm_nvfp4, lib.agq_gather_qmv, lib.agq_qmm, lib.agq_gather_qmm, lib.agq_dequantize,
              lib.agq_plan_product, lib.agq_plan_launch):
        f.restype = I
    return lib


lib = _load()


def _check(status: int):
    if status != AGQ_OK:
        raise AgqError(status, lib.agq_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need(t, name, dtypes, device):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}; expected one of {dtypes}")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}; expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


_BF16 = (torch.bfloat16,)
_U32 = (torch.int32, torch.uint32)


def _weights(w, scales, biases, K, bits, group_size, device, planes):
    _need(w, "w", _U32, device)
    _need(scales, "scales", _BF16, device)
    _need(biases, "biases", _BF16, device)
    if bits not in (2, 3, 4, 5, 6, 8) or group_size <= 0 or K % group_size or (K * bits) % 32:
        raise ValueError(f"bad format: K={K} bits={bits} group_size={group_size}")
    lead = w.shape[:-1]
    if w.dim() != planes + 1 or w.shape[-1] != K * bits // 32:
        raise ValueError(f"w has shape {tuple(w.shape)}; expected {planes + 1} dims ending in {K * bits // 32}")
    gshape = tuple(lead) + (K // group_size,)
    if tuple(scales.shape) != gshape or tuple(biases.shape) != gshape:
        raise ValueError(f"scales/biases must have shape {gshape}")
    return lead


def qmv(x, w, scales, biases, bits: int = 4, group_size: int = 64, out=None):
    """Batch-1 product: ``x`` [K] (or [1, K]) bf16 -> ``y`` [N] (or [1, N]) bf16."""
    device = x.device
    _need(x, "x", _BF16, device)
    K = x.shape[-1]
    if x.numel() != K:
        raise ValueError("qmv takes a single activation row; use qmv_wide for M > 1")
    (N,) = _weights(w, scales, biases, K, bits, group_size, device, 1)
    shape = tuple(x.shape[:-1]) + (N,)
    if out is None:
        out = torch.empty(shape, dtype=torch.bfloat16, device=device)
    else:
        _need(out, "out", _BF16, device)
        if out.numel() != N:
            raise ValueError("out has the wrong size")
    with torch.cuda.device(device):
        _check(lib.agq_qmv(_ptr(x), _ptr(w), _ptr(scales), _ptr(biases), _ptr(out), N, K, bits, group_size,
                           _stream(device)))
    return out


ACT_NONE, ACT_SWIGLU, ACT_GEGLU = 0, 1, 2


def qmv_fused(x, w, scales, biases, bits: int = 4, group_size: int = 64, norm_weight=None, eps: float = 1e-5,
              residual=None, act: int = ACT_NONE, out=None):
    """Batch-1 product with an RMS-norm prologue and a residual or GLU epilogue.

    ``x`` [K] bf16; ``norm_weight`` [K] bf16 or None (no norm); ``residual`` [N]
    bf16 or None (act 0 only; may be ``out`` itself). act 0 returns [N]; acts 1
    (SwiGLU) and 2 (GeGLU) take gate and up rows interleaved in ``w`` and
    return [N/2].
    """
    device = x.device
    _need(x, "x", _BF16, device)
    K = x.shape[-1]
    if x.numel() != K:
        raise ValueError("qmv_fused takes a single activation row")
    (N,) = _weights(w, scales, biases, K, bits, group_size, device, 1)
    if norm_weight is not None:
        _need(norm_weight, "norm_weight", _BF16, device)
        if norm_weight.numel() != K:
            raise ValueError("norm_weight must have K elements")
    if residual is not None:
        _need(residual, "residual", _BF16, device)
        if residual.numel() != N:
            raise ValueError("residual must have N elements")
    n_out = N if act == ACT_NONE else N // 2
    if out is None:
        out = torch.empty((n_out,), dtype=torch.bfloat16, device=device)
    else:
        _need(out, "out", _BF16, device)
        if out.numel() != n_out:
            raise ValueError("out has the wrong size")
    with torch.cuda.device(device):
        _check(lib.agq_qmv_fused(_ptr(x), _ptr(norm_weight), float(eps), _ptr(w), _ptr(scales), _ptr(biases),
                                 _ptr(residual), act, _ptr(out), N, K, bits, group_size, _stream(device)))
    return out


def _workspace(nbytes, workspace, device):
    """(pointer, bytes) of the GEMM workspace: ``workspace`` if given (a device uint8
    tensor), else a fresh one of ``nbytes`` when the call can use one, else none."""
    if workspace is False or (workspace is None and nbytes <= 0):
        return None, 0
    if workspace is None:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=device)
    _need(workspace, "workspace", (torch.uint8,), device)
    return workspace, workspace.numel()


def _nvfp4(fn, x, w, scales, tensor_scale, out, workspace=False):
    device = x.device
    _need(x, "x", _BF16, device)
    _need(w, "w", _U32, device)
    _need(scales, "scales", (torch.uint8,), device)
    K = x.shape[-1]
    M = x.numel() // K
    if w.dim() != 2 or w.shape[1] * 8 != K:
        raise ValueError(f"w has shape {tuple(w.shape)}; expected [N, {K // 8}]")
    N = w.shape[0]
    if tuple(scales.shape) != (N, K // 16):
        raise ValueError(f"scales must have shape {(N, K // 16)}")
    shape = tuple(x.shape[:-1]) + (N,)
    if out is None:
        out = torch.empty(shape, dtype=torch.bfloat16, device=device)
    else:
        _need(out, "out", _BF16, device)
        if out.numel() != M * N:
            raise ValueError("out has the wrong size")
    with torch.cuda.device(device):
        if fn is lib.agq_qmm_nvfp4:
            ws, nb = _workspace(lib.agq_qmm_nvfp4_workspace(M, N, K) if workspace is None else 0, workspace, device)
            _check(fn(_ptr(x), _ptr(w), _ptr(scales), float(tensor_scale), _ptr(out), M, N, K, _ptr(ws), nb,
                      _stream(device)))
        else:
            _check(fn(_ptr(x), _ptr(w), _ptr(scales), float(tensor_scale), _ptr(out), M, N, K, _stream(device)))
    return out


def qmv_nvfp4(x, w, scales, tensor_scale: float = 1.0, out=None):
    """NVFP4 product: ``x`` [K] or [M, K] bf16 (M <= 4), ``w`` [N, K/8] int32/uint32 E2M1 codes,
    ``scales`` [N, K/16] uint8 E4M3 block scales -> ``y`` [N] or [M, N] bf16."""
    return _nvfp4(lib.agq_qmv_nvfp4, x, w, scales, tensor_scale, out)


def qmm_nvfp4(x, w, scales, tensor_scale: float = 1.0, out=None, workspace=None):
    """NVFP4 product for any number of rows ``x`` [M, K] (agq_qmm_nvfp4: up to 4 rows the
    matvec kernel, beyond it the matrix-core GEMM, which needs K % 64 == 0). ``workspace``:
    None allocates the K split's scratch where the call can use one, a device uint8 tensor
    is used as given, False runs without a split."""
    return _nvfp4(lib.agq_qmm_nvfp4, x, w, scales, tensor_scale, out, workspace)


def prepare_qmv(x, w, scales, biases, out, bits: int = 4, group_size: int = 64, stream=None):
    """Validate once and return a zero-argument callable that queues the product.

    For hot loops (decode steps, benchmarks), each call is one C call with
    cached pointers, so per-call host overhead stays well below the kernel
    time. ``x`` is ``[K]`` or ``[M, K]`` (M <= 8), and ``out`` is the matching
    ``[N]`` / ``[M, N]`` bf16 buffer. The tensors must outlive the callable.
    Work is queued on ``stream``, or on the current stream at preparation time.
    """
    device = x.device
    _need(x, "x", _BF16, device)
    _need(out, "out", _BF16, device)
    K = x.shape[-1]
    M = x.numel() // K
    (N,) = _weights(w, scales, biases, K, bits, group_size, device, 1)
    if out.numel() != M * N:
        raise ValueError("out has the wrong size")
    st = ctypes.c_void_p((stream or torch.cuda.current_stream(device)).cuda_stream)
    args = (_ptr(x), _ptr(w), _ptr(scales), _ptr(biases), _ptr(out))
    fn = lib.agq_qmv_wide

    def call():
        status = fn(*args, M, N, K, bits, group_size, st)
        if status:
            _check(status)
    return call


def qmv_wide(x, w, scales, biases, bits: int = 4, group_size: int = 64, out=None):
    """Small-batch product: ``x`` [M, K] bf16 (1 <= M <= 8) -> ``y`` [M, N] bf16."""
    device = x.device
    _need(x, "x", _BF16, device)
    if x.dim() != 2:
        raise ValueError("x must be [M, K]")
    M, K = x.shape
    (N,) = _weights(w, scales, biases, K, bits, group_size, device, 1)
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=device)
    else:
        _need(out, "out", _BF16, device)
        if tuple(out.shape) != (M, N):
            raise ValueError("out has the wrong shape")
    with torch.cuda.device(device):
        _check(lib.agq_qmv_wide(_ptr(x), _ptr(w), _ptr(scales), _ptr(biases), _ptr(out), M, N, K, bits,
                                group_size, _stream(device)))
    return out


def qmm(x, w, scales, biases, bits: int = 4, group_size: int = 64, out=None, workspace=None):
    """Quantized matrix-matrix product: ``x`` [M, K] bf16 (any M) -> ``y`` [M, N] bf16.
    ``workspace``: None allocates the K split's scratch where the call can use one, a device
    uint8 tensor is used as given, False runs without a split."""
    device = x.device
    _need(x, "x", _BF16, device)
    if x.dim() != 2:
        raise ValueError("x must be [M, K]")
    M, K = x.shape
    (N,) = _weights(w, scales, biases, K, bits, group_size, device, 1)
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=device)
    else:
        _need(out, "out", _BF16, device)
        if tuple(out.shape) != (M, N):
            raise ValueError("out has the wrong shape")
    with torch.cuda.device(device):
        need = lib.agq_qmm_workspace(M, N, K, bits, group_size) if workspace is None else 0
        ws, nb = _workspace(need, workspace, device)
        _check(lib.agq_qmm(_ptr(x), _ptr(w), _ptr(scales), _ptr(biases), _ptr(out), M, N, K, bits, group_size,
                           _ptr(ws), nb, _stream(device)))
    return out


def gather_qmm(x, w, scales, biases, rhs_indices=None, lhs_indices=None, bits: int = 4, group_size: int = 64,
               out=None, num_pairs: int | None = None):
    """Expert-gathered matrix-matrix product (MoE prefill); arguments and result as
    :func:`gather_qmv`, for any number of pairs per expert."""
    return gather_qmv(x, w, scales, biases, rhs_indices, lhs_indices, bits, group_size, out, num_pairs,
                      _fn="agq_gather_qmm")


def gather_qmv(x, w, scales, biases, rhs_indices=None, lhs_indices=None, bits: int = 4, group_size: int = 64,
               out=None, num_pairs: int | None = None, _fn: str = "agq_gather_qmv"):
    """Expert-gathered product, one output row per (token, expert) pair.

    ``x`` [R, K] bf16; ``w`` [E, N, K*bits/32]; ``scales``/``biases`` [E, N, K/64];
    ``rhs_indices`` [P] expert per pair; ``lhs_indices`` [P] row of ``x`` per pair.
    A missing index array is the identity. Returns ``y`` [P, N] bf16.
    """
    device = x.device
    _need(x, "x", _BF16, device)
    if x.dim() != 2:
        raise ValueError("x must be [R, K]")
    R, K = x.shape
    E, N = _weights(w, scales, biases, K, bits, group_size, device, 2)
    for name, t in (("lhs_indices", lhs_indices), ("rhs_indices", rhs_indices)):
        if t is not None:
            _need(t, name, _U32, device)
            if t.dim() != 1:
                raise ValueError(f"{name} must be 1-D")
    if num_pairs is None:
        idx = rhs_indices if rhs_indices is not None else lhs_indices
        num_pairs = idx.shape[0] if idx is not None else R
    P = int(num_pairs)
    for t in (lhs_indices, rhs_indices):
        if t is not None and t.shape[0] != P:
            raise ValueError("index arrays must have P entries")
    if out is None:
        out = torch.empty((P, N), dtype=torch.bfloat16, device=device)
    else:
        _need(out, "out", _BF16, device)
        if tuple(out.shape) != (P, N):
            raise ValueError("out has the wrong shape")
    with torch.cuda.device(device):
        _check(getattr(lib, _fn)(_ptr(x), _ptr(w), _ptr(scales), _ptr(biases), _ptr(lhs_indices),
                                 _ptr(rhs_indices), _ptr(out), P, R, E, N, K, bits, group_size, _stream(device)))
    return out


def moe_decode_workspace(T: int, k: int, H: int, F: int) -> int:
    """Bytes of device workspace agq_moe_decode needs for T tokens, k experts each, width H, F units."""
    return int(lib.agq_moe_decode_workspace(T, k, H, F))


def moe_decode(x, gate, up, down, experts, weights, bits: int = 4, group_size: int = 64, out=None, workspace=None):
    """Fused decode MoE layer with SwiGLU experts.

    ``x`` [T, H] bf16; ``gate``/``up``: (w [E, F, H*bits/32], scales, biases [E, F, H/64]);
    ``down``: (w [E, H, F*bits/32], scales, biases [E, H, F/64]); ``experts`` [T, k] int32/uint32;
    ``weights`` [T, k] float32. Returns ``y`` [T, H] bf16. ``workspace`` (uint8, at least
    :func:`moe_decode_workspace` bytes) is allocated here when not given.
    """
    device = x.device
    _need(x, "x", _BF16, device)
    if x.dim() != 2:
        raise ValueError("x must be [T, H]")
    T, H = x.shape
    E, F = _weights(*gate, H, bits, group_size, device, 2)
    if tuple(_weights(*up, H, bits, group_size, device, 2)) != (E, F):
        raise ValueError("gate and up planes must have the same shape")
    if tuple(_weights(*down, F, bits, group_size, device, 2)) != (E, H):
        raise ValueError(f"down planes must be [{E}, {H}, .]")
    _need(experts, "experts", _U32, device)
    _need(weights, "weights", (torch.float32,), device)
    if experts.dim() != 2 or experts.shape[0] != T or tuple(weights.shape) != tuple(experts.shape):
        raise ValueError("experts and weights must be [T, k]")
    k = experts.shape[1]
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=device)
    else:
        _need(out, "out", _BF16, device)
        if tuple(out.shape) != (T, H):
            raise ValueError("out has the wrong shape")
    need = moe_decode_workspace(T, k, H, F)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=device)
    else:
        _need(workspace, "workspace", (torch.uint8,), device)
    with torch.cuda.device(device):
        _check(lib.agq_moe_decode(_ptr(x), *[_ptr(t) for t in gate], *[_ptr(t) for t in up],
                                  *[_ptr(t) for t in down], _ptr(experts), _ptr(weights), _ptr(out), _ptr(workspace),
                                  workspace.numel(), T, k, E, H, F, bits, group_size, _stream(device)))
    return out


def quantize(w, bits: int = 4, group_size: int = 64):
    """Affine group quantization on the device: ``w`` [..., K] float32 or bf16 ->
    (codes int32 [..., K*bits/32], scales bf16 [..., K/group_size], biases bf16)."""
    device = w.device
    _need(w, "w", (torch.float32, torch.bfloat16), device)
    K = w.shape[-1]
    lead = tuple(w.shape[:-1])
    rows = w.numel() // K
    codes = torch.empty(lead + (K * bits // 32,), dtype=torch.int32, device=device)
    scales = torch.empty(lead + (K // group_size,), dtype=torch.bfloat16, device=device)
    biases = torch.empty_like(scales)
    with torch.cuda.device(device):
        _check(lib.agq_quantize(_ptr(w), 0 if w.dtype == torch.float32 else 1, _ptr(codes), _ptr(scales),
                                _ptr(biases), rows, K, bits, group_size, _stream(device)))
    return codes, scales, biases


def dequantize(w, scales, biases, bits: int = 4, group_size: int = 64, out=None):
    """Dequantized fp32 weights, shape ``w.shape[:-1] + (K,)``."""
    device = w.device
    K = w.shape[-1] * 32 // bits
    lead = _weights(w, scales, biases, K, bits, group_size, device, w.dim() - 1)
    rows = 1
    for d in lead:
        rows *= d
    if out is None:
        out = torch.empty(tuple(lead) + (K,), dtype=torch.float32, device=device)
    else:
        _need(out, "out", (torch.float32,), device)
        if out.numel() != rows * K:
            raise ValueError("out has the wrong size")
    with torch.cuda.device(device):
        _check(lib.agq_dequantize(_ptr(w), _ptr(scales), _ptr(biases), _ptr(out), rows, K, bits, group_size,
                                  _stream(device)))
    return out


def plan(M: int, N: int, K: int, bits: int = 4, group_size: int = 64, num_cus: int = 256, experts: int = 0,
         waves_per_cu: int = 8):
    """The library's launch plan for a product of this shape (host only).

    ``waves_per_cu`` is the kernel's residency; the product calls take it from
    the HIP occupancy query, so their grids can differ from this estimate.
    """
    p = Plan()
    _check(lib.agq_plan_product(M, N, K, bits, group_size, num_cus, waves_per_cu, experts, ctypes.byref(p)))
    return {name: getattr(p, name) for name, _ in Plan._fields_}


def launch_plan(M: int, N: int, K: int, bits: int = 4, group_size: int = 64, experts: int = 0):
    """The plan the product calls launch on the current device (queries HIP occupancy)."""
    p = Plan()
    _check(lib.agq_plan_launch(M, N, K, bits, group_size, experts, ctypes.byref(p)))
    return {name: getattr(p, name) for name, _ in Plan._fields_}
