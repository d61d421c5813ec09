"""Helpers shared by the GPU tests: device transfer, the parity tolerance, progress lines."""
from __future__ import annotations

import sys

import numpy as np
import torch

REL_TOL = 2e-3   # |y_gpu - y_ref| <= 2e-3 * sum_k |x_k * w_k| per output element


def progress(msg: str):
    """Name the case on the real stdout before a GPU step (bypasses pytest capture)."""
    sys.__stdout__.write(f"[gpu] {msg}\n")
    sys.__stdout__.flush()


def bf16_dev(a: np.ndarray, device="cuda"):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint16).view(np.int16)).view(torch.bfloat16).to(device)


def u32_dev(a: np.ndarray, device="cuda"):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint32).view(np.int32)).to(device)


def bf16_host(t) -> np.ndarray:
    """bf16 tensor -> float64 numpy (exact)."""
    u = t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def bf16_bits_host(t) -> np.ndarray:
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def half_ulp_bf16(v: np.ndarray) -> np.ndarray:
    """Half a bfloat16 ulp at |v| (the bound of one RNE rounding to bf16)."""
    v = np.abs(np.asarray(v, dtype=np.float64))
    e = np.floor(np.log2(np.maximum(v, np.finfo(np.float32).tiny)))
    return np.ldexp(1.0, (e - 8).astype(int))


def check_close(y_gpu, y_ref, A, what: str, extra_half_ulp: bool = False):
    """Element-wise parity check; returns the worst |err|/A for reporting."""
    y = bf16_host(y_gpu).reshape(y_ref.shape) if isinstance(y_gpu, torch.Tensor) else y_gpu
    tol = REL_TOL * A
    if extra_half_ulp:
        tol = tol + half_ulp_bf16(y_ref)
    err = np.abs(y - y_ref)
    bad = ~(err <= tol)
    if bad.any():
        i = np.unravel_index(np.argmax(np.where(bad, err / np.maximum(tol, 1e-300), 0)), err.shape)
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} outside tolerance; worst at {i}: "
                             f"gpu={y[i]!r} ref={y_ref[i]!r} A={A[i]!r}")
    ratio = err / np.maximum(A, 1e-300)
    return float(ratio.max())
