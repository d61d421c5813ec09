"""The allocation-free MoE entry point (agq_moe_decode_noalloc) through the C ABI.

It must give the same output bits as agq_moe_decode with a caller workspace (the same
kernels on the same inputs), meet the oracle's tolerance, and keep doing so on a second
call with a smaller input (the scratch array keeps the first call's contents). Sizes above
its scratch are rejected on the host.
"""
from __future__ import annotations

import ctypes

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

lib = agq.lib
P, I64, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
lib.agq_moe_decode_noalloc.argtypes = [P] * 13 + [I64] * 5 + [I, I, P]
lib.agq_moe_decode_noalloc.restype = I


def layer(seed, E, H, F):
    out = []
    for t, (n, k) in enumerate(((F, H), (F, H), (H, F))):
        planes = [si.draw_quantized_weight(60 + seed, 100 * t + e, n, k, 4) for e in range(E)]
        out.append({key: np.stack([p[key] for p in planes]) for key in ("w", "scales", "biases")})
    return out


def router(seed, T, E, k):
    g = np.random.default_rng([61, seed])
    ids = np.stack([g.choice(E, k, replace=False) for _ in range(T)]).astype(np.uint32)
    w = g.random((T, k)).astype(np.float32)
    return ids, (w / w.sum(axis=1, keepdims=True)).astype(np.float32)


def noalloc(x, dev_planes, ids, w, y, T, k, E, H, F):
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    ptrs = [t.data_ptr() for trio in dev_planes for t in trio]
    return lib.agq_moe_decode_noalloc(x.data_ptr(), *ptrs, ids.data_ptr(), w.data_ptr(), y.data_ptr(),
                                      T, k, E, H, F, 4, 64, st)


def test_noalloc_matches_the_workspace_call_twice():
    E, H, F = 4, 1024, 2048
    gate, up, down = layer(1, E, H, F)
    dev_planes = [(u32_dev(d["w"]), bf16_dev(d["scales"]), bf16_dev(d["biases"])) for d in (gate, up, down)]
    for T, k in ((12, 3), (5, 2)):  # the second call is smaller
        x = si.draw_activations(62, T, T, H)
        ids, w = router(T, T, E, k)
        xd, idd, wd = bf16_dev(x), u32_dev(ids), torch.as_tensor(w, device="cuda")
        progress(f"noalloc MoE T={T} k={k}")
        y_ref_gpu = agq.moe_decode(xd, *dev_planes, idd, wd)
        y = torch.full((T, H), float("nan"), dtype=torch.bfloat16, device="cuda")
        assert noalloc(xd, dev_planes, idd, wd, y, T, k, E, H, F) == 0, lib.agq_last_error()
        torch.cuda.synchronize()
        assert np.array_equal(bf16_bits_host(y), bf16_bits_host(y_ref_gpu))
        y_ref, A = oracle.moe_swiglu(x, gate, up, down, ids, w, 4)
        check_close(y, y_ref, A, f"noalloc T={T}", extra_half_ulp=True)


def test_noalloc_rejects_sizes_beyond_its_scratch():
    E, H, F = 2, 512, 14336 * 2
    z = torch.zeros(16, dtype=torch.int32, device="cuda")
    planes = [(z, z, z)] * 3
    T, k = 64, 2  # 4*T*k*(F + H) bytes = 14.9 MB > 8 MiB
    rc = noalloc(z, planes, z, z.float(), z, T, k, E, H, F)
    assert rc == agq.AGQ_ENOTSUP and b"scratch" in lib.agq_last_error()
