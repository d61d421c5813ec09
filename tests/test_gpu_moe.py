"""GPU parity of the fused decode MoE layer (agq_moe_decode) against the CPU oracle.

Tolerance per output element: |y_gpu - y_ref| <= 2e-3 * A, with
A = sum_j |r_j| * sum_n |w_down[e_j][m, n] * h_j[n]| from the oracle (exact float64),
plus half a bf16 ulp of y_ref for the output rounding where |y| can approach A (small F).
The layer's intermediate h is carried at about 17 significant bits on the GPU, so the
budget is spent almost entirely on the final projection's fp32 accumulation.
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


def planes_dev(d):
    return u32_dev(d["w"]), bf16_dev(d["scales"]), bf16_dev(d["biases"])


def random_layer(seed, E, H, F, bits=4):
    mk = lambda t, n, k: [si.draw_quantized_weight(40 + seed, 100 * t + e, n, k, bits) for e in range(E)]  # noqa: E731
    out = []
    for t, (n, k) in enumerate(((F, H), (F, H), (H, F))):
        planes = mk(t, n, k)
        out.append({key: np.stack([p[key] for p in planes]) for key in ("w", "scales", "biases")})
    return out


def router(seed, T, E, k):
    g = np.random.default_rng([41, seed])
    ids = np.stack([g.choice(E, k, replace=False) for _ in range(T)]).astype(np.uint32)
    z = -np.sort(-g.standard_normal((T, k)), axis=1)
    w = np.exp(z - z[:, :1])
    return ids, (w / w.sum(axis=1, keepdims=True)).astype(np.float32)


def run(x, gate, up, down, ids, w, what, extra_half_ulp=False):
    progress(f"{what}: T={x.shape[0]} H={x.shape[1]} F={gate['w'].shape[1]} E={gate['w'].shape[0]} "
             f"k={ids.shape[1]}")
    y = agq.moe_decode(bf16_dev(x), planes_dev(gate), planes_dev(up), planes_dev(down), u32_dev(ids),
                       torch.as_tensor(w, device="cuda"))
    torch.cuda.synchronize()
    y_ref, A = oracle.moe_swiglu(x, gate, up, down, ids, w, 4)
    worst = check_close(y, y_ref, A, what, extra_half_ulp=extra_half_ulp)
    progress(f"{what}: ok, worst |err|/A = {worst:.3e}")
    return y


def test_moe_decode_mixtral_layer():
    """Mixtral-shaped decode layer: 16 tokens, top-2 of 8 experts, H 4096, F 14336 (gate
    planes = the gather workload's W1, down planes = its W2, its expert ids)."""
    moe = si.workload(4)
    lay = si.moe_layer()
    run(moe["x"], moe["w1"], lay["w3"], moe["w2"], moe["ids"], lay["weights"], "moe mixtral")


@pytest.mark.parametrize("T,k,E,H,F", [(7, 3, 6, 1024, 1536), (1, 1, 1, 512, 512), (33, 2, 5, 512, 2048),
                                       (4, 8, 8, 2048, 1024)])
def test_moe_decode_shapes(T, k, E, H, F):
    gate, up, down = random_layer(T, E, H, F)
    x = si.draw_activations(42, T, T, H)
    ids, w = router(T, T, E, k)
    run(x, gate, up, down, ids, w, f"moe T={T} k={k}", extra_half_ulp=F <= 1024)


def test_moe_decode_deterministic_and_invalid_expert():
    T, k, E, H, F = 6, 2, 4, 1024, 2048
    gate, up, down = random_layer(9, E, H, F)
    x = si.draw_activations(43, 1, T, H)
    ids, w = router(9, T, E, k)
    bad = ids.copy()
    bad[2, 1] = E + 5
    args = [planes_dev(gate), planes_dev(up), planes_dev(down)]
    xd, wd = bf16_dev(x), torch.as_tensor(w, device="cuda")
    progress("moe determinism and invalid expert")
    y1 = agq.moe_decode(xd, *args, u32_dev(ids), wd)
    y2 = agq.moe_decode(xd, *args, u32_dev(ids), wd)
    yb = agq.moe_decode(xd, *args, u32_dev(bad), wd)
    torch.cuda.synchronize()
    assert np.array_equal(bf16_bits_host(y1), bf16_bits_host(y2))
    yh = bf16_host(yb)
    assert np.all(np.isnan(yh[2]))
    ok = [t for t in range(T) if t != 2]
    assert np.array_equal(bf16_bits_host(yb)[ok], bf16_bits_host(y1)[ok])
    y_ref, A = oracle.moe_swiglu(x, gate, up, down, ids, w, 4)
    check_close(y1, y_ref, A, "moe determinism")


def test_moe_decode_matches_the_unfused_gathers():
    """The layer against its pieces on the GPU: gate and up through agq_gather_qmv, the
    SwiGLU in float32 torch, the down projection through agq_gather_qmv on bf16 h, and the
    weighted sum; both meet the tolerance against the oracle (the unfused path rounds h to
    bf16, so it is checked against a tolerance scaled for that: 2^-8 of sum |w h| more)."""
    T, k, E, H, F = 5, 2, 4, 1024, 1536
    gate, up, down = random_layer(11, E, H, F)
    x = si.draw_activations(44, 1, T, H)
    ids, w = router(11, T, E, k)
    xd = bf16_dev(x)
    rhs = u32_dev(ids.reshape(-1))
    lhs = u32_dev(np.repeat(np.arange(T, dtype=np.uint32), k))
    progress("moe vs unfused gathers")
    g = agq.gather_qmv(xd, *planes_dev(gate), rhs_indices=rhs, lhs_indices=lhs).float()
    u = agq.gather_qmv(xd, *planes_dev(up), rhs_indices=rhs, lhs_indices=lhs).float()
    h = (torch.nn.functional.silu(g) * u).to(torch.bfloat16)
    o = agq.gather_qmv(h, *planes_dev(down), rhs_indices=rhs).float()
    y_unfused = (o.view(T, k, H) * torch.as_tensor(w, device="cuda")[:, :, None]).sum(1)
    y = agq.moe_decode(xd, planes_dev(gate), planes_dev(up), planes_dev(down), u32_dev(ids),
                       torch.as_tensor(w, device="cuda"))
    torch.cuda.synchronize()
    y_ref, A = oracle.moe_swiglu(x, gate, up, down, ids, w, 4)
    check_close(y, y_ref, A, "fused", extra_half_ulp=True)
    err = np.abs(y_unfused.cpu().numpy().astype(np.float64) - y_ref)
    assert np.all(err <= 6e-3 * A + 1e-30), float(np.max(err / A))
