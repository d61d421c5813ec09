"""Seeded synthetic inputs for affine group-quantized matrix-vector workloads.

This module is the producer side only. It draws float activations and
weights, rounds them to bfloat16, quantizes weights per 64-column group, and
packs the integer codes into uint32 words. It contains none of the
consumer-side arithmetic (unpacking codes, the affine map back to weights,
the dot product).

Both the CPU oracle (through the tests) and the GPU library consume its
arrays. Neither of them imports it.

Recipe (every draw is reproducible from the integers below):

* A stream is ``numpy.random.default_rng([0, cfg, t, c])`` (PCG64). ``cfg``
  is the workload number, ``t`` the tensor's ordinal within it, and ``c`` the
  1024-row chunk index. Chunks are independent, so they are drawn in
  parallel and the result does not depend on the thread count.
* Activations: ``standard_normal`` in float32, then bfloat16 by
  round-to-nearest-even.
* Weights: ``0.02 * standard_normal`` in float32.
* The quantizer takes, per (row, 64-column group), max and min in float32.
  It sets ``scale = (max - min) / (2**bits - 1)`` and ``bias = min``, both
  rounded to bfloat16 (RNE). Then ``q = clip(rint((w - bias) / scale), 0,
  2**bits - 1)``, computed in float32 with the rounded scale and bias. A
  group with ``max == min`` gets ``scale = 0`` and ``q = 0``.
* Packing: element ``k`` of a row occupies bits ``[bits*k, bits*k + bits)`` of
  the row's little-endian bit stream of uint32 words (low-first). For 2, 4 and
  8 bits that is bits ``[bits*(k % per), +bits)`` of word ``k // per``, with
  ``per = 32 // bits``; a 3-, 5- or 6-bit code may run into the next word.

Shapes follow the decode workloads: Llama-3-8B-class projections at 4 bits,
a 0.5B-class model at 8 bits, and a Mixtral-class 8-expert MoE layer.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

GROUP_SIZE = 64
CHUNK_ROWS = 1024

__all__ = [
    "GROUP_SIZE", "CHUNK_ROWS", "stream", "bf16_bits", "bf16_to_f32",
    "pack_codes", "quantize_rows", "draw_activations", "draw_quantized_weight",
    "random_codes", "workload", "WORKLOADS", "moe_expert_ids", "moe_prefill", "moe_layer", "decode_layer", "nvfp4_weight",
]


def _workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def stream(cfg: int, t: int, c: int = 0) -> np.random.Generator:
    """The PCG64 stream for workload ``cfg``, tensor ``t``, row chunk ``c``."""
    return np.random.default_rng([0, cfg, t, c])


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round-to-nearest-even."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    nan = (u & 0x7FFFFFFF) > 0x7F800000
    r = ((u + np.uint32(0x7FFF) + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    if nan.any():
        r[nan] = ((u[nan] >> 16) | 0x40).astype(np.uint16)
    return r


def bf16_to_f32(h: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> float32 (exact)."""
    return (np.asarray(h, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def pack_codes(q: np.ndarray, bits: int) -> np.ndarray:
    """Integer codes ``[..., K]`` (uint8) -> packed uint32 ``[..., K*bits/32]``, low-first: code k
    fills bits bits*k .. bits*k + bits - 1 of the row's little-endian bit stream (a 3-, 5- or
    6-bit code can run into the next word). Every 32 codes fill exactly ``bits`` words."""
    q = np.asarray(q, dtype=np.uint64)
    K = q.shape[-1]
    assert (K * bits) % 32 == 0 and 2 <= bits <= 8
    if K % 32:  # a partial chunk of 32 codes: pad with zero codes, keep the row's own words
        q = np.concatenate([q, np.zeros(q.shape[:-1] + (32 - K % 32,), np.uint64)], axis=-1)
    qs = q.reshape(q.shape[:-1] + (q.shape[-1] // 32, 32))
    out = np.zeros(qs.shape[:-1] + (bits,), dtype=np.uint64)
    for j in range(32):
        word, shift = divmod(bits * j, 32)
        v = qs[..., j] << np.uint64(shift)                 # up to 39 bits
        out[..., word] |= v & np.uint64(0xFFFFFFFF)
        if shift + bits > 32:
            out[..., word + 1] |= v >> np.uint64(32)
    return out.astype(np.uint32).reshape(q.shape[:-1] + (q.shape[-1] * bits // 32,))[..., :K * bits // 32]


def quantize_rows(w: np.ndarray, bits: int, group_size: int = GROUP_SIZE):
    """float32 ``[N, K]`` -> (codes uint8 ``[N, K]``, scale bf16 ``[N, G]``, bias bf16 ``[N, G]``)."""
    w = np.asarray(w, dtype=np.float32)
    n, k = w.shape
    assert k % group_size == 0
    wg = w.reshape(n, k // group_size, group_size)
    mx = wg.max(axis=-1)
    mn = wg.min(axis=-1)
    levels = np.float32(2 ** bits - 1)
    scale = (mx - mn) / levels
    s16 = bf16_bits(scale)
    b16 = bf16_bits(mn)
    sf = bf16_to_f32(s16)[..., None]
    bf = bf16_to_f32(b16)[..., None]
    num = wg - bf
    ratio = np.divide(num, sf, out=np.zeros_like(num), where=(sf != 0))
    q = np.clip(np.rint(ratio), 0, levels).astype(np.uint8)
    return q.reshape(n, k), s16, b16


def draw_activations(cfg: int, t: int, rows: int, k: int) -> np.ndarray:
    """bf16 bit patterns ``[rows, k]`` drawn from N(0, 1)."""
    out = np.empty((rows, k), dtype=np.uint16)
    for c in range(0, (rows + CHUNK_ROWS - 1) // CHUNK_ROWS):
        r0, r1 = c * CHUNK_ROWS, min(rows, (c + 1) * CHUNK_ROWS)
        out[r0:r1] = bf16_bits(stream(cfg, t, c).standard_normal((r1 - r0, k), dtype=np.float32))
    return out


def draw_quantized_weight(cfg: int, t: int, n: int, k: int, bits: int,
                          std: float = 0.02, keep_codes: bool = False):
    """A weight ``[n, k]`` ~ N(0, std), quantized and packed.

    Returns a dict with ``w`` (uint32 ``[n, k*bits/32]``), ``scales`` and
    ``biases`` (bf16 bits ``[n, k/64]``). With ``keep_codes`` it also returns
    ``codes`` (uint8 ``[n, k]``).
    """
    g = k // GROUP_SIZE
    wq = np.empty((n, k * bits // 32), dtype=np.uint32)
    s = np.empty((n, g), dtype=np.uint16)
    b = np.empty((n, g), dtype=np.uint16)
    codes = np.empty((n, k), dtype=np.uint8) if keep_codes else None
    nchunks = (n + CHUNK_ROWS - 1) // CHUNK_ROWS

    def one(c):
        r0, r1 = c * CHUNK_ROWS, min(n, (c + 1) * CHUNK_ROWS)
        wf = stream(cfg, t, c).standard_normal((r1 - r0, k), dtype=np.float32)
        wf *= np.float32(std)
        q, s16, b16 = quantize_rows(wf, bits)
        wq[r0:r1] = pack_codes(q, bits)
        s[r0:r1] = s16
        b[r0:r1] = b16
        if codes is not None:
            codes[r0:r1] = q

    if nchunks == 1:
        one(0)
    else:
        with ThreadPoolExecutor(_workers()) as ex:
            list(ex.map(one, range(nchunks)))
    out = {"w": wq, "scales": s, "biases": b}
    if codes is not None:
        out["codes"] = codes
    return out


def random_codes(seed, shape, bits: int) -> np.ndarray:
    """Uniform integer codes in ``[0, 2**bits)`` (for small structural cases)."""
    return np.random.default_rng(seed).integers(0, 2 ** bits, size=shape, dtype=np.uint8)


def moe_expert_ids(cfg: int, t: int, tokens: int, experts: int, top_k: int) -> np.ndarray:
    """Per token, ``top_k`` distinct expert ids drawn uniformly (slot order as drawn)."""
    g = stream(cfg, t, 0)
    return np.stack([g.choice(experts, top_k, replace=False) for _ in range(tokens)]).astype(np.uint32)


# Workload shapes: (name, N, K, bits) per weight, plus activation shapes.
WORKLOADS = {
    0: {"name": "qmv 4096x4096 4-bit gs64, batch 1",
        "x": [(0, "x", 1, 4096)],
        "w": [(1, "w", 4096, 4096, 4, "x")]},
    1: {"name": "Llama-3-8B-shaped decode GEMV set, batch 1, 4-bit gs64",
        "x": [(0, "x4096", 1, 4096), (1, "x14336", 1, 14336)],
        "w": [(2, "qkv", 6144, 4096, 4, "x4096"),
              (3, "o", 4096, 4096, 4, "x4096"),
              (4, "gate_up", 28672, 4096, 4, "x4096"),
              (5, "down", 4096, 14336, 4, "x14336"),
              (6, "lm_head", 128256, 4096, 4, "x4096")]},
    2: {"name": "qmv_wide, M in {2,4,8}, 4-bit gs64",
        "x": [(0, "x4096", 8, 4096), (1, "x14336", 8, 14336)],
        "w": [(2, "w_a", 14336, 4096, 4, "x4096"),
              (3, "w_b", 4096, 14336, 4, "x14336")]},
    3: {"name": "0.5B-class decode GEMVs, batch 1, 8-bit gs64",
        "x": [(0, "x896", 1, 896), (1, "x4864", 1, 4864)],
        "w": [(2, "gate_up", 4864, 896, 8, "x896"),
              (3, "down", 896, 4864, 8, "x4864"),
              (4, "qkv", 1152, 896, 8, "x896"),
              (5, "lm_head", 151936, 896, 8, "x896")]},
}

MOE = {"experts": 8, "tokens": 16, "top_k": 2, "hidden": 4096, "ffn": 14336, "bits": 4}


def moe_layer() -> dict:
    """The rest of a Mixtral-shaped decode MoE layer around workload 4: the up planes
    ``w3`` (8 x [14336, 4096], 4-bit gs64, streams t = 19..26, drawn like W1) and
    router weights ``weights`` [16, 2]: per token the softmax of 2 logits ~ N(0, 1)
    sorted in decreasing order (stream t = 27), float32. Workload 4's ``w1`` are the
    gate planes, ``w2`` the down planes and ``ids`` the experts."""
    m = MOE
    planes = [draw_quantized_weight(4, 19 + e, m["ffn"], m["hidden"], m["bits"]) for e in range(m["experts"])]
    w3 = {key: np.stack([p[key] for p in planes]) for key in planes[0]}
    w3.update(N=m["ffn"], K=m["hidden"], bits=m["bits"], E=m["experts"])
    z = -np.sort(-stream(4, 27).standard_normal((m["tokens"], m["top_k"])), axis=1)
    ez = np.exp(z - z[:, :1])
    return {"w3": w3, "weights": (ez / ez.sum(axis=1, keepdims=True)).astype(np.float32)}


def moe_prefill(tokens: int = 512) -> dict:
    """Routing and activations of a Mixtral-shaped MoE prefill (stream cfg 5): ``x``
    [tokens, 4096] ~ N(0,1) bf16, ``ids`` [tokens, 2] distinct experts per token,
    ``rhs`` = ids flattened (pair p = token*2 + slot) and ``lhs`` = the token of each
    pair. The expert planes are those of workload 4 (its ``w1``)."""
    m = MOE
    ids = moe_expert_ids(5, 1, tokens, m["experts"], m["top_k"])
    return {"x": draw_activations(5, 0, tokens, m["hidden"]), "ids": ids,
            "rhs": ids.reshape(-1).astype(np.uint32),
            "lhs": np.repeat(np.arange(tokens, dtype=np.uint32), m["top_k"])}


_E2M1_MID = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], np.float32)  # midpoints of 0, 0.5, 1, ..., 6


def nvfp4_weight(cfg: int, t: int, n: int, k: int, std: float = 0.02) -> dict:
    """A weight ``[n, k]`` ~ N(0, std) in NVFP4: ``tensor_scale`` = amax / (6 * 448) (fp32),
    one E4M3 byte per 16 columns (torch's float8_e4m3fn rounding of amax_block / 6 /
    tensor_scale), and the nearest E2M1 code of each w / (scale * tensor_scale) (ties to
    the smaller magnitude), packed 8 per uint32 low-first. Rows are drawn in 1024-row
    chunks (stream c). Returns ``w``, ``scales`` (uint8 ``[n, k/16]``) and ``tensor_scale``."""
    import torch
    parts = [(stream(cfg, t, c).standard_normal((min(CHUNK_ROWS, n - c * CHUNK_ROWS), k), dtype=np.float32)
              * np.float32(std)) for c in range((n + CHUNK_ROWS - 1) // CHUNK_ROWS)]
    amax = max(float(np.abs(p).max()) for p in parts)
    ts = np.float32(max(amax, 1e-30) / (6.0 * 448.0))
    wq = np.empty((n, k // 8), np.uint32)
    scales = np.empty((n, k // 16), np.uint8)
    for c, w in enumerate(parts):
        r0, r1 = c * CHUNK_ROWS, c * CHUNK_ROWS + w.shape[0]
        blk = np.abs(w.reshape(w.shape[0], k // 16, 16)).max(axis=2) / np.float32(6.0) / ts
        s8 = torch.from_numpy(blk.astype(np.float32)).to(torch.float8_e4m3fn)
        scales[r0:r1] = s8.view(torch.uint8).numpy()
        sval = s8.to(torch.float32).numpy()
        v = w.reshape(w.shape[0], k // 16, 16) / np.where(sval == 0, np.float32(1), sval)[..., None] / ts
        idx = np.searchsorted(_E2M1_MID, np.abs(v), side="left").astype(np.uint8)
        codes = (idx | ((v < 0).astype(np.uint8) << 3)).reshape(w.shape[0], k)
        wq[r0:r1] = pack_codes(codes, 4)
    return {"w": wq, "scales": scales, "tensor_scale": float(ts)}


def decode_layer() -> dict:
    """The non-weight tensors of a Llama-shaped decode layer around workload 1's
    projections (stream cfg 6): RMS-norm weights ``gamma_attn``, ``gamma_mlp`` and
    ``gamma_final`` [4096] drawn as 1 + 0.1 * N(0, 1) (t = 0, 1, 2) and a residual
    stream ``h`` [4096] ~ N(0, 1) (t = 3), all bf16, and ``eps`` = 1e-5. The
    gate/up weight of workload 1 (28672 rows) is read as 14336 interleaved gate
    and up row pairs."""
    out = {"eps": 1e-5}
    for t, name in enumerate(("gamma_attn", "gamma_mlp", "gamma_final")):
        out[name] = bf16_bits(np.float32(1) + np.float32(0.1) * stream(6, t).standard_normal(4096, dtype=np.float32))
    out["h"] = draw_activations(6, 3, 1, 4096)[0]
    return out


def workload(cfg: int, only=None, keep_codes: bool = False) -> dict:
    """All tensors of workload ``cfg`` (0-4) as numpy arrays.

    ``only`` restricts the weights to the listed names. Workload 4 (MoE) returns
    ``x`` [16,4096], ``ids`` [16,2], ``rhs``/``lhs1`` [32], ``h`` [32,14336],
    and per-matrix dicts ``w1``/``w2`` holding stacked expert planes.
    """
    if cfg in WORKLOADS:
        spec = WORKLOADS[cfg]
        out = {}
        for t, name, rows, k in spec["x"]:
            out[name] = draw_activations(cfg, t, rows, k)
        for t, name, n, k, bits, xname in spec["w"]:
            if only is not None and name not in only:
                continue
            d = draw_quantized_weight(cfg, t, n, k, bits, keep_codes=keep_codes)
            d.update(N=n, K=k, bits=bits, x=xname)
            out[name] = d
        return out
    if cfg == 4:
        m = MOE
        out = {"x": draw_activations(4, 0, m["tokens"], m["hidden"])}
        ids = moe_expert_ids(4, 1, m["tokens"], m["experts"], m["top_k"])
        out["ids"] = ids
        out["rhs"] = ids.reshape(-1).astype(np.uint32)
        out["lhs1"] = np.repeat(np.arange(m["tokens"], dtype=np.uint32), m["top_k"])
        for name, t0, n, k in (("w1", 2, m["ffn"], m["hidden"]), ("w2", 10, m["hidden"], m["ffn"])):
            if only is not None and name not in only:
                continue
            planes = [draw_quantized_weight(4, t0 + e, n, k, m["bits"], keep_codes=keep_codes)
                      for e in range(m["experts"])]
            d = {key: np.stack([p[key] for p in planes]) for key in planes[0]}
            d.update(N=n, K=k, bits=m["bits"], E=m["experts"])
            out[name] = d
        out["h"] = draw_activations(4, 18, m["tokens"] * m["top_k"], m["ffn"])
        return out
    raise ValueError(f"unknown workload {cfg}")
