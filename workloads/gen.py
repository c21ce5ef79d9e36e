"""Seeded input generators.

Every tensor is drawn from ``numpy.random.default_rng(SeedSequence([cfg_id,
variant, layer, tensor_id]))`` as float32 standard normals and then cast,
round-to-nearest-even, to the storage dtype (torch's CPU casts).  Both the
oracle and the GPU library read the *cast* values, so the cast is part of the
input, not of either computation.

The 4-bit encoder builds the quantized KV cache that the quantized decode path
consumes.  Its choices (min-max range, rounding) only shape the inputs: the
oracle and the kernels both start from the produced codes, scales and biases.
"""

from __future__ import annotations

import numpy as np
import torch

TENSOR_ID = {"q": 0, "k": 1, "v": 2, "lens": 3}

_TORCH_DTYPES = {
    "f32": torch.float32,
    "bf16": torch.bfloat16,
    "f16": torch.float16,
}


def seed_sequence(cfg_id: int, variant: int, layer: int, tensor: str) -> np.random.SeedSequence:
    return np.random.SeedSequence([int(cfg_id), int(variant), int(layer), TENSOR_ID[tensor]])


def _rng(cfg_id: int, variant: int, layer: int, tensor: str) -> np.random.Generator:
    return np.random.default_rng(seed_sequence(cfg_id, variant, layer, tensor))


def normal(shape, dtype: str, cfg_id: int, variant: int, layer: int, tensor: str) -> torch.Tensor:
    """i.i.d. N(0,1) float32 draws cast to ``dtype``; returns a CPU tensor."""
    x = _rng(cfg_id, variant, layer, tensor).standard_normal(size=tuple(shape), dtype=np.float32)
    return torch.from_numpy(x).to(_TORCH_DTYPES[dtype])


def request_lengths(n: int, lo: int, hi: int, cfg_id: int, variant: int = 0) -> np.ndarray:
    """``n`` per-request KV lengths drawn uniformly from the integers [lo, hi]."""
    r = _rng(cfg_id, variant, 0, "lens")
    return r.integers(lo, hi, size=n, endpoint=True).astype(np.int32)


def q4_pack_codes(codes: np.ndarray) -> np.ndarray:
    """Pack 4-bit codes along the last axis: element 2j goes to the low nibble
    of byte j and element 2j+1 to its high nibble."""
    codes = np.asarray(codes, dtype=np.uint8)
    if codes.shape[-1] % 2:
        raise ValueError("last axis must be even")
    if codes.size and int(codes.max()) > 15:
        raise ValueError("codes must be < 16")
    lo = codes[..., 0::2]
    hi = codes[..., 1::2]
    return (lo | (hi << 4)).astype(np.uint8)


def q4_encode(x: np.ndarray, group: int):
    """Min-max group-affine 4-bit encoding of ``x`` along its last axis.

    Per group of ``group`` consecutive elements: scale = (max - min) / 15 and
    bias = min, both rounded to float16; code = clamp(rint((x - bias) / scale),
    0, 15) in float32 (code 0 where the scale rounds to zero).

    Returns ``(packed uint8 [..., D/2], scales f16 [..., D/group],
    biases f16 [..., D/group])``.
    """
    x = np.asarray(x, dtype=np.float32)
    d = x.shape[-1]
    if d % group or group % 2:
        raise ValueError("D must be a multiple of an even group size")
    xg = x.reshape(*x.shape[:-1], d // group, group)
    mn = xg.min(axis=-1)
    mx = xg.max(axis=-1)
    scale16 = ((mx - mn) / np.float32(15.0)).astype(np.float16)
    bias16 = mn.astype(np.float16)
    s32 = scale16.astype(np.float32)[..., None]
    b32 = bias16.astype(np.float32)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        c = np.rint((xg - b32) / s32)
    c = np.where(s32 == 0, 0.0, c)
    c = np.clip(c, 0, 15).astype(np.uint8).reshape(x.shape)
    return q4_pack_codes(c), scale16, bias16


def seam_planted(B: int, Hq: int, Hkv: int, D: int, Tq: int, Tk: int, dtype: str, seed: int,
                 tile: int = 64, gain: float = 3.0, s_cap=None):
    """Causal-prefill inputs whose every key-tile boundary is visible in the output.

    Q, K, V are seeded N(0,1) float32.  Then, for every request and KV head,
    each key j on either side of a boundary between ``tile``-key tiles (j a
    multiple of ``tile``, and j - 1) is replaced by ``gain`` times the query
    row of one (row, query head of the group) pair that can see it (row
    i >= j - (Tk - Tq)), drawn from the same generator.  At the usual scale
    1/sqrt(D) that key's score for that pair is about gain * sqrt(D) above
    the typical one, so its weight there is close to 1 and leaving the key
    out, or counting it twice, moves that output row by O(1).  Rows past Tk
    up to ``s_cap`` are NaN.  Returns CPU tensors (q, k, v) cast to ``dtype``
    and the sorted list of planted keys.
    """
    s_cap = Tk if s_cap is None else s_cap
    rng = np.random.default_rng(np.random.SeedSequence([97, int(seed), Tq, Tk]))
    q = rng.standard_normal((B, Hq, Tq, D), dtype=np.float32)
    k = rng.standard_normal((B, Hkv, Tk, D), dtype=np.float32)
    v = rng.standard_normal((B, Hkv, Tk, D), dtype=np.float32)
    off = Tk - Tq
    G = Hq // Hkv
    keys = sorted({j for t in range(1, (Tk + tile - 1) // tile) for j in (t * tile - 1, t * tile) if j < Tk})
    for b in range(B):
        for g in range(Hkv):
            for j in keys:
                lo = max(0, j - off)
                if lo >= Tq:
                    continue
                i = int(rng.integers(lo, Tq))
                h = g * G + int(rng.integers(0, G))
                k[b, g, j] = np.float32(gain) * q[b, h, i]
    if s_cap > Tk:
        pad = np.full((B, Hkv, s_cap - Tk, D), np.nan, np.float32)
        k = np.concatenate([k, pad], axis=2)
        v = np.concatenate([v, pad], axis=2)
    t = _TORCH_DTYPES[dtype]
    return torch.from_numpy(q).to(t), torch.from_numpy(k).to(t), torch.from_numpy(v).to(t), keys
