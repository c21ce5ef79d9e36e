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
