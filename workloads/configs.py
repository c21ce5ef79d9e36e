"""The five workloads, with the head geometries of the pages' models.

* decode_0p5b      -- single-token decode, Qwen2.5-0.5B heads (14 query / 2 KV,
                      head dim 64), KV length 128, fp32, one layer.
* decode_7b        -- single-token decode, Qwen2.5-7B heads (28 / 4, dim 128),
                      fp32, KV length swept 128..4096, 28 layers.
* prefill_0p5b     -- causal prefill, 0.5B heads, bf16, T in {513, 2049, 4097},
                      plus a 256-query chunk at offset 3841 into 4097 keys.
* batched_qwen3_4b -- batched decode, Qwen3-4B heads (32 / 8, dim 128), bf16,
                      B in {1, 2, 4, 8}, per-request lengths U{64..4096} in a
                      4096-row preallocated cache, 36 layers.
* q4_decode        -- decode over a 4-bit group-affine KV cache (groups of 64
                      along the head dim, f16 scale and bias), 64 / 8 heads,
                      dim 128, f16 queries, KV length 2048 or 16384, 80 layers.

The geometries come from "2x faster Qwen2 decode on Metal in Candle" (section
"Why It Matters: 7x KV Expansion", the two model bullets) and from the
VeloxQuant-MLX "attention" posts (Result 4: Qwen3-4B, 36 layers, 32 query and
8 KV heads).  All tensors are seeded N(0,1) stand-ins for the pages' real
prompts and weights.
"""

from __future__ import annotations

import dataclasses
from typing import Optional, Tuple

import numpy as np
import torch

from . import gen


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    cfg_id: int
    kind: str            # "decode" | "batched" | "prefill" | "q4"
    B: int
    Hq: int
    Hkv: int
    D: int
    dtype: str           # storage dtype of q/k/v (q only, for q4)
    layers: int
    sweep: Tuple[int, ...]   # S values (decode, q4), T values (prefill), B values (batched)
    s_cap: Optional[int] = None
    group: int = 64

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    def scale(self) -> float:
        """1/sqrt(D) as the float32 value the kernels receive."""
        return float(np.float32(1.0) / np.sqrt(np.float32(self.D)))


CONFIGS = {
    "decode_0p5b": Workload("decode_0p5b", 1, "decode", 1, 14, 2, 64, "f32", 1, (128,)),
    "decode_7b": Workload("decode_7b", 2, "decode", 1, 28, 4, 128, "f32", 28,
                          (128, 256, 512, 1024, 2048, 4096)),
    "prefill_0p5b": Workload("prefill_0p5b", 3, "prefill", 1, 14, 2, 64, "bf16", 1,
                             (513, 2049, 4097)),
    "batched_qwen3_4b": Workload("batched_qwen3_4b", 4, "batched", 8, 32, 8, 128, "bf16", 36,
                                 (1, 2, 4, 8), s_cap=4096),
    "q4_decode": Workload("q4_decode", 5, "q4", 1, 64, 8, 128, "f16", 80, (2048, 16384)),
}

# The chunked-prefill case: the last 256 queries of the T=4097 prompt.
PREFILL_CHUNK = {"Tq": 256, "Tk": 4097, "offset": 4097 - 256}

# Per-request lengths of the batched workload: one draw of 8 from U{64..4096};
# B uses the first B of them, so smaller batches are prefixes of larger ones.
BATCHED_LEN_RANGE = (64, 4096)


def by_name(name: str) -> Workload:
    return CONFIGS[name]


def decode_inputs(w: Workload, S: int, layer: int, s_cap: Optional[int] = None, B: Optional[int] = None):
    """q [B,Hq,1,D], k/v [B,Hkv,s_cap,D] (rows >= S filled with NaN when s_cap > S)."""
    B = w.B if B is None else B
    s_cap = S if s_cap is None else s_cap
    variant = w.sweep.index(S) if S in w.sweep else 1000 + S
    q = gen.normal((B, w.Hq, 1, w.D), w.dtype, w.cfg_id, variant, layer, "q")
    k = gen.normal((B, w.Hkv, S, w.D), w.dtype, w.cfg_id, variant, layer, "k")
    v = gen.normal((B, w.Hkv, S, w.D), w.dtype, w.cfg_id, variant, layer, "v")
    if s_cap > S:
        pad = torch.full((B, w.Hkv, s_cap - S, w.D), float("nan"), dtype=k.dtype)
        k = torch.cat([k, pad], dim=2)
        v = torch.cat([v, pad], dim=2)
    return q, k, v


def batched_lengths(w: Workload, B: int) -> np.ndarray:
    lens = gen.request_lengths(max(w.sweep), *BATCHED_LEN_RANGE, cfg_id=w.cfg_id)
    return lens[:B].copy()


def batched_inputs(w: Workload, B: int, layer: int):
    """q [B,Hq,1,D]; k/v [B,Hkv,s_cap,D] with rows >= kv_lens[b] NaN; kv_lens int32[B].

    Request b's tensors are seeded by (b, layer), so a request's data does not
    depend on the batch it sits in."""
    s_cap = w.s_cap
    lens = batched_lengths(w, B)
    qs, ks, vs = [], [], []
    for b in range(B):
        variant = b
        q = gen.normal((1, w.Hq, 1, w.D), w.dtype, w.cfg_id, variant, layer, "q")
        n = int(lens[b])
        k = gen.normal((1, w.Hkv, n, w.D), w.dtype, w.cfg_id, variant, layer, "k")
        v = gen.normal((1, w.Hkv, n, w.D), w.dtype, w.cfg_id, variant, layer, "v")
        pad = torch.full((1, w.Hkv, s_cap - n, w.D), float("nan"), dtype=k.dtype)
        qs.append(q)
        ks.append(torch.cat([k, pad], dim=2))
        vs.append(torch.cat([v, pad], dim=2))
    return torch.cat(qs), torch.cat(ks), torch.cat(vs), lens


def prefill_inputs(w: Workload, T: int, layer: int = 0):
    """q [1,Hq,T,D], k/v [1,Hkv,T,D]."""
    variant = w.sweep.index(T) if T in w.sweep else 1000 + T
    q = gen.normal((1, w.Hq, T, w.D), w.dtype, w.cfg_id, variant, layer, "q")
    k = gen.normal((1, w.Hkv, T, w.D), w.dtype, w.cfg_id, variant, layer, "k")
    v = gen.normal((1, w.Hkv, T, w.D), w.dtype, w.cfg_id, variant, layer, "v")
    return q, k, v


def q4_inputs(w: Workload, S: int, layer: int, s_cap: Optional[int] = None):
    """Quantized decode inputs: q f16 [1,Hq,1,D]; for K and for V: packed codes
    uint8 [1,Hkv,s_cap,D/2], scales and biases f16 [1,Hkv,s_cap,D/group]."""
    s_cap = S if s_cap is None else s_cap
    variant = w.sweep.index(S) if S in w.sweep else 1000 + S
    q = gen.normal((1, w.Hq, 1, w.D), "f16", w.cfg_id, variant, layer, "q")
    out = {"q": q}
    for name in ("k", "v"):
        x = gen.normal((1, w.Hkv, S, w.D), "f32", w.cfg_id, variant, layer, name).numpy()
        codes, scales, biases = gen.q4_encode(x, w.group)
        if s_cap > S:
            extra = s_cap - S
            codes = np.concatenate([codes, np.full((1, w.Hkv, extra, w.D // 2), 0xFF, np.uint8)], axis=2)
            nanf16 = np.full((1, w.Hkv, extra, w.D // w.group), np.nan, np.float16)
            scales = np.concatenate([scales, nanf16], axis=2)
            biases = np.concatenate([biases, nanf16], axis=2)
        out[name + "_codes"] = torch.from_numpy(np.ascontiguousarray(codes))
        out[name + "_scales"] = torch.from_numpy(np.ascontiguousarray(scales))
        out[name + "_biases"] = torch.from_numpy(np.ascontiguousarray(biases))
    return out
