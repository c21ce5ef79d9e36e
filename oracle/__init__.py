"""fp64 CPU oracle for grouped-query attention (ctypes binding to gqa_oracle.c).

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the
benchmark's ``cpu_baseline`` leg are the only importers.  The library under
``prefill_split_gqa_amd`` never imports this package, and this package never
imports the library.

Inputs may be numpy arrays or CPU torch tensors of any floating dtype; they
are widened exactly to float64 before the C code sees them.  Outputs are
unrounded float64 numpy arrays.
"""

from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gqa_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libgqa_oracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile gqa_oracle.c with gcc into oracle/libgqa_oracle.so."""
    if not force and os.path.exists(_LIB_PATH) and os.path.getmtime(_LIB_PATH) >= os.path.getmtime(_SRC):
        return _LIB_PATH
    tmp = _LIB_PATH + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
           "-fPIC", "-shared", "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    build(force=False)
    lib = ctypes.CDLL(_LIB_PATH)
    dp = ctypes.POINTER(ctypes.c_double)
    lib.gqa_oracle_attend.argtypes = [dp, dp, dp, dp, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                      ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                      ctypes.POINTER(ctypes.c_int32), ctypes.c_int, ctypes.c_double,
                                      dp, ctypes.c_int]
    lib.gqa_oracle_attend.restype = ctypes.c_int
    lib.gqa_oracle_attend_ex.argtypes = [dp, dp, dp, dp, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                         ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                         ctypes.POINTER(ctypes.c_int32), ctypes.c_int, ctypes.c_double,
                                         ctypes.c_int, dp, dp, ctypes.c_int]
    lib.gqa_oracle_attend_ex.restype = ctypes.c_int
    lib.gqa_oracle_q4_unpack.argtypes = [ctypes.c_void_p, ctypes.c_long, ctypes.c_int, ctypes.c_void_p]
    lib.gqa_oracle_q4_unpack.restype = ctypes.c_int
    lib.gqa_oracle_q4_dequant.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                          ctypes.c_long, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    lib.gqa_oracle_q4_dequant.restype = ctypes.c_int
    lib.gqa_oracle_f16_to_f32.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_long]
    lib.gqa_oracle_f16_to_f32.restype = ctypes.c_int
    lib.gqa_oracle_max_threads.restype = ctypes.c_int
    lib.gqa_oracle_f32_to_f16.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_long]
    lib.gqa_oracle_f32_to_f16.restype = ctypes.c_int
    lib.gqa_oracle_q4_quantize.argtypes = [ctypes.c_void_p, ctypes.c_long, ctypes.c_int, ctypes.c_int,
                                           ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    lib.gqa_oracle_q4_quantize.restype = ctypes.c_int
    _lib = lib
    return lib


def max_threads() -> int:
    return int(_load().gqa_oracle_max_threads())


def _f64(x) -> np.ndarray:
    """Exact widening of a numpy array or CPU torch tensor to contiguous float64."""
    if hasattr(x, "detach"):  # torch tensor
        x = x.detach()
        if x.device.type != "cpu":
            raise ValueError("oracle inputs must live in host memory")
        import torch

        x = x.to(torch.float64).numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _u8(x) -> np.ndarray:
    if hasattr(x, "detach"):
        x = x.detach().cpu().numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.uint8))


def _f16bits(x) -> np.ndarray:
    if hasattr(x, "detach"):
        import torch

        x = x.detach().cpu().to(torch.float16).numpy()
    x = np.asarray(x)
    if x.dtype != np.float16:
        raise ValueError("scales/biases must be float16")
    return np.ascontiguousarray(x).view(np.uint16)


def attend(q, k, v, kv_lens=None, causal: bool = False, scale: Optional[float] = None,
           return_probs: bool = False, nthreads: int = 0, window: int = 0, sinks=None):
    """Grouped-query attention in fp64.

    q [B,Hq,Tq,D]; k, v [B,Hkv,s_cap,D]; kv_lens: None (= s_cap), an int, or a
    length-B sequence of valid key counts.  ``causal`` aligns the Tq queries
    to the end of each request's keys.  ``scale`` defaults to the float32
    value of 1/sqrt(D).  ``window`` (> 0) keeps only the last ``window`` keys
    up to each row's own position; ``sinks`` ([Hq] logits) join each softmax's
    normaliser without a value.  Returns O [B,Hq,Tq,D] (and the softmax
    weights [B,Hq,Tq,s_cap] when ``return_probs``).
    """
    q = _f64(q)
    k = _f64(k)
    v = _f64(v)
    if q.ndim != 4 or k.ndim != 4 or v.ndim != 4 or k.shape != v.shape:
        raise ValueError("expected q [B,Hq,Tq,D] and k, v [B,Hkv,S,D]")
    B, Hq, Tq, D = q.shape
    Bk, Hkv, s_cap, Dk = k.shape
    if Bk != B or Dk != D:
        raise ValueError("batch or head-dim mismatch")
    if kv_lens is None:
        lens = np.full(B, s_cap, dtype=np.int32)
    elif np.isscalar(kv_lens):
        lens = np.full(B, int(kv_lens), dtype=np.int32)
    else:
        lens = np.ascontiguousarray(np.asarray(kv_lens, dtype=np.int32).reshape(B))
    if scale is None:
        scale = float(np.float32(1.0) / np.sqrt(np.float32(D)))
    out = np.empty((B, Hq, Tq, D), dtype=np.float64)
    probs = np.empty((B, Hq, Tq, s_cap), dtype=np.float64) if return_probs else None
    dp = ctypes.POINTER(ctypes.c_double)
    sk = None
    if sinks is not None:
        sk = _f64(sinks).reshape(Hq)
    rc = _load().gqa_oracle_attend_ex(
        q.ctypes.data_as(dp), k.ctypes.data_as(dp), v.ctypes.data_as(dp), out.ctypes.data_as(dp),
        B, Hq, Hkv, Tq, D, s_cap, lens.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
        1 if causal else 0, float(scale), int(window), sk.ctypes.data_as(dp) if sk is not None else None,
        probs.ctypes.data_as(dp) if probs is not None else None, int(nthreads))
    if rc != 0:
        raise ValueError("gqa_oracle_attend rejected its arguments (code %d)" % rc)
    return (out, probs) if return_probs else out


def f16_to_f32(x) -> np.ndarray:
    bits = _f16bits(x)
    out = np.empty(bits.shape, dtype=np.float32)
    rc = _load().gqa_oracle_f16_to_f32(bits.ctypes.data, out.ctypes.data, bits.size)
    if rc != 0:
        raise ValueError("bad arguments")
    return out


def q4_unpack(packed) -> np.ndarray:
    """uint8 [..., D/2] -> uint8 codes [..., D]."""
    p = _u8(packed)
    D = p.shape[-1] * 2
    n_rows = p.size // max(p.shape[-1], 1)
    codes = np.empty(p.shape[:-1] + (D,), dtype=np.uint8)
    rc = _load().gqa_oracle_q4_unpack(p.ctypes.data, n_rows, D, codes.ctypes.data)
    if rc != 0:
        raise ValueError("bad arguments")
    return codes


def q4_dequant(packed, scales, biases, group: int) -> np.ndarray:
    """float32 [..., D] = scale*code + bias per group (one rounding)."""
    p = _u8(packed)
    s = _f16bits(scales)
    b = _f16bits(biases)
    D = p.shape[-1] * 2
    n_rows = p.size // max(p.shape[-1], 1)
    if s.shape != p.shape[:-1] + (D // group,) or b.shape != s.shape:
        raise ValueError("scales/biases must be [..., D/group]")
    out = np.empty(p.shape[:-1] + (D,), dtype=np.float32)
    rc = _load().gqa_oracle_q4_dequant(p.ctypes.data, s.ctypes.data, b.ctypes.data, n_rows, D,
                                       int(group), out.ctypes.data)
    if rc != 0:
        raise ValueError("bad arguments")
    return out


def q4_attend(q, k_codes, k_scales, k_biases, v_codes, v_scales, v_biases, group: int,
              kv_lens=None, scale: Optional[float] = None, nthreads: int = 0):
    """Decode attention over a 4-bit cache: dequantize K and V, then attend."""
    k = q4_dequant(k_codes, k_scales, k_biases, group)
    v = q4_dequant(v_codes, v_scales, v_biases, group)
    return attend(q, k, v, kv_lens=kv_lens, causal=False, scale=scale, nthreads=nthreads)


def f32_to_f16(x) -> np.ndarray:
    """float32 values -> float16 (round to nearest, ties to even), as bit patterns viewed as float16."""
    a = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    out = np.empty(a.shape, dtype=np.uint16)
    rc = _load().gqa_oracle_f32_to_f16(a.ctypes.data, out.ctypes.data, a.size)
    if rc != 0:
        raise ValueError("bad arguments")
    return out.view(np.float16)


def q4_quantize(x, group: int):
    """Min-max group-affine 4-bit encoding of x [..., D] (widened exactly to
    float32): (packed codes uint8 [..., D/2], scales f16 [..., D/group],
    biases f16 [..., D/group]).  See gqa_oracle_q4_quantize for the steps."""
    if hasattr(x, "detach"):
        import torch

        x = x.detach().cpu().to(torch.float32).numpy()
    a = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    D = a.shape[-1]
    n_rows = a.size // max(D, 1)
    packed = np.empty(a.shape[:-1] + (D // 2,), dtype=np.uint8)
    sc = np.empty(a.shape[:-1] + (D // group,), dtype=np.uint16)
    bi = np.empty(a.shape[:-1] + (D // group,), dtype=np.uint16)
    rc = _load().gqa_oracle_q4_quantize(a.ctypes.data, n_rows, D, int(group), packed.ctypes.data, sc.ctypes.data,
                                        bi.ctypes.data)
    if rc != 0:
        raise ValueError("bad arguments")
    return packed, sc.view(np.float16), bi.view(np.float16)


def kv_append(cache, new, kv_lens):
    """A preallocated cache after appending new rows: cache [B, H, s_cap, ...]
    (any dtype), new [B, H, T_new, ...].  Request b's rows go to positions
    p_b .. p_b + T_new - 1, p_b = kv_lens[b] clamped to [0, s_cap]; rows that
    would land at or past s_cap are dropped.  Returns (updated copy of cache,
    new lengths min(p_b + T_new, s_cap))."""
    c = np.array(cache, copy=True)
    n = np.asarray(new)
    s_cap = c.shape[2]
    t_new = n.shape[2]
    out_lens = np.empty(c.shape[0], dtype=np.int32)
    for b in range(c.shape[0]):
        p = min(max(int(kv_lens[b]), 0), s_cap)
        m = min(t_new, s_cap - p)
        c[b, :, p:p + m] = n[b, :, :m]
        out_lens[b] = p + m
    return c, out_lens


# ---------------------------------------------------------------------------
# 4-bit cache with a float16 residual window.
#
# The VeloxQuant posts ("What this means in practice"; Part 4's caveats)
# note that a production KIVI cache keeps the most recent tokens in float16
# and only older ones quantized, which their test cache lacked.  Reading
# taken here (block flush): with residual capacity R, a request of n tokens
# holds positions [0, n_q) in the 4-bit arrays, n_q = R * floor(n / R), and
# positions [n_q, n) as exact float16 rows in the residual buffer, position
# p at slot p - n_q.  An append that fills the residual quantizes its rows
# (and any new rows that age at once) as one block; every quantized row is
# encoded on its own, with q4_quantize.
# ---------------------------------------------------------------------------


def q4r_split(n: int, R: int):
    """(n_q, n_r): rows of an n-token request held 4-bit and held in float16."""
    if R < 1:
        raise ValueError("R must be positive")
    n_q = R * (int(n) // R)
    return n_q, int(n) - n_q


def kv_append_q4r(state, k_new, v_new, kv_lens, group: int, R: int):
    """Append float16 rows to a residual-window 4-bit cache.

    state: dict with k_codes, v_codes (uint8 [B, H, s_cap, D/2]), k_scales,
    k_biases, v_scales, v_biases (float16 [B, H, s_cap, D/group]) and k_res,
    v_res (float16 [B, H, R, D]).  k_new, v_new: float16 [B, H, T_new, D].
    Request b holds n = kv_lens[b] (clamped to [0, s_cap]) tokens; its new
    rows take positions n .. n + T_new - 1, and rows at or past s_cap are
    dropped.  Returns (updated copy of state, new lengths).

    The request's recent rows, positions [n_q(n), n'), are the residual's
    rows followed by the kept new rows; of those, positions [n_q(n), n_q(n'))
    are encoded into the 4-bit arrays and positions [n_q(n'), n') become the
    residual, from slot 0.  Other rows and slots are left as they were.
    """
    st = {key: np.array(val, copy=True) for key, val in state.items()}
    kn = np.asarray(k_new)
    vn = np.asarray(v_new)
    if kn.dtype != np.float16 or vn.dtype != np.float16:
        raise ValueError("new rows must be float16 (the residual's type)")
    s_cap = st["k_codes"].shape[2]
    if st["k_res"].shape[2] != R:
        raise ValueError("residual buffers must hold R rows")
    t_new = kn.shape[2]
    out_lens = np.empty(st["k_codes"].shape[0], dtype=np.int32)
    for b in range(st["k_codes"].shape[0]):
        n = min(max(int(kv_lens[b]), 0), s_cap)
        m = min(t_new, s_cap - n)
        n2 = n + m
        nq_old, nr_old = q4r_split(n, R)
        nq_new, _ = q4r_split(n2, R)
        for name, new in (("k", kn), ("v", vn)):
            recent = np.concatenate([st[name + "_res"][b, :, :nr_old], new[b, :, :m]], axis=1)
            aged = recent[:, :nq_new - nq_old]
            if aged.shape[1] > 0:
                codes, sc, bi = q4_quantize(aged.astype(np.float32), group)
                st[name + "_codes"][b, :, nq_old:nq_new] = codes
                st[name + "_scales"][b, :, nq_old:nq_new] = sc
                st[name + "_biases"][b, :, nq_old:nq_new] = bi
            keep = recent[:, nq_new - nq_old:]
            st[name + "_res"][b, :, :keep.shape[1]] = keep
        out_lens[b] = n2
    return st, out_lens


def q4r_view(state, kv_lens, group: int, R: int):
    """The values a residual-window 4-bit cache holds, in position order:
    float32 (K, V) [B, H, s_cap, D] with positions [0, n_q) dequantized
    (q4_dequant), positions [n_q, n) the residual's float16 rows widened, and
    zeros from n on."""
    kc = np.asarray(state["k_codes"])
    B, H, s_cap, half = kc.shape
    D = 2 * half
    out = []
    for name in ("k", "v"):
        x = np.zeros((B, H, s_cap, D), dtype=np.float32)
        for b in range(B):
            n = min(max(int(kv_lens[b]), 0), s_cap)
            n_q, n_r = q4r_split(n, R)
            if n_q > 0:
                x[b, :, :n_q] = q4_dequant(state[name + "_codes"][b, :, :n_q], state[name + "_scales"][b, :, :n_q],
                                           state[name + "_biases"][b, :, :n_q], group)
            x[b, :, n_q:n] = np.asarray(state[name + "_res"][b, :, :n_r], dtype=np.float32)
        out.append(x)
    return out[0], out[1]


def q4r_attend(q, state, kv_lens, group: int, R: int, causal: bool = False, scale: Optional[float] = None,
               nthreads: int = 0):
    """Attention over a residual-window 4-bit cache: its values in position
    order (q4r_view), then attend (decode: one query row; causal: a prefill
    chunk aligned to the end of each request's tokens)."""
    k, v = q4r_view(state, kv_lens, group, R)
    return attend(q, k, v, kv_lens=kv_lens, causal=causal, scale=scale, nthreads=nthreads)
