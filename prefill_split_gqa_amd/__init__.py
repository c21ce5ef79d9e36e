"""Python binding of libgqa.so (fused grouped-query attention for MI355X).

The functions carry the C entry points' names and only marshal arguments:
they read sizes from tensor shapes, check devices and dtypes, and pass
``data_ptr()`` values and torch's current HIP stream to the library.  Every
step of the attention runs in the library's kernels; there is no fallback
path, and a missing ``libgqa.so`` raises :class:`GqaError`.

PyTorch supplies device memory and streams only.
"""

from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgqa.so")

(GQA_OK, GQA_ERR_NULL, GQA_ERR_SHAPE, GQA_ERR_UNSUPPORTED, GQA_ERR_WORKSPACE, GQA_ERR_HIP, GQA_ERR_ALIGN,
 GQA_ERR_SCRATCH) = range(8)
GQA_F32, GQA_BF16, GQA_F16 = 0, 1, 2
_DTYPE_CODE = {torch.float32: GQA_F32, torch.bfloat16: GQA_BF16, torch.float16: GQA_F16}

EXPORTED = (
    "gqa_abi_version",
    "gqa_status_string",
    "gqa_decode_workspace_bytes",
    "gqa_prefill_workspace_bytes",
    "gqa_workspace_init",
    "gqa_decode_attend",
    "gqa_decode_attend_noalloc",
    "gqa_decode_attend_batched",
    "gqa_decode_attend_ex",
    "gqa_prefill_workspace_bytes_ex",
    "gqa_prefill_causal_ex",
    "gqa_prefill_causal",
    "gqa_decode_attend_q4",
    "gqa_dequant_q4",
    "gqa_kv_append",
    "gqa_kv_append_q4",
    "gqa_decode_q4r_workspace_bytes",
    "gqa_decode_attend_q4r",
    "gqa_kv_append_q4r",
    "gqa_prefill_causal_q4r",
    "gqa_read_probe",
)


class GqaError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__("%s failed: %s (status %d)" % (what, status_string(status) if _lib else "?", status))


_lib: Optional[ctypes.CDLL] = None


def load() -> ctypes.CDLL:
    """Load libgqa.so once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise GqaError(-1, "loading %s (not built: run python -m prefill_split_gqa_amd.build)" % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.gqa_abi_version.restype = i
    lib.gqa_status_string.argtypes = [i]
    lib.gqa_status_string.restype = ctypes.c_char_p
    lib.gqa_decode_workspace_bytes.argtypes = [i, i, i, i, i]
    lib.gqa_decode_workspace_bytes.restype = sz
    lib.gqa_prefill_workspace_bytes.argtypes = [i, i, i, i, i, i]
    lib.gqa_prefill_workspace_bytes.restype = sz
    lib.gqa_workspace_init.argtypes = [vp, sz, vp]
    lib.gqa_workspace_init.restype = i
    lib.gqa_decode_attend.argtypes = [vp, vp, vp, vp, i, i, i, i, i, i, f, i, vp, sz, vp]
    lib.gqa_decode_attend.restype = i
    lib.gqa_decode_attend_noalloc.argtypes = [vp, vp, vp, vp, i, i, i, i, i, i, f, i, vp]
    lib.gqa_decode_attend_noalloc.restype = i
    lib.gqa_decode_attend_batched.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp, sz, vp]
    lib.gqa_decode_attend_batched.restype = i
    lib.gqa_prefill_causal.argtypes = [vp, vp, vp, vp, i, i, i, i, i, i, i, f, i, vp, sz, vp]
    lib.gqa_prefill_causal.restype = i
    lib.gqa_decode_attend_ex.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, i, i, vp, vp, sz, vp]
    lib.gqa_decode_attend_ex.restype = i
    lib.gqa_prefill_workspace_bytes_ex.argtypes = [i, i, i, i, i, i, i]
    lib.gqa_prefill_workspace_bytes_ex.restype = sz
    lib.gqa_prefill_causal_ex.argtypes = [vp, vp, vp, vp, i, i, i, i, i, i, i, f, i, i, vp, vp, sz, vp]
    lib.gqa_prefill_causal_ex.restype = i
    lib.gqa_decode_attend_q4.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, f, vp, sz, vp]
    lib.gqa_decode_attend_q4.restype = i
    lib.gqa_dequant_q4.argtypes = [vp, vp, vp, vp, i, i, i, vp]
    lib.gqa_dequant_q4.restype = i
    lib.gqa_kv_append.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, vp]
    lib.gqa_kv_append.restype = i
    lib.gqa_kv_append_q4.argtypes = [vp, vp, i, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, vp]
    lib.gqa_kv_append_q4.restype = i
    lib.gqa_decode_q4r_workspace_bytes.argtypes = [i, i, i, i, i, i]
    lib.gqa_decode_q4r_workspace_bytes.restype = sz
    lib.gqa_decode_attend_q4r.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, f, vp, sz,
                                          vp]
    lib.gqa_decode_attend_q4r.restype = i
    lib.gqa_kv_append_q4r.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, vp]
    lib.gqa_kv_append_q4r.restype = i
    lib.gqa_prefill_causal_q4r.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, i, i, f, vp,
                                           sz, vp]
    lib.gqa_prefill_causal_q4r.restype = i
    lib.gqa_read_probe.argtypes = [vp, sz, vp, vp]
    lib.gqa_read_probe.restype = i
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().gqa_status_string(int(status)).decode()


def _check(status: int, what: str) -> None:
    if status != GQA_OK:
        raise GqaError(status, what)


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _ptr(t: Optional[torch.Tensor]):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _dense(name: str, t: torch.Tensor, ndim: int) -> None:
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise ValueError("%s must be a GPU tensor" % name)
    if t.dim() != ndim or not t.is_contiguous():
        raise ValueError("%s must be a contiguous %d-d tensor" % (name, ndim))


def _same_device(ref: torch.Tensor, **named) -> None:
    for n, t in named.items():
        if t.device != ref.device:
            raise ValueError("%s is on %s, expected %s" % (n, t.device, ref.device))


def _workspace(ws: torch.Tensor, ref: torch.Tensor):
    """Device pointer and size in bytes of a workspace tensor on ref's device."""
    if not isinstance(ws, torch.Tensor) or ws.device != ref.device or not ws.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on %s" % ref.device)
    return _ptr(ws), ws.numel() * ws.element_size()


def default_scale(D: int) -> float:
    """1/sqrt(D) rounded to float32 (the value the kernels receive)."""
    return float(torch.tensor(1.0 / math.sqrt(D), dtype=torch.float32))


def gqa_abi_version() -> int:
    return int(load().gqa_abi_version())


def gqa_decode_workspace_bytes(B: int, Hq: int, Hkv: int, D: int, s_cap: int) -> int:
    return int(load().gqa_decode_workspace_bytes(B, Hq, Hkv, D, s_cap))


def make_workspace(B: int, Hq: int, Hkv: int, D: int, s_cap: int, device="cuda") -> torch.Tensor:
    """A zero-filled (hence ready) decode workspace for these sizes."""
    n = gqa_decode_workspace_bytes(B, Hq, Hkv, D, s_cap)
    if n == 0:
        raise ValueError("invalid decode sizes")
    return torch.zeros(n, dtype=torch.uint8, device=device)


def gqa_workspace_init(workspace: torch.Tensor) -> None:
    if not isinstance(workspace, torch.Tensor) or workspace.device.type != "cuda" or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous GPU tensor")
    _check(load().gqa_workspace_init(_ptr(workspace), workspace.numel() * workspace.element_size(),
                                     _stream(workspace)), "gqa_workspace_init")


def gqa_decode_attend(q, k, v, out, kv_len: int, workspace, scale: Optional[float] = None) -> torch.Tensor:
    """q, out [B,Hq,1,D]; k, v [B,Hkv,s_cap,D] (same dtype); attends over rows < kv_len."""
    for n, t in (("q", q), ("k", k), ("v", v), ("out", out)):
        _dense(n, t, 4)
    B, Hq, Tq, D = q.shape
    _, Hkv, s_cap, _ = k.shape
    if Tq != 1 or out.shape != q.shape or k.shape != v.shape or k.shape[0] != B or k.shape[3] != D:
        raise ValueError("shape mismatch")
    dt = _DTYPE_CODE.get(q.dtype, -1)
    if not (q.dtype == k.dtype == v.dtype == out.dtype):
        raise ValueError("q, k, v and out must share one dtype")
    _same_device(q, k=k, v=v, out=out)
    ws, ws_bytes = _workspace(workspace, q)
    scale = default_scale(D) if scale is None else scale
    _check(load().gqa_decode_attend(_ptr(q), _ptr(k), _ptr(v), _ptr(out), B, Hq, Hkv, D, int(kv_len), s_cap,
                                    float(scale), dt, ws, ws_bytes, _stream(q)),
           "gqa_decode_attend")
    return out


def gqa_decode_attend_noalloc(q, k, v, out, kv_len: int, scale: Optional[float] = None) -> torch.Tensor:
    """As gqa_decode_attend, with the library's built-in scratch instead of a workspace (allocates nothing)."""
    for n, t in (("q", q), ("k", k), ("v", v), ("out", out)):
        _dense(n, t, 4)
    B, Hq, Tq, D = q.shape
    _, Hkv, s_cap, _ = k.shape
    if Tq != 1 or out.shape != q.shape or k.shape != v.shape or k.shape[0] != B or k.shape[3] != D:
        raise ValueError("shape mismatch")
    if not (q.dtype == k.dtype == v.dtype == out.dtype):
        raise ValueError("q, k, v and out must share one dtype")
    _same_device(q, k=k, v=v, out=out)
    scale = default_scale(D) if scale is None else scale
    _check(load().gqa_decode_attend_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(out), B, Hq, Hkv, D, int(kv_len), s_cap,
                                            float(scale), _DTYPE_CODE.get(q.dtype, -1), _stream(q)),
           "gqa_decode_attend_noalloc")
    return out


def gqa_decode_attend_batched(q, k, v, out, kv_lens, workspace, scale: Optional[float] = None) -> torch.Tensor:
    """As gqa_decode_attend with a device int32 [B] of per-request lengths."""
    for n, t in (("q", q), ("k", k), ("v", v), ("out", out)):
        _dense(n, t, 4)
    _dense("kv_lens", kv_lens, 1)
    B, Hq, Tq, D = q.shape
    _, Hkv, s_cap, _ = k.shape
    if Tq != 1 or out.shape != q.shape or k.shape != v.shape or k.shape[0] != B or k.shape[3] != D:
        raise ValueError("shape mismatch")
    if kv_lens.dtype != torch.int32 or kv_lens.numel() != B:
        raise ValueError("kv_lens must be int32 [B]")
    if not (q.dtype == k.dtype == v.dtype == out.dtype):
        raise ValueError("q, k, v and out must share one dtype")
    dt = _DTYPE_CODE.get(q.dtype, -1)
    _same_device(q, k=k, v=v, out=out, kv_lens=kv_lens)
    ws, ws_bytes = _workspace(workspace, q)
    scale = default_scale(D) if scale is None else scale
    _check(load().gqa_decode_attend_batched(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(kv_lens), B, Hq, Hkv, D,
                                            s_cap, float(scale), dt, ws, ws_bytes,
                                            _stream(q)), "gqa_decode_attend_batched")
    return out


def gqa_prefill_workspace_bytes(B: int, Hq: int, Hkv: int, D: int, Tq: int, Tk: int) -> int:
    return int(load().gqa_prefill_workspace_bytes(B, Hq, Hkv, D, Tq, Tk))


def make_prefill_workspace(B: int, Hq: int, Hkv: int, D: int, Tq: int, Tk: int, device="cuda") -> torch.Tensor:
    """A zero-filled (hence ready) prefill workspace for these sizes."""
    n = gqa_prefill_workspace_bytes(B, Hq, Hkv, D, Tq, Tk)
    if n == 0:
        raise ValueError("invalid prefill sizes")
    return torch.zeros(n, dtype=torch.uint8, device=device)


def gqa_prefill_causal(q, k, v, out, workspace, Tk: Optional[int] = None,
                       scale: Optional[float] = None) -> torch.Tensor:
    """q, out [B,Hq,Tq,D]; k, v [B,Hkv,s_cap,D]; queries aligned to the end of the first Tk keys.
    workspace: uint8 device tensor of gqa_prefill_workspace_bytes(...) bytes, zero-filled once."""
    for n, t in (("q", q), ("k", k), ("v", v), ("out", out)):
        _dense(n, t, 4)
    B, Hq, Tq, D = q.shape
    _, Hkv, s_cap, _ = k.shape
    if out.shape != q.shape or k.shape != v.shape or k.shape[0] != B or k.shape[3] != D:
        raise ValueError("shape mismatch")
    if not (q.dtype == k.dtype == v.dtype == out.dtype):
        raise ValueError("q, k, v and out must share one dtype")
    Tk = s_cap if Tk is None else int(Tk)
    dt = _DTYPE_CODE.get(q.dtype, -1)
    _same_device(q, k=k, v=v, out=out)
    ws, ws_bytes = _workspace(workspace, q)
    scale = default_scale(D) if scale is None else scale
    _check(load().gqa_prefill_causal(_ptr(q), _ptr(k), _ptr(v), _ptr(out), B, Hq, Hkv, D, Tq, Tk, s_cap,
                                     float(scale), dt, ws, ws_bytes, _stream(q)),
           "gqa_prefill_causal")
    return out


def _sinks(sinks, ref, Hq):
    if sinks is None:
        return ctypes.c_void_p(0)
    _dense("sinks", sinks, 1)
    if sinks.dtype != torch.float32 or sinks.numel() != Hq:
        raise ValueError("sinks must be float32 [Hq]")
    _same_device(ref, sinks=sinks)
    return _ptr(sinks)


def gqa_decode_attend_ex(q, k, v, out, kv_lens, workspace, window: int = 0, sinks=None,
                         scale: Optional[float] = None) -> torch.Tensor:
    """Batched decode with a sliding window (last `window` keys; 0 = none) and per-head sink logits [Hq]."""
    for n, t in (("q", q), ("k", k), ("v", v), ("out", out)):
        _dense(n, t, 4)
    _dense("kv_lens", kv_lens, 1)
    B, Hq, Tq, D = q.shape
    _, Hkv, s_cap, _ = k.shape
    if Tq != 1 or out.shape != q.shape or k.shape != v.shape or k.shape[0] != B or k.shape[3] != D:
        raise ValueError("shape mismatch")
    if kv_lens.dtype != torch.int32 or kv_lens.numel() != B:
        raise ValueError("kv_lens must be int32 [B]")
    if not (q.dtype == k.dtype == v.dtype == out.dtype):
        raise ValueError("q, k, v and out must share one dtype")
    _same_device(q, k=k, v=v, out=out, kv_lens=kv_lens)
    ws, ws_bytes = _workspace(workspace, q)
    scale = default_scale(D) if scale is None else scale
    _check(load().gqa_decode_attend_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(kv_lens), B, Hq, Hkv, D, s_cap,
                                       float(scale), _DTYPE_CODE.get(q.dtype, -1), int(window), _sinks(sinks, q, Hq),
                                       ws, ws_bytes, _stream(q)), "gqa_decode_attend_ex")
    return out


def gqa_prefill_workspace_bytes_ex(B: int, Hq: int, Hkv: int, D: int, Tq: int, Tk: int, window: int) -> int:
    return int(load().gqa_prefill_workspace_bytes_ex(B, Hq, Hkv, D, Tq, Tk, window))


def gqa_prefill_causal_ex(q, k, v, out, workspace, Tk: Optional[int] = None, window: int = 0, sinks=None,
                          scale: Optional[float] = None) -> torch.Tensor:
    """Causal prefill with a sliding window (0 = none) and per-head sink logits [Hq]."""
    for n, t in (("q", q), ("k", k), ("v", v), ("out", out)):
        _dense(n, t, 4)
    B, Hq, Tq, D = q.shape
    _, Hkv, s_cap, _ = k.shape
    if out.shape != q.shape or k.shape != v.shape or k.shape[0] != B or k.shape[3] != D:
        raise ValueError("shape mismatch")
    if not (q.dtype == k.dtype == v.dtype == out.dtype):
        raise ValueError("q, k, v and out must share one dtype")
    Tk = s_cap if Tk is None else int(Tk)
    _same_device(q, k=k, v=v, out=out)
    ws, ws_bytes = _workspace(workspace, q)
    scale = default_scale(D) if scale is None else scale
    _check(load().gqa_prefill_causal_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(out), B, Hq, Hkv, D, Tq, Tk, s_cap,
                                        float(scale), _DTYPE_CODE.get(q.dtype, -1), int(window),
                                        _sinks(sinks, q, Hq), ws, ws_bytes, _stream(q)), "gqa_prefill_causal_ex")
    return out


def gqa_decode_attend_q4(q, k_codes, k_scales, k_biases, v_codes, v_scales, v_biases, out, group_size: int,
                         kv_len: int, workspace, scale: Optional[float] = None) -> torch.Tensor:
    """q, out f16 [B,Hq,1,D]; codes uint8 [B,Hkv,s_cap,D/2]; scales, biases f16 [B,Hkv,s_cap,D/group]."""
    for n, t in (("q", q), ("out", out), ("k_codes", k_codes), ("v_codes", v_codes), ("k_scales", k_scales),
                 ("k_biases", k_biases), ("v_scales", v_scales), ("v_biases", v_biases)):
        _dense(n, t, 4)
    B, Hq, Tq, D = q.shape
    _, Hkv, s_cap, half = k_codes.shape
    if Tq != 1 or out.shape != q.shape or half * 2 != D or v_codes.shape != k_codes.shape:
        raise ValueError("shape mismatch")
    if q.dtype != torch.float16 or out.dtype != torch.float16:
        raise ValueError("q and out must be float16")
    if k_codes.dtype != torch.uint8 or v_codes.dtype != torch.uint8:
        raise ValueError("codes must be uint8")
    gshape = (B, Hkv, s_cap, D // group_size)
    for n, t in (("k_scales", k_scales), ("k_biases", k_biases), ("v_scales", v_scales), ("v_biases", v_biases)):
        if t.dtype != torch.float16 or tuple(t.shape) != gshape:
            raise ValueError("%s must be float16 %s" % (n, gshape))
    _same_device(q, out=out, k_codes=k_codes, v_codes=v_codes, k_scales=k_scales, k_biases=k_biases,
                 v_scales=v_scales, v_biases=v_biases)
    ws, ws_bytes = _workspace(workspace, q)
    scale = default_scale(D) if scale is None else scale
    _check(load().gqa_decode_attend_q4(_ptr(q), _ptr(k_codes), _ptr(k_scales), _ptr(k_biases), _ptr(v_codes),
                                       _ptr(v_scales), _ptr(v_biases), _ptr(out), B, Hq, Hkv, D, int(group_size),
                                       int(kv_len), s_cap, float(scale), ws, ws_bytes,
                                       _stream(q)), "gqa_decode_attend_q4")
    return out


def gqa_dequant_q4(codes, scales, biases, out, group_size: int) -> torch.Tensor:
    """codes uint8 [..., D/2], scales/biases f16 [..., D/group] -> out float32 [..., D]."""
    for n, t in (("codes", codes), ("scales", scales), ("biases", biases), ("out", out)):
        if t.device.type != "cuda" or not t.is_contiguous():
            raise ValueError("%s must be a contiguous GPU tensor" % n)
    D = codes.shape[-1] * 2
    n_rows = codes.numel() // max(codes.shape[-1], 1)
    if codes.dtype != torch.uint8:
        raise ValueError("codes must be uint8")
    if out.dtype != torch.float32 or out.numel() != n_rows * D:
        raise ValueError("out must be float32 with D elements per row")
    group_size = int(group_size)
    for n, t in (("scales", scales), ("biases", biases)):
        if t.dtype != torch.float16 or group_size <= 0 or t.numel() != n_rows * (D // group_size):
            raise ValueError("%s must be float16 with D/group_size elements per row" % n)
    _same_device(codes, scales=scales, biases=biases, out=out)
    _check(load().gqa_dequant_q4(_ptr(codes), _ptr(scales), _ptr(biases), _ptr(out), n_rows, D,
                                 int(group_size), _stream(codes)), "gqa_dequant_q4")
    return out


def gqa_kv_append(k_new, v_new, k_cache, v_cache, kv_lens, new_lens=None) -> None:
    """k_new, v_new [B,Hkv,T_new,D]; caches [B,Hkv,s_cap,D] (same dtype); kv_lens, new_lens int32 [B] (device)."""
    for n, t in (("k_new", k_new), ("v_new", v_new), ("k_cache", k_cache), ("v_cache", v_cache)):
        _dense(n, t, 4)
    _dense("kv_lens", kv_lens, 1)
    B, Hkv, T_new, D = k_new.shape
    s_cap = k_cache.shape[2]
    if v_new.shape != k_new.shape or k_cache.shape != v_cache.shape or k_cache.shape[:2] != (B, Hkv) \
            or k_cache.shape[3] != D:
        raise ValueError("shape mismatch")
    if not (k_new.dtype == v_new.dtype == k_cache.dtype == v_cache.dtype):
        raise ValueError("new rows and caches must share one dtype")
    if kv_lens.dtype != torch.int32 or kv_lens.numel() != B:
        raise ValueError("kv_lens must be int32 [B]")
    if new_lens is not None:
        _dense("new_lens", new_lens, 1)
        if new_lens.dtype != torch.int32 or new_lens.numel() != B:
            raise ValueError("new_lens must be int32 [B]")
        _same_device(k_new, new_lens=new_lens)
    _same_device(k_new, v_new=v_new, k_cache=k_cache, v_cache=v_cache, kv_lens=kv_lens)
    _check(load().gqa_kv_append(_ptr(k_new), _ptr(v_new), _ptr(k_cache), _ptr(v_cache), _ptr(kv_lens),
                                _ptr(new_lens), B, Hkv, D, T_new, s_cap, _DTYPE_CODE.get(k_new.dtype, -1),
                                _stream(k_new)), "gqa_kv_append")


def gqa_kv_append_q4(k_new, v_new, k_codes, k_scales, k_biases, v_codes, v_scales, v_biases, group_size: int,
                     kv_lens, new_lens=None) -> None:
    """k_new, v_new [B,Hkv,T_new,D] (f32/bf16/f16); 4-bit caches as in gqa_decode_attend_q4; lengths int32 [B]."""
    for n, t in (("k_new", k_new), ("v_new", v_new), ("k_codes", k_codes), ("v_codes", v_codes),
                 ("k_scales", k_scales), ("k_biases", k_biases), ("v_scales", v_scales), ("v_biases", v_biases)):
        _dense(n, t, 4)
    _dense("kv_lens", kv_lens, 1)
    B, Hkv, T_new, D = k_new.shape
    s_cap = k_codes.shape[2]
    group_size = int(group_size)
    if v_new.shape != k_new.shape or k_codes.shape != (B, Hkv, s_cap, D // 2) or v_codes.shape != k_codes.shape:
        raise ValueError("shape mismatch")
    if k_new.dtype != v_new.dtype or k_codes.dtype != torch.uint8 or v_codes.dtype != torch.uint8:
        raise ValueError("dtype mismatch")
    gshape = (B, Hkv, s_cap, D // max(group_size, 1))
    for n, t in (("k_scales", k_scales), ("k_biases", k_biases), ("v_scales", v_scales), ("v_biases", v_biases)):
        if t.dtype != torch.float16 or tuple(t.shape) != gshape:
            raise ValueError("%s must be float16 %s" % (n, gshape))
    if kv_lens.dtype != torch.int32 or kv_lens.numel() != B:
        raise ValueError("kv_lens must be int32 [B]")
    if new_lens is not None:
        _dense("new_lens", new_lens, 1)
        if new_lens.dtype != torch.int32 or new_lens.numel() != B:
            raise ValueError("new_lens must be int32 [B]")
        _same_device(k_new, new_lens=new_lens)
    _same_device(k_new, v_new=v_new, k_codes=k_codes, v_codes=v_codes, k_scales=k_scales, k_biases=k_biases,
                 v_scales=v_scales, v_biases=v_biases, kv_lens=kv_lens)
    _check(load().gqa_kv_append_q4(_ptr(k_new), _ptr(v_new), _DTYPE_CODE.get(k_new.dtype, -1), _ptr(k_codes),
                                   _ptr(k_scales), _ptr(k_biases), _ptr(v_codes), _ptr(v_scales), _ptr(v_biases),
                                   _ptr(kv_lens), _ptr(new_lens), B, Hkv, D, group_size, T_new, s_cap,
                                   _stream(k_new)), "gqa_kv_append_q4")


def _q4r_cache_shapes(k_codes, v_codes, k_scales, k_biases, v_scales, v_biases, k_res, v_res, group_size: int):
    """Checks a residual-window 4-bit cache; returns (B, Hkv, s_cap, D, R)."""
    for n, t in (("k_codes", k_codes), ("v_codes", v_codes), ("k_scales", k_scales), ("k_biases", k_biases),
                 ("v_scales", v_scales), ("v_biases", v_biases), ("k_res", k_res), ("v_res", v_res)):
        _dense(n, t, 4)
    B, Hkv, s_cap, half = k_codes.shape
    D = 2 * half
    R = k_res.shape[2]
    if v_codes.shape != k_codes.shape or k_codes.dtype != torch.uint8 or v_codes.dtype != torch.uint8:
        raise ValueError("codes must be uint8 [B,Hkv,s_cap,D/2], K and V alike")
    gshape = (B, Hkv, s_cap, D // max(int(group_size), 1))
    for n, t in (("k_scales", k_scales), ("k_biases", k_biases), ("v_scales", v_scales), ("v_biases", v_biases)):
        if t.dtype != torch.float16 or tuple(t.shape) != gshape:
            raise ValueError("%s must be float16 %s" % (n, gshape))
    for n, t in (("k_res", k_res), ("v_res", v_res)):
        if t.dtype != torch.float16 or tuple(t.shape) != (B, Hkv, R, D):
            raise ValueError("%s must be float16 [B,Hkv,R,D]" % n)
    _same_device(k_codes, v_codes=v_codes, k_scales=k_scales, k_biases=k_biases, v_scales=v_scales,
                 v_biases=v_biases, k_res=k_res, v_res=v_res)
    return B, Hkv, s_cap, D, R


def gqa_decode_q4r_workspace_bytes(B: int, Hq: int, Hkv: int, D: int, s_cap: int, R: int) -> int:
    return int(load().gqa_decode_q4r_workspace_bytes(B, Hq, Hkv, D, s_cap, R))


def make_q4r_workspace(B: int, Hq: int, Hkv: int, D: int, s_cap: int, R: int, device="cuda") -> torch.Tensor:
    """A zero-filled workspace for gqa_decode_attend_q4r."""
    n = gqa_decode_q4r_workspace_bytes(B, Hq, Hkv, D, s_cap, R)
    if n == 0:
        raise ValueError("invalid residual-window decode sizes")
    return torch.zeros(n, dtype=torch.uint8, device=device)


def gqa_decode_attend_q4r(q, k_codes, k_scales, k_biases, v_codes, v_scales, v_biases, k_res, v_res, out,
                          group_size: int, kv_lens, workspace, scale: Optional[float] = None) -> torch.Tensor:
    """Decode over a residual-window 4-bit cache: q, out f16 [B,Hq,1,D]; 4-bit arrays as in
    gqa_decode_attend_q4; k_res, v_res f16 [B,Hkv,R,D]; kv_lens int32 [B] (tokens per request)."""
    B, Hkv, s_cap, D, R = _q4r_cache_shapes(k_codes, v_codes, k_scales, k_biases, v_scales, v_biases, k_res, v_res,
                                            group_size)
    _dense("q", q, 4)
    _dense("out", out, 4)
    _dense("kv_lens", kv_lens, 1)
    if q.shape[0] != B or q.shape[2] != 1 or q.shape[3] != D or out.shape != q.shape:
        raise ValueError("q and out must be [B,Hq,1,D]")
    if q.dtype != torch.float16 or out.dtype != torch.float16:
        raise ValueError("q and out must be float16")
    if kv_lens.dtype != torch.int32 or kv_lens.numel() != B:
        raise ValueError("kv_lens must be int32 [B]")
    _same_device(q, out=out, k_codes=k_codes, kv_lens=kv_lens)
    ws, ws_bytes = _workspace(workspace, q)
    Hq = q.shape[1]
    scale = default_scale(D) if scale is None else scale
    _check(load().gqa_decode_attend_q4r(_ptr(q), _ptr(k_codes), _ptr(k_scales), _ptr(k_biases), _ptr(v_codes),
                                        _ptr(v_scales), _ptr(v_biases), _ptr(k_res), _ptr(v_res), _ptr(out),
                                        _ptr(kv_lens), B, Hq, Hkv, D, int(group_size), R, s_cap, float(scale), ws,
                                        ws_bytes, _stream(q)), "gqa_decode_attend_q4r")
    return out


def gqa_kv_append_q4r(k_new, v_new, k_codes, k_scales, k_biases, v_codes, v_scales, v_biases, k_res, v_res,
                      group_size: int, kv_lens, new_lens=None) -> None:
    """Append f16 rows k_new, v_new [B,Hkv,T_new,D] to a residual-window 4-bit cache."""
    B, Hkv, s_cap, D, R = _q4r_cache_shapes(k_codes, v_codes, k_scales, k_biases, v_scales, v_biases, k_res, v_res,
                                            group_size)
    _dense("k_new", k_new, 4)
    _dense("v_new", v_new, 4)
    _dense("kv_lens", kv_lens, 1)
    T_new = k_new.shape[2]
    if v_new.shape != k_new.shape or tuple(k_new.shape) != (B, Hkv, T_new, D):
        raise ValueError("k_new, v_new must be [B,Hkv,T_new,D]")
    if k_new.dtype != torch.float16 or v_new.dtype != torch.float16:
        raise ValueError("new rows must be float16")
    if kv_lens.dtype != torch.int32 or kv_lens.numel() != B:
        raise ValueError("kv_lens must be int32 [B]")
    if new_lens is not None:
        _dense("new_lens", new_lens, 1)
        if new_lens.dtype != torch.int32 or new_lens.numel() != B:
            raise ValueError("new_lens must be int32 [B]")
        _same_device(k_new, new_lens=new_lens)
    _same_device(k_new, v_new=v_new, k_codes=k_codes, kv_lens=kv_lens)
    _check(load().gqa_kv_append_q4r(_ptr(k_new), _ptr(v_new), _ptr(k_codes), _ptr(k_scales), _ptr(k_biases),
                                    _ptr(v_codes), _ptr(v_scales), _ptr(v_biases), _ptr(k_res), _ptr(v_res),
                                    _ptr(kv_lens), _ptr(new_lens), B, Hkv, D, int(group_size), R, T_new, s_cap,
                                    _stream(k_new)), "gqa_kv_append_q4r")


def gqa_prefill_causal_q4r(q, k_codes, k_scales, k_biases, v_codes, v_scales, v_biases, k_res, v_res, out,
                           group_size: int, Tk: int, workspace=None, scale: Optional[float] = None) -> torch.Tensor:
    """Causal prefill of q, out f16 [B,Hq,Tq,D] (the last Tq of Tk tokens) over a residual-window 4-bit cache."""
    B, Hkv, s_cap, D, R = _q4r_cache_shapes(k_codes, v_codes, k_scales, k_biases, v_scales, v_biases, k_res, v_res,
                                            group_size)
    _dense("q", q, 4)
    _dense("out", out, 4)
    if q.shape[0] != B or q.shape[3] != D or out.shape != q.shape:
        raise ValueError("q and out must be [B,Hq,Tq,D]")
    if q.dtype != torch.float16 or out.dtype != torch.float16:
        raise ValueError("q and out must be float16")
    _same_device(q, out=out, k_codes=k_codes)
    Hq, Tq = q.shape[1], q.shape[2]
    if workspace is None:
        workspace = make_prefill_workspace(B, Hq, Hkv, D, Tq, int(Tk), device=q.device)
    ws, ws_bytes = _workspace(workspace, q)
    scale = default_scale(D) if scale is None else scale
    _check(load().gqa_prefill_causal_q4r(_ptr(q), _ptr(k_codes), _ptr(k_scales), _ptr(k_biases), _ptr(v_codes),
                                         _ptr(v_scales), _ptr(v_biases), _ptr(k_res), _ptr(v_res), _ptr(out), B, Hq,
                                         Hkv, D, int(group_size), R, Tq, int(Tk), s_cap, float(scale), ws, ws_bytes,
                                         _stream(q)), "gqa_prefill_causal_q4r")
    return out


def gqa_read_probe(src: torch.Tensor, sink: torch.Tensor) -> None:
    """Stream every byte of `src` once (measurement helper; see gqa.h)."""
    for n, t in (("src", src), ("sink", sink)):
        if t.device.type != "cuda" or not t.is_contiguous():
            raise ValueError("%s must be a contiguous GPU tensor" % n)
    if sink.numel() * sink.element_size() < 4:
        raise ValueError("sink must hold at least 4 bytes")
    _same_device(src, sink=sink)
    _check(load().gqa_read_probe(_ptr(src), src.numel() * src.element_size(), _ptr(sink), _stream(src)),
           "gqa_read_probe")
