"""The allocation-free decode entry point (gqa_decode_attend_noalloc).

For callers that cannot allocate device memory: its partial results live in
a scratch array built into the library instead of a workspace.  Checked
through the C ABI:
* sizes past the scratch are rejected with GQA_ERR_SCRATCH before any
  device work (no GPU needed);
* on the GPU, two calls in a row -- the 28 query / 4 KV head fp32 decode at
  KV length 4096, then a smaller one (14 / 2 heads, dim 64, bf16, KV length
  300) -- and the first size again, each bit-identical to gqa_decode_attend
  with a workspace (same kernels, same split plan) and within the fp32 /
  bf16 bounds of the oracle.
"""

import ctypes

import numpy as np
import pytest
import torch

import oracle
import prefill_split_gqa_amd as gqa
from tests.helpers import assert_close, note
from workloads import configs as W

FAKE = ctypes.c_void_p(0x10000)
NULL = ctypes.c_void_p(0)


def test_noalloc_rejects_sizes_past_its_scratch():
    lib = gqa.load()
    call = lambda B, Hq, Hkv, D, s_cap: lib.gqa_decode_attend_noalloc(  # noqa: E731
        FAKE, FAKE, FAKE, FAKE, B, Hq, Hkv, D, 1, s_cap, ctypes.c_float(0.1), 0, NULL)
    # 64 requests of 32/8 heads at 4096 rows: 33 MB of partials > 7.5 MiB
    assert call(64, 32, 8, 128, 4096) == gqa.GQA_ERR_SCRATCH
    assert call(9, 28, 4, 128, 4096) == gqa.GQA_ERR_SCRATCH
    assert lib.gqa_decode_attend_noalloc(NULL, FAKE, FAKE, FAKE, 1, 28, 4, 128, 1, 64, ctypes.c_float(0.1), 0,
                                         NULL) == gqa.GQA_ERR_NULL
    assert gqa.status_string(gqa.GQA_ERR_SCRATCH).startswith("sizes exceed")


def _case(w, S, layer, dtype=None):
    q, k, v = W.decode_inputs(w, S, layer)
    if dtype is not None:
        q, k, v = (t.to(dtype) for t in (q, k, v))
    return q, k, v


@pytest.mark.gpu
def test_noalloc_matches_the_workspace_entry_point(gpu_lib):
    big = _case(W.by_name("decode_7b"), 4096, 3)
    small = _case(W.by_name("decode_0p5b"), 300, 0, torch.bfloat16)
    for name, (q, k, v), tol in (("7b S=4096 fp32", big, 2e-5), ("0.5b S=300 bf16 (smaller)", small, 2e-2),
                                 ("7b S=4096 fp32 again", big, 2e-5)):
        S = k.shape[2]
        dq, dk, dv = q.cuda(), k.cuda(), v.cuda()
        note("noalloc decode %s" % name)
        out_na = torch.empty_like(dq)
        gpu_lib.gqa_decode_attend_noalloc(dq, dk, dv, out_na, S)
        ws = gpu_lib.make_workspace(q.shape[0], q.shape[1], k.shape[1], q.shape[3], S)
        out_ws = torch.empty_like(dq)
        gpu_lib.gqa_decode_attend(dq, dk, dv, out_ws, S, ws)
        torch.cuda.synchronize()
        assert torch.equal(out_na, out_ws), name
        assert_close(out_na, oracle.attend(q, k, v), tol, name)
