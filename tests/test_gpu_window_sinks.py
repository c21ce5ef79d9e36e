"""GPU parity of the sliding window and attention sinks against the oracle.

Readings (the Fornace prefill page, "What this does not prove"; the
VeloxQuant-MLX "attention" posts, "Part 4"): with a window W a query sees
only the W most recent keys up to its own position; a sink is one logit per
query head that joins the softmax normaliser and carries no value.

* gqa_decode_attend_ex: windows from 1 key to past the length, ragged
  lengths (a zero-length request too), sinks of either sign and large ones
  (a sink far above every score leaves outputs near 0; far below, no
  effect), fp32 at 2e-5 and bf16 at 2e-2; with no window and no sinks it is
  bit-identical to the batched entry point.
* gqa_prefill_causal_ex: square prompts and a query chunk at an offset,
  windows of 1, 2, 5 and 17 keys (one key more or less at the window's
  lower edge moves a row by far more than the bound) and windows that
  start inside, at and past key-tile edges (64, 65, 100, 128, 129, 1000),
  long rows split into key chunks, sinks, bf16 and f16, D = 64 and 128.
"""

import numpy as np
import pytest
import torch

import oracle
from tests.helpers import assert_close, note, tol_for

pytestmark = pytest.mark.gpu

DT = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


def _rand(rng, shape, dtype):
    return torch.from_numpy(rng.standard_normal(shape, dtype=np.float32)).to(DT[dtype])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("Hq,Hkv,D", [(28, 4, 128), (14, 2, 64), (32, 8, 128)])
def test_decode_window_sinks(gpu_lib, dtype, Hq, Hkv, D):
    rng = np.random.default_rng(Hq * 10 + D + len(dtype))
    B, s_cap = 4, 700
    lens = np.array([700, 1, 333, 0], np.int32)
    q = _rand(rng, (B, Hq, 1, D), dtype)
    k = _rand(rng, (B, Hkv, s_cap, D), dtype)
    v = _rand(rng, (B, Hkv, s_cap, D), dtype)
    for b in range(B):
        k[b, :, lens[b]:] = float("nan")
        v[b, :, lens[b]:] = float("nan")
    dq, dk, dv = q.cuda(), k.cuda(), v.cuda()
    lens_d = torch.from_numpy(lens).cuda()
    ws = gpu_lib.make_workspace(B, Hq, Hkv, D, s_cap)
    for window in (0, 1, 5, 64, 100, 333, 699, 700, 5000):
        for sinks in (None, rng.standard_normal(Hq).astype(np.float32) * 3,
                      np.where(np.arange(Hq) % 2 == 0, 60.0, -60.0).astype(np.float32)):
            note("decode_ex %s Hq=%d Hkv=%d D=%d window=%d sinks=%s" % (dtype, Hq, Hkv, D, window,
                                                                          None if sinks is None else "set"))
            out = torch.empty_like(dq)
            sk = None if sinks is None else torch.from_numpy(sinks).cuda()
            gpu_lib.gqa_decode_attend_ex(dq, dk, dv, out, lens_d, ws, window=window, sinks=sk)
            torch.cuda.synchronize()
            want = oracle.attend(q, k, v, kv_lens=lens, window=window, sinks=sinks)
            assert_close(out, want, tol_for(DT[dtype]), "window=%d" % window)
            if window == 0 and sinks is None:
                ref = torch.empty_like(dq)
                gpu_lib.gqa_decode_attend_batched(dq, dk, dv, ref, lens_d, ws)
                torch.cuda.synchronize()
                assert torch.equal(out, ref)


PF_CASES = [
    # B, Hq, Hkv, D, Tq, Tk, dtype
    (1, 14, 2, 64, 300, 300, "bf16"),
    (1, 4, 2, 64, 1100, 1100, "bf16"),     # long rows split into key chunks
    (2, 4, 1, 128, 130, 1300, "f16"),      # a query chunk at an offset, D = 128
    (1, 7, 1, 64, 1057, 1057, "f16"),
]


@pytest.mark.parametrize("case", range(len(PF_CASES)))
def test_prefill_window_sinks(gpu_lib, case):
    B, Hq, Hkv, D, Tq, Tk, dtype = PF_CASES[case]
    rng = np.random.default_rng(case + 40)
    q = _rand(rng, (B, Hq, Tq, D), dtype)
    k = _rand(rng, (B, Hkv, Tk, D), dtype)
    v = _rand(rng, (B, Hkv, Tk, D), dtype)
    dq, dk, dv = q.cuda(), k.cuda(), v.cuda()
    for window in (1, 2, 5, 17, 63, 64, 65, 100, 128, 129, 1000, 0):
        for sinks in ((None, rng.standard_normal(Hq).astype(np.float32) * 2) if window in (5, 100, 0) else (None,)):
            note("prefill_ex %s B=%d Hq=%d Hkv=%d D=%d Tq=%d Tk=%d window=%d sinks=%s"
                 % (dtype, B, Hq, Hkv, D, Tq, Tk, window, sinks is not None))
            ws = torch.zeros(gpu_lib.gqa_prefill_workspace_bytes_ex(B, Hq, Hkv, D, Tq, Tk, window),
                             dtype=torch.uint8, device="cuda")
            out = torch.empty_like(dq)
            sk = None if sinks is None else torch.from_numpy(sinks).cuda()
            gpu_lib.gqa_prefill_causal_ex(dq, dk, dv, out, ws, window=window, sinks=sk)
            torch.cuda.synchronize()
            want = oracle.attend(q, k, v, causal=True, window=window, sinks=sinks)
            assert_close(out, want, 2e-2, "window=%d" % window)
