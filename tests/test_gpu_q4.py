"""GPU parity of the 4-bit quantized decode path.

* The dequant hook (the device routine the attention kernel applies to every
  element) is bit-identical to the oracle's unpack + dequant, on random
  codes with the edge codes 0 and 15 and zero scales, and on the encoded
  workload cache.
* Decode over the quantized cache (64 query / 8 KV heads, dim 128, group 64,
  f16 queries; KV length 2048 and 16384) matches the oracle's attention over
  the dequantized cache within 2e-2 (f16 outputs).
"""

import numpy as np
import pytest
import torch

import oracle
from tests.helpers import Guarded, assert_close, note
from workloads import configs as W
from workloads import gen

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("group", [32, 64, 128])
def test_dequant_hook_bit_exact(gpu_lib, group):
    rng = np.random.default_rng(group)
    D = 128
    codes = rng.integers(0, 16, size=(3, 40, D), dtype=np.uint8)
    codes[0, 0] = 0
    codes[0, 1] = 15
    scales = (rng.random((3, 40, D // group)) * 0.5).astype(np.float16)
    biases = (rng.standard_normal((3, 40, D // group)) * 3).astype(np.float16)
    scales[1, 3] = 0
    packed = gen.q4_pack_codes(codes)
    out = torch.empty((3, 40, D), dtype=torch.float32, device="cuda")
    gpu_lib.gqa_dequant_q4(torch.from_numpy(packed).cuda(), torch.from_numpy(scales).cuda(),
                           torch.from_numpy(biases).cuda(), out, group)
    torch.cuda.synchronize()
    want = oracle.q4_dequant(packed, scales, biases, group)
    got = out.cpu().numpy()
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


@pytest.mark.parametrize("D,group", [(128, 64), (64, 32)])
def test_dequant_hook_many_rows(gpu_lib, D, group):
    # more elements than one pass of the launch grid covers (grid-stride loop)
    rng = np.random.default_rng(D + group)
    n_rows = 150000 if D == 128 else 300000
    codes = rng.integers(0, 16, size=(n_rows, D), dtype=np.uint8)
    scales = (rng.random((n_rows, D // group)) * 0.5).astype(np.float16)
    biases = rng.standard_normal((n_rows, D // group)).astype(np.float16)
    packed = gen.q4_pack_codes(codes)
    out = torch.empty((n_rows, D), dtype=torch.float32, device="cuda")
    gpu_lib.gqa_dequant_q4(torch.from_numpy(packed).cuda(), torch.from_numpy(scales).cuda(),
                           torch.from_numpy(biases).cuda(), out, group)
    torch.cuda.synchronize()
    want = oracle.q4_dequant(packed, scales, biases, group)
    assert np.array_equal(out.cpu().numpy().view(np.uint32), want.view(np.uint32))


def run_q4(gqa, inp, w, kv_len):
    dev = {k: t.cuda() for k, t in inp.items()}
    q = dev["q"]
    B, Hq, _, D = q.shape
    Hkv, s_cap = dev["k_codes"].shape[1], dev["k_codes"].shape[2]
    ws = gqa.make_workspace(B, Hq, Hkv, D, s_cap)
    g = Guarded(q.shape, q.dtype)
    gqa.gqa_decode_attend_q4(q, dev["k_codes"], dev["k_scales"], dev["k_biases"], dev["v_codes"],
                             dev["v_scales"], dev["v_biases"], g.t, w.group, kv_len, ws, scale=w.scale())
    torch.cuda.synchronize()
    g.check()
    return g.t


def oracle_q4(inp, w, kv_len):
    return oracle.q4_attend(inp["q"], inp["k_codes"], inp["k_scales"], inp["k_biases"], inp["v_codes"],
                            inp["v_scales"], inp["v_biases"], w.group, kv_lens=kv_len, scale=w.scale())


@pytest.mark.parametrize("S", [2048, 16384])
def test_q4_decode_workload(gpu_lib, S):
    w = W.by_name("q4_decode")
    for layer in ((0, 79) if S == 2048 else (0,)):
        inp = W.q4_inputs(w, S, layer)
        note("q4 S=%d layer=%d" % (S, layer))
        got = run_q4(gpu_lib, inp, w, S)
        assert_close(got, oracle_q4(inp, w, S), 2e-2, "q4 S=%d layer %d" % (S, layer))


def test_q4_dequant_of_workload_cache(gpu_lib):
    w = W.by_name("q4_decode")
    inp = W.q4_inputs(w, 2048, 5)
    out = torch.empty((1, w.Hkv, 2048, w.D), dtype=torch.float32, device="cuda")
    gpu_lib.gqa_dequant_q4(inp["k_codes"].cuda(), inp["k_scales"].cuda(), inp["k_biases"].cuda(), out, w.group)
    torch.cuda.synchronize()
    want = oracle.q4_dequant(inp["k_codes"], inp["k_scales"], inp["k_biases"], w.group)
    assert np.array_equal(out.cpu().numpy().view(np.uint32), want.view(np.uint32))


@pytest.mark.parametrize("D,group", [(128, 64), (128, 32), (64, 64), (64, 32), (128, 128)])
def test_q4_small_ragged(gpu_lib, D, group):
    rng = np.random.default_rng(D + group)
    # (32, 2): 16 query heads per KV head, two head tiles of 8 reading the same KV head
    for Hq, Hkv, n, s_cap in [(8, 8, 1, 4), (64, 8, 33, 70), (16, 2, 100, 100), (12, 4, 777, 800),
                              (32, 2, 300, 320), (10, 2, 64, 64)]:
        x_k = rng.standard_normal((1, Hkv, s_cap, D)).astype(np.float32)
        x_v = rng.standard_normal((1, Hkv, s_cap, D)).astype(np.float32)
        kc, ks, kb = gen.q4_encode(x_k, group)
        vc, vs, vb = gen.q4_encode(x_v, group)
        ks[:, :, n:] = np.nan
        vb[:, :, n:] = np.nan
        inp = {"q": torch.from_numpy(rng.standard_normal((1, Hq, 1, D)).astype(np.float16)),
               "k_codes": torch.from_numpy(kc), "k_scales": torch.from_numpy(ks), "k_biases": torch.from_numpy(kb),
               "v_codes": torch.from_numpy(vc), "v_scales": torch.from_numpy(vs), "v_biases": torch.from_numpy(vb)}

        class Wg:
            pass

        wg = Wg()
        wg.group = group
        wg.scale = lambda: float(np.float32(1.0) / np.sqrt(np.float32(D)))
        note("q4 D=%d group=%d Hq=%d Hkv=%d n=%d" % (D, group, Hq, Hkv, n))
        got = run_q4(gpu_lib, inp, wg, n)
        assert_close(got, oracle_q4(inp, wg, n), 2e-2, "q4 n=%d" % n)


@pytest.mark.parametrize("scale", [-0.2, 0.0, 2.0])
def test_q4_scale_sign(gpu_lib, scale):
    # the running maximum is exact in this kernel: a negative scale, a zero
    # scale (plain mean of the dequantized value rows) and a large one
    w = W.by_name("q4_decode")
    inp = W.q4_inputs(w, 2048, 7)

    class Wg:
        pass

    wg = Wg()
    wg.group = w.group
    wg.scale = lambda: scale
    note("q4 scale=%g" % scale)
    got = run_q4(gpu_lib, inp, wg, 1500)
    assert_close(got, oracle_q4(inp, wg, 1500), 2e-2, "q4 scale=%g" % scale)


def test_q4_two_requests_merge_workgroups(gpu_lib):
    """Two requests of the 4-bit workload geometry (64 query / 8 KV heads,
    KV length 4096): 512 splits, more than the device has compute units, so
    the launch merges the splits with merge workgroups placed after them
    instead of in place; both requests match the oracle, and the first one
    is bit-identical to the same request decoded alone (the split of the KV
    length does not depend on the batch)."""
    w = W.by_name("q4_decode")
    S = 4096
    parts = [W.q4_inputs(w, S, layer) for layer in (3, 4)]
    inp = {k: torch.cat([p[k] for p in parts], dim=0) for k in parts[0]}
    note("q4 B=2 S=%d" % S)
    got = run_q4(gpu_lib, inp, w, S)
    assert_close(got, oracle_q4(inp, w, S), 2e-2, "q4 B=2")
    alone = run_q4(gpu_lib, parts[0], w, S)
    assert torch.equal(got[:1], alone)
