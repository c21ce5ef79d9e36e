"""GPU parity of the cache-append entry points against the oracle.

* gqa_kv_append: new K/V rows land at each request's length in a
  preallocated cache, bit for bit as the oracle's definition places them
  (ragged and zero lengths, rows past the capacity dropped, new lengths
  returned, every dtype); nothing else in the caches changes.
* gqa_kv_append_q4: new rows are encoded with the min-max group-affine
  quantizer; codes, f16 scales and biases equal the oracle's quantizer bit
  for bit (f16, bf16 and f32 inputs, every group size, constant groups,
  signed zeros, ties), placed at each request's length; other rows keep
  their bytes.
* Decode after appends: a 4-bit cache grown one token at a time (append,
  then decode over the new length, twenty steps) matches the oracle's
  attention over the oracle-quantized cache at every step, and its bytes
  equal the oracle's; a bf16 cache grown by appends for a ragged batch then
  decoded with the returned lengths matches the oracle.
"""

import numpy as np
import pytest
import torch

import oracle
from tests.helpers import assert_close, note
from workloads import configs as W

pytestmark = pytest.mark.gpu

DT = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("D", [64, 128])
def test_dense_append_bit_exact(gpu_lib, dtype, D):
    rng = np.random.default_rng(D + len(dtype))
    for B, Hkv, T_new, s_cap, lens in [(1, 4, 1, 64, [10]), (3, 8, 3, 40, [0, 39, 17]), (4, 2, 17, 50, [50, 40, 0, 7]),
                                       (2, 1, 5, 5, [-3, 2])]:
        cache_k = torch.from_numpy(rng.standard_normal((B, Hkv, s_cap, D), dtype=np.float32)).to(DT[dtype])
        cache_v = torch.from_numpy(rng.standard_normal((B, Hkv, s_cap, D), dtype=np.float32)).to(DT[dtype])
        new_k = torch.from_numpy(rng.standard_normal((B, Hkv, T_new, D), dtype=np.float32)).to(DT[dtype])
        new_v = torch.from_numpy(rng.standard_normal((B, Hkv, T_new, D), dtype=np.float32)).to(DT[dtype])
        want_k, want_lens = oracle.kv_append(cache_k.view(torch.int16 if dtype != "f32" else torch.int32).numpy(),
                                             new_k.view(torch.int16 if dtype != "f32" else torch.int32).numpy(), lens)
        want_v, _ = oracle.kv_append(cache_v.view(torch.int16 if dtype != "f32" else torch.int32).numpy(),
                                     new_v.view(torch.int16 if dtype != "f32" else torch.int32).numpy(), lens)
        dk, dv = cache_k.cuda(), cache_v.cuda()
        lens_d = torch.tensor(lens, dtype=torch.int32).cuda()
        out_lens = torch.full((B,), -1, dtype=torch.int32).cuda()
        note("append %s D=%d B=%d Hkv=%d T_new=%d s_cap=%d lens=%s" % (dtype, D, B, Hkv, T_new, s_cap, lens))
        gpu_lib.gqa_kv_append(new_k.cuda(), new_v.cuda(), dk, dv, lens_d, out_lens)
        torch.cuda.synchronize()
        iv = torch.int16 if dtype != "f32" else torch.int32
        assert np.array_equal(dk.cpu().view(iv).numpy(), want_k)
        assert np.array_equal(dv.cpu().view(iv).numpy(), want_v)
        assert out_lens.cpu().numpy().tolist() == want_lens.tolist()
        # without new_lens: the same placement
        dk2 = cache_k.cuda()
        gpu_lib.gqa_kv_append(new_k.cuda(), new_v.cuda(), dk2, cache_v.cuda(), lens_d)
        torch.cuda.synchronize()
        assert np.array_equal(dk2.cpu().view(iv).numpy(), want_k)


def _q4_cache(rng, B, Hkv, s_cap, D, group):
    codes = rng.integers(0, 256, size=(B, Hkv, s_cap, D // 2), dtype=np.uint8)
    sc = rng.standard_normal((B, Hkv, s_cap, D // group)).astype(np.float16)
    bi = rng.standard_normal((B, Hkv, s_cap, D // group)).astype(np.float16)
    return codes, sc, bi


def _edge_rows(x, group):
    """Plant edge groups in the first rows of x [B,Hkv,T,D] (float32 values
    representable in every input dtype)."""
    flat = x.reshape(-1, x.shape[-1])
    if flat.shape[0] >= 3:
        flat[0, :group] = 0.75                                  # constant group: scale 0, codes 0
        flat[1, :group] = 0.0
        flat[1, 0:group:2] = -0.0                               # signed zeros
        ramp = np.arange(group, dtype=np.float32) % 16
        flat[2, :group] = ramp                                  # scale 1: exact codes
        flat[2, 0] = 2.5                                        # a tie (code 2)
    return x


@pytest.mark.parametrize("dtype", ["f16", "bf16", "f32"])
@pytest.mark.parametrize("D,group", [(128, 64), (128, 32), (128, 128), (64, 64), (64, 32)])
def test_q4_append_bit_exact(gpu_lib, dtype, D, group):
    rng = np.random.default_rng(D * 3 + group + len(dtype))
    B, Hkv, T_new, s_cap = 3, 8, 2, 48
    lens = [0, 47, 20]
    x = {n: _edge_rows((rng.standard_normal((B, Hkv, T_new, D)) * 3).astype(np.float32), group) for n in "kv"}
    xt = {n: torch.from_numpy(x[n]).to(DT[dtype]) for n in "kv"}
    cache = {n: _q4_cache(rng, B, Hkv, s_cap, D, group) for n in "kv"}
    dev = {n: [torch.from_numpy(a.copy()).cuda() for a in cache[n]] for n in "kv"}
    lens_d = torch.tensor(lens, dtype=torch.int32).cuda()
    out_lens = torch.zeros(B, dtype=torch.int32).cuda()
    note("q4 append %s D=%d group=%d" % (dtype, D, group))
    gpu_lib.gqa_kv_append_q4(xt["k"].cuda(), xt["v"].cuda(), *dev["k"], *dev["v"], group, lens_d, out_lens)
    torch.cuda.synchronize()
    for n in "kv":
        qc, qs, qb = oracle.q4_quantize(xt[n], group)  # the oracle reads the same (cast) values
        wc, want_lens = oracle.kv_append(cache[n][0], qc, lens)
        ws, _ = oracle.kv_append(cache[n][1].view(np.uint16), qs.view(np.uint16), lens)
        wb, _ = oracle.kv_append(cache[n][2].view(np.uint16), qb.view(np.uint16), lens)
        assert np.array_equal(dev[n][0].cpu().numpy(), wc), n + " codes"
        assert np.array_equal(dev[n][1].cpu().numpy().view(np.uint16), ws), n + " scales"
        assert np.array_equal(dev[n][2].cpu().numpy().view(np.uint16), wb), n + " biases"
    assert out_lens.cpu().numpy().tolist() == want_lens.tolist()


def test_q4_decode_after_appends(gpu_lib):
    """The 4-bit workload geometry (64 query / 8 KV heads, dim 128, group 64)
    grown one token at a time from 100 rows: append, then decode over the new
    length, for 20 steps; every output against the oracle, and the cache bytes
    equal to the oracle's quantization of the same rows."""
    w = W.by_name("q4_decode")
    rng = np.random.default_rng(77)
    L0, steps, s_cap = 100, 20, 128
    k_all = torch.from_numpy(rng.standard_normal((1, w.Hkv, L0 + steps, w.D), dtype=np.float32)).to(torch.float16)
    v_all = torch.from_numpy(rng.standard_normal((1, w.Hkv, L0 + steps, w.D), dtype=np.float32)).to(torch.float16)
    cache = {}
    for n, x in (("k", k_all), ("v", v_all)):
        c, s_, b_ = oracle.q4_quantize(x[:, :, :L0], w.group)
        pad = s_cap - L0
        cache[n] = [np.concatenate([c, np.zeros((1, w.Hkv, pad, w.D // 2), np.uint8)], 2),
                    np.concatenate([s_, np.full((1, w.Hkv, pad, w.D // w.group), np.nan, np.float16)], 2),
                    np.concatenate([b_, np.full((1, w.Hkv, pad, w.D // w.group), np.nan, np.float16)], 2)]
    dev = {n: [torch.from_numpy(a.copy()).cuda() for a in cache[n]] for n in "kv"}
    ws = gpu_lib.make_workspace(1, w.Hq, w.Hkv, w.D, s_cap)
    lens = torch.tensor([L0], dtype=torch.int32).cuda()
    nxt = torch.zeros(1, dtype=torch.int32).cuda()
    for t in range(steps):
        q = torch.from_numpy(rng.standard_normal((1, w.Hq, 1, w.D), dtype=np.float32)).to(torch.float16)
        gpu_lib.gqa_kv_append_q4(k_all[:, :, L0 + t:L0 + t + 1].contiguous().cuda(),
                                 v_all[:, :, L0 + t:L0 + t + 1].contiguous().cuda(), *dev["k"], *dev["v"], w.group,
                                 lens, nxt)
        lens, nxt = nxt, lens
        n = L0 + t + 1
        out = torch.empty_like(q).cuda()
        gpu_lib.gqa_decode_attend_q4(q.cuda(), *dev["k"], *dev["v"], out, w.group, n, ws, scale=w.scale())
        torch.cuda.synchronize()
        assert int(lens.cpu()[0]) == n
        qk = oracle.q4_quantize(k_all[:, :, :n], w.group)
        qv = oracle.q4_quantize(v_all[:, :, :n], w.group)
        want = oracle.q4_attend(q, *qk, *qv, w.group, scale=w.scale())
        assert_close(out, want, 2e-2, "step %d (length %d)" % (t, n))
    for n, x in (("k", k_all), ("v", v_all)):
        c, s_, b_ = oracle.q4_quantize(x, w.group)
        assert np.array_equal(dev[n][0].cpu().numpy()[:, :, :L0 + steps], c)
        assert np.array_equal(dev[n][1].cpu().numpy()[:, :, :L0 + steps].view(np.uint16), s_.view(np.uint16))
        assert np.array_equal(dev[n][2].cpu().numpy()[:, :, :L0 + steps].view(np.uint16), b_.view(np.uint16))


def test_batched_decode_after_appends(gpu_lib):
    """Qwen3-4B heads (32 / 8, dim 128), bf16: four requests of ragged
    lengths receive 3 new tokens each through the append, then a batched
    decode over the returned lengths matches the oracle."""
    w = W.by_name("batched_qwen3_4b")
    rng = np.random.default_rng(5)
    B, s_cap, T_new = 4, 512, 3
    lens0 = np.array([0, 100, 509, 300], np.int32)
    k = torch.from_numpy(rng.standard_normal((B, w.Hkv, s_cap, w.D), dtype=np.float32)).to(torch.bfloat16)
    v = torch.from_numpy(rng.standard_normal((B, w.Hkv, s_cap, w.D), dtype=np.float32)).to(torch.bfloat16)
    kn = torch.from_numpy(rng.standard_normal((B, w.Hkv, T_new, w.D), dtype=np.float32)).to(torch.bfloat16)
    vn = torch.from_numpy(rng.standard_normal((B, w.Hkv, T_new, w.D), dtype=np.float32)).to(torch.bfloat16)
    q = torch.from_numpy(rng.standard_normal((B, w.Hq, 1, w.D), dtype=np.float32)).to(torch.bfloat16)
    dk, dv = k.cuda(), v.cuda()
    lens_d = torch.from_numpy(lens0).cuda()
    new_lens = torch.zeros(B, dtype=torch.int32).cuda()
    gpu_lib.gqa_kv_append(kn.cuda(), vn.cuda(), dk, dv, lens_d, new_lens)
    out = torch.empty_like(q).cuda()
    ws = gpu_lib.make_workspace(B, w.Hq, w.Hkv, w.D, s_cap)
    gpu_lib.gqa_decode_attend_batched(q.cuda(), dk, dv, out, new_lens, ws)
    torch.cuda.synchronize()
    kk, got_lens = oracle.kv_append(k.float().numpy(), kn.float().numpy(), lens0)
    vv, _ = oracle.kv_append(v.float().numpy(), vn.float().numpy(), lens0)
    assert new_lens.cpu().numpy().tolist() == got_lens.tolist() == [3, 103, 512, 303]
    assert_close(out, oracle.attend(q, kk, vv, kv_lens=got_lens), 2e-2, "batched decode after append")
