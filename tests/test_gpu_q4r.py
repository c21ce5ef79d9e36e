"""GPU parity of the residual-window 4-bit cache against the oracle.

* gqa_kv_append_q4r: after appends of every shape (single tokens across a
  flush, blocks longer than the residual, ragged and zero lengths, rows past
  the capacity), codes, f16 scales and biases and the float16 residual equal
  the oracle's (oracle.kv_append_q4r) bit for bit, every byte of every array
  (rows and slots the append must not touch keep their random contents).
* gqa_decode_attend_q4r: attention over the cache's values in position
  order (oracle.q4r_attend) within the 4-bit decode's bound, for requests
  with no 4-bit rows, no residual rows, both, and none; with an empty
  residual the output is bit-identical to gqa_decode_attend_q4 over the same
  4-bit rows; with no 4-bit rows the residual pass alone matches; a cache
  grown one token at a time across a flush matches the oracle at every step; the 4-bit decode workload's
  geometry at 16k keys.
* gqa_prefill_causal_q4r: a chunk of queries at the end of each request's
  tokens, causal, over 4-bit and residual rows (chunks that start inside the
  4-bit rows, a whole prompt, one query, an empty residual) within the f16
  bound; with no 4-bit rows bit-identical to gqa_prefill_causal over the
  residual; the pages' 256-query chunk after 3841 tokens on the 0.5B
  geometry.
"""

import numpy as np
import pytest
import torch

import oracle
from tests.helpers import TOL_16, assert_close, note
from workloads import configs as W

pytestmark = pytest.mark.gpu


def _rand_state(rng, B, H, s_cap, D, group, R):
    return {
        "k_codes": rng.integers(0, 256, size=(B, H, s_cap, D // 2), dtype=np.uint8),
        "v_codes": rng.integers(0, 256, size=(B, H, s_cap, D // 2), dtype=np.uint8),
        "k_scales": (rng.random((B, H, s_cap, D // group)) * 0.2).astype(np.float16),
        "k_biases": rng.standard_normal((B, H, s_cap, D // group)).astype(np.float16),
        "v_scales": (rng.random((B, H, s_cap, D // group)) * 0.2).astype(np.float16),
        "v_biases": rng.standard_normal((B, H, s_cap, D // group)).astype(np.float16),
        "k_res": rng.standard_normal((B, H, R, D)).astype(np.float16),
        "v_res": rng.standard_normal((B, H, R, D)).astype(np.float16),
    }


ORDER = ("k_codes", "k_scales", "k_biases", "v_codes", "v_scales", "v_biases", "k_res", "v_res")


def _to_dev(st):
    return {k: torch.from_numpy(np.ascontiguousarray(v)).cuda() for k, v in st.items()}


def _append(gpu_lib, dev, k_new, v_new, lens, group, new_lens=None):
    gpu_lib.gqa_kv_append_q4r(torch.from_numpy(k_new).cuda(), torch.from_numpy(v_new).cuda(), dev["k_codes"],
                              dev["k_scales"], dev["k_biases"], dev["v_codes"], dev["v_scales"], dev["v_biases"],
                              dev["k_res"], dev["v_res"], group, torch.tensor(lens, dtype=torch.int32).cuda(),
                              new_lens)


def _assert_state(dev, want, what):
    torch.cuda.synchronize()
    for key in ORDER:
        got = dev[key].cpu().numpy()
        assert np.array_equal(got.view(np.uint8), np.ascontiguousarray(want[key]).view(np.uint8)), "%s: %s" % (what,
                                                                                                            key)


@pytest.mark.parametrize("D,group,R", [(64, 32, 64), (128, 64, 128), (128, 128, 64), (128, 32, 192)])
def test_append_bit_exact(gpu_lib, D, group, R):
    rng = np.random.default_rng(D * 7 + group + R)
    B, H, s_cap = 4, 2, 4 * R
    for T_new, lens in [(1, [0, R - 1, R, 2 * R + 5]), (3, [R - 2, 1, s_cap - 1, s_cap]), (R + 9, [0, 5, R, 3 * R]),
                        (2 * R + 1, [R - 1, 0, 7, -4])]:
        st = _rand_state(rng, B, H, s_cap, D, group, R)
        k_new = rng.standard_normal((B, H, T_new, D)).astype(np.float16)
        v_new = (rng.standard_normal((B, H, T_new, D)) * 3).astype(np.float16)
        want, want_lens = oracle.kv_append_q4r(st, k_new, v_new, lens, group, R)
        dev = _to_dev(st)
        out_lens = torch.full((B,), -1, dtype=torch.int32).cuda()
        note("q4r append D=%d group=%d R=%d T_new=%d lens=%s" % (D, group, R, T_new, lens))
        _append(gpu_lib, dev, k_new, v_new, lens, group, out_lens)
        _assert_state(dev, want, "T_new=%d lens=%s" % (T_new, lens))
        assert out_lens.cpu().numpy().tolist() == want_lens.tolist()


def _decode(gpu_lib, dev, q, lens, group, ws, scale=None):
    out = torch.empty_like(q)
    gpu_lib.gqa_decode_attend_q4r(q, dev["k_codes"], dev["k_scales"], dev["k_biases"], dev["v_codes"],
                                  dev["v_scales"], dev["v_biases"], dev["k_res"], dev["v_res"], out, group,
                                  torch.tensor(lens, dtype=torch.int32).cuda(), ws, scale)
    torch.cuda.synchronize()
    return out


def _grown_state(rng, B, H, s_cap, D, group, R, lens):
    """A cache filled by the oracle's own append from float16 rows: request b holds lens[b] tokens."""
    st = {k: np.zeros_like(v) for k, v in _rand_state(rng, B, H, s_cap, D, group, R).items()}
    T = max(max(lens), 1)
    k = rng.standard_normal((B, H, T, D)).astype(np.float16)
    v = rng.standard_normal((B, H, T, D)).astype(np.float16)
    st, _ = oracle.kv_append_q4r(st, k, v, [0] * B, group, R)
    # trim each request to its length: a fresh cache appended to lens[b]
    st2 = {k_: np.zeros_like(v_) for k_, v_ in st.items()}
    for b, n in enumerate(lens):
        one = {k_: v_[b:b + 1] * 0 for k_, v_ in st.items()}
        one, _ = oracle.kv_append_q4r(one, k[b:b + 1, :, :n], v[b:b + 1, :, :n], [0], group, R)
        for k_ in st2:
            st2[k_][b] = one[k_][0]
    return st2


@pytest.mark.parametrize("D,group,R", [(64, 64, 64), (128, 64, 128), (128, 32, 64)])
def test_decode_ragged_lengths(gpu_lib, D, group, R):
    rng = np.random.default_rng(D + group * 3 + R)
    Hq, H, s_cap = 8, 2, 6 * R
    lens = [0, 1, R - 1, R, R + 1, 3 * R + 17, s_cap]
    B = len(lens)
    st = _grown_state(rng, B, H, s_cap, D, group, R, lens)
    dev = _to_dev(st)
    q = torch.from_numpy(rng.standard_normal((B, Hq, 1, D)).astype(np.float16)).cuda()
    ws = gpu_lib.make_q4r_workspace(B, Hq, H, D, s_cap, R)
    note("q4r decode D=%d group=%d R=%d lens=%s" % (D, group, R, lens))
    got = _decode(gpu_lib, dev, q, lens, group, ws)
    want = oracle.q4r_attend(q.cpu(), st, lens, group, R)
    assert_close(got, want, TOL_16, "q4r decode lens=%s" % lens)
    assert not got[0].float().abs().max().item()  # no tokens: zeros
    # the workspace is reusable without clearing: the same call again, bit for bit
    again = _decode(gpu_lib, dev, q, lens, group, ws)
    assert torch.equal(got, again)


@pytest.mark.parametrize("D,group,R", [(128, 64, 128), (64, 32, 64)])
def test_decode_reduces_to_plain_kernels(gpu_lib, D, group, R):
    rng = np.random.default_rng(17 + D + R)
    # (at these sizes both plans cut the rows into the same splits; the
    # residual-window plan keeps one more for the residual)
    Hq, H, s_cap = 8, 2, 8 * R
    # empty residual (n a multiple of R): bit-identical to the plain 4-bit decode
    n = 5 * R
    st = _grown_state(rng, 1, H, s_cap, D, group, R, [n])
    dev = _to_dev(st)
    q = torch.from_numpy(rng.standard_normal((1, Hq, 1, D)).astype(np.float16)).cuda()
    note("q4r decode == q4 decode D=%d group=%d R=%d n=%d" % (D, group, R, n))
    got = _decode(gpu_lib, dev, q, [n], group, gpu_lib.make_q4r_workspace(1, Hq, H, D, s_cap, R))
    ref = torch.empty_like(q)
    gpu_lib.gqa_decode_attend_q4(q, dev["k_codes"], dev["k_scales"], dev["k_biases"], dev["v_codes"],
                                 dev["v_scales"], dev["v_biases"], ref, group, n,
                                 gpu_lib.make_workspace(1, Hq, H, D, s_cap))
    torch.cuda.synchronize()
    assert torch.equal(got, ref)
    # no 4-bit rows (n < R): the residual pass alone (one split per head
    # tile), against the oracle and the dense float16 decode of the residual
    n = R - 3
    st = _grown_state(rng, 1, H, s_cap, D, group, R, [n])
    dev = _to_dev(st)
    note("q4r decode, residual only D=%d R=%d n=%d" % (D, R, n))
    got = _decode(gpu_lib, dev, q, [n], group, gpu_lib.make_q4r_workspace(1, Hq, H, D, s_cap, R))
    ref = torch.empty_like(q)
    gpu_lib.gqa_decode_attend_batched(q, dev["k_res"], dev["v_res"], ref, torch.tensor([n], dtype=torch.int32).cuda(),
                                      gpu_lib.make_workspace(1, Hq, H, D, R))
    torch.cuda.synchronize()
    want = oracle.q4r_attend(q.cpu(), st, [n], group, R)
    assert_close(got, want, TOL_16, "q4r residual only")
    assert_close(ref, want, TOL_16, "dense f16 decode of the residual")


def test_decode_while_growing_across_a_flush(gpu_lib):
    rng = np.random.default_rng(23)
    B, Hq, H, D, group, R, s_cap = 2, 8, 2, 128, 64, 64, 512
    lens = np.array([40, 120], np.int32)
    st = _grown_state(rng, B, H, s_cap, D, group, R, lens.tolist())
    dev = _to_dev(st)
    ws = gpu_lib.make_q4r_workspace(B, Hq, H, D, s_cap, R)
    lens_d = torch.from_numpy(lens.copy()).cuda()
    new_d = torch.empty_like(lens_d)
    for step in range(30):  # request 0 crosses 64, request 1 crosses 128
        kn = rng.standard_normal((B, H, 1, D)).astype(np.float16)
        vn = rng.standard_normal((B, H, 1, D)).astype(np.float16)
        st, lens_next = oracle.kv_append_q4r(st, kn, vn, lens, group, R)
        gpu_lib.gqa_kv_append_q4r(torch.from_numpy(kn).cuda(), torch.from_numpy(vn).cuda(), dev["k_codes"],
                                  dev["k_scales"], dev["k_biases"], dev["v_codes"], dev["v_scales"], dev["v_biases"],
                                  dev["k_res"], dev["v_res"], group, lens_d, new_d)
        lens = lens_next
        lens_d, new_d = new_d, lens_d
        q = torch.from_numpy(rng.standard_normal((B, Hq, 1, D)).astype(np.float16)).cuda()
        got = _decode(gpu_lib, dev, q, lens.tolist(), group, ws)
        assert_close(got, oracle.q4r_attend(q.cpu(), st, lens, group, R), TOL_16, "grow step %d lens=%s"
                     % (step, lens.tolist()))
    _assert_state(dev, st, "after 30 appends")


def test_decode_q4_workload_geometry_16k(gpu_lib):
    w = W.by_name("q4_decode")
    rng = np.random.default_rng(31)
    R, n = 128, 16300
    Hq, H, D, group = w.Hq, w.Hkv, w.D, w.group
    s_cap = 16384
    # the 4-bit rows from the workload's own cache, the residual from fresh float16 rows
    inp = W.q4_inputs(w, s_cap, 0)
    q = inp["q"]
    n_q, n_r = oracle.q4r_split(n, R)
    st = {key: inp[key].numpy() for key in ("k_codes", "k_scales", "k_biases", "v_codes", "v_scales", "v_biases")}
    st["k_res"] = rng.standard_normal((1, H, R, D)).astype(np.float16)
    st["v_res"] = rng.standard_normal((1, H, R, D)).astype(np.float16)
    dev = _to_dev(st)
    note("q4r decode %d/%d heads, D=%d, n=%d (n_q=%d n_r=%d)" % (Hq, H, D, n, n_q, n_r))
    got = _decode(gpu_lib, dev, q.cuda(), [n], group, gpu_lib.make_q4r_workspace(1, Hq, H, D, s_cap, R))
    assert_close(got, oracle.q4r_attend(q, st, [n], group, R), TOL_16, "q4r 16k")


def _prefill(gpu_lib, dev, q, Tk, group, scale=None):
    out = torch.empty_like(q)
    gpu_lib.gqa_prefill_causal_q4r(q, dev["k_codes"], dev["k_scales"], dev["k_biases"], dev["v_codes"],
                                   dev["v_scales"], dev["v_biases"], dev["k_res"], dev["v_res"], out, group, Tk,
                                   scale=scale)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("D,group,R,Tk,Tq", [(64, 32, 64, 229, 100), (128, 64, 128, 700, 700), (128, 128, 64, 640, 77),
                                             (64, 64, 192, 1000, 1), (128, 32, 64, 385, 385)])
def test_prefill_chunk_over_q4r_cache(gpu_lib, D, group, R, Tk, Tq):
    rng = np.random.default_rng(D + group + R + Tk + Tq)
    B, Hq, H, s_cap = 2, 4, 2, Tk + 64
    st = _grown_state(rng, B, H, s_cap, D, group, R, [Tk, Tk])
    dev = _to_dev(st)
    q = torch.from_numpy((rng.standard_normal((B, Hq, Tq, D)) * 0.8).astype(np.float16)).cuda()
    n_q, n_r = oracle.q4r_split(Tk, R)
    note("q4r prefill D=%d group=%d R=%d Tk=%d Tq=%d (n_q=%d n_r=%d)" % (D, group, R, Tk, Tq, n_q, n_r))
    got = _prefill(gpu_lib, dev, q, Tk, group)
    want = oracle.q4r_attend(q.cpu(), st, [Tk, Tk], group, R, causal=True)
    assert_close(got, want, TOL_16, "q4r prefill Tk=%d Tq=%d" % (Tk, Tq))


def test_prefill_without_4bit_rows_is_the_f16_prefill(gpu_lib):
    rng = np.random.default_rng(41)
    B, Hq, H, D, group, R = 1, 4, 2, 128, 64, 256
    Tk, Tq = 200, 120  # Tk < R: every token in the residual
    st = _grown_state(rng, B, H, 512, D, group, R, [Tk])
    dev = _to_dev(st)
    q = torch.from_numpy(rng.standard_normal((B, Hq, Tq, D)).astype(np.float16)).cuda()
    note("q4r prefill == f16 prefill Tk=%d Tq=%d" % (Tk, Tq))
    got = _prefill(gpu_lib, dev, q, Tk, group)
    ref = torch.empty_like(q)
    gpu_lib.gqa_prefill_causal(q, dev["k_res"], dev["v_res"], ref, gpu_lib.make_prefill_workspace(B, Hq, H, D, Tq, Tk),
                               Tk)
    torch.cuda.synchronize()
    assert_close(got, oracle.q4r_attend(q.cpu(), st, [Tk], group, R, causal=True), TOL_16, "q4r prefill no 4-bit")
    assert torch.equal(got, ref)


def test_prefill_chunk_at_3841_of_4097(gpu_lib):
    # the pages' chunked-prefill case (256 queries after 3841 tokens) on
    # the 0.5B geometry, over a 4-bit cache with a 128-row residual
    w = W.by_name("prefill_0p5b")
    rng = np.random.default_rng(43)
    Hq, H, D, group, R = w.Hq, w.Hkv, w.D, 32, 128
    Tk, Tq = 4097, 256
    st = _grown_state(rng, 1, H, Tk, D, group, R, [Tk])
    dev = _to_dev(st)
    q = torch.from_numpy(rng.standard_normal((1, Hq, Tq, D)).astype(np.float16)).cuda()
    note("q4r prefill chunk Tk=%d Tq=%d heads %d/%d D=%d" % (Tk, Tq, Hq, H, D))
    got = _prefill(gpu_lib, dev, q, Tk, group)
    assert_close(got, oracle.q4r_attend(q.cpu(), st, [Tk], group, R, causal=True), TOL_16, "q4r chunk at 3841")
