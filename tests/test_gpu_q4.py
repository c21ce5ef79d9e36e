"""GPU parity of the 4-bit quantized decode path.

* The dequant hook (s*c + b per element, rounded once: the values the 4-bit
  attention is defined over) is bit-identical to the oracle's unpack +
  dequant, on random codes with the edge codes 0 and 15 and zero scales, and
  on the encoded workload cache.  The attention kernel does not call it.
* The attention kernel's own unpack and dequant, bit for bit: with one
  visible key the output is the oracle's dequantized value row 0 rounded to
  f16; with one key whose weight is exactly 1 (every other weight
  underflows to 0; single split, so no partial is merged) the output is
  that key's dequantized value row rounded to f16.  The dominant key is
  picked by one K code per row, so a wrong K nibble slot picks another row;
  the V rows carry random codes, so a wrong V nibble or row slot changes the
  output.  Every (head dim, group) pair, several head geometries.
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


# ---------------------------------------------------------------------------
# The kernel's own unpack and dequant, bit for bit
# ---------------------------------------------------------------------------
Q4_PAIRS = [(128, 64), (128, 32), (128, 128), (64, 64), (64, 32)]


def _f16(x):
    return torch.from_numpy(np.ascontiguousarray(x))


def _q4_random_v(rng, Hkv, s_cap, D, group):
    """V codes with every code value, scales in [2^-9, 2) (so s/16 is an exact
    f16 for the rows facing high nibbles) and biases of both signs."""
    codes = rng.integers(0, 16, size=(1, Hkv, s_cap, D), dtype=np.uint8)
    codes[..., 0] = 0
    codes[..., 1] = 15
    scales = np.exp2(rng.uniform(-9, 1, size=(1, Hkv, s_cap, D // group))).astype(np.float16)
    biases = (rng.standard_normal((1, Hkv, s_cap, D // group)) * 2).astype(np.float16)
    return gen.q4_pack_codes(codes), scales, biases


def _run_q4_raw(gqa, q, kc, ks, kb, vc, vs, vb, group, kv_len, scale):
    B, Hq, _, D = q.shape
    Hkv, s_cap = kc.shape[1], kc.shape[2]
    ws = gqa.make_workspace(B, Hq, Hkv, D, s_cap)
    g = Guarded(q.shape, torch.float16)
    d = lambda a: _f16(a).cuda()  # noqa: E731
    gqa.gqa_decode_attend_q4(q.cuda(), d(kc), d(ks), d(kb), d(vc), d(vs), d(vb), g.t, group, kv_len, ws, scale=scale)
    torch.cuda.synchronize()
    g.check()
    return g.t.cpu()


@pytest.mark.parametrize("D,group", Q4_PAIRS)
@pytest.mark.parametrize("Hq,Hkv", [(64, 8), (14, 2), (256, 256)])
def test_q4_kernel_one_key_bit_exact(gpu_lib, D, group, Hq, Hkv):
    """kv_len = 1: the output is V row 0 dequantized (s*c + b, one fp32
    rounding) and rounded to f16, bit for bit, for every query head."""
    rng = np.random.default_rng(D * 1000 + group + Hq)
    s_cap = 40
    kc = rng.integers(0, 256, size=(1, Hkv, s_cap, D // 2), dtype=np.uint8)
    ks = rng.standard_normal((1, Hkv, s_cap, D // group)).astype(np.float16)
    kb = rng.standard_normal((1, Hkv, s_cap, D // group)).astype(np.float16)
    vc, vs, vb = _q4_random_v(rng, Hkv, s_cap, D, group)
    # rows past the valid one hold NaN scales and biases: never read
    for a in (ks, kb, vs, vb):
        a[:, :, 1:] = np.nan
    q = torch.from_numpy(rng.standard_normal((1, Hq, 1, D)).astype(np.float16))
    note("q4 one key D=%d group=%d Hq=%d Hkv=%d" % (D, group, Hq, Hkv))
    got = _run_q4_raw(gpu_lib, q, kc, ks, kb, vc, vs, vb, group, 1, 1.0 / np.sqrt(D))
    v0 = oracle.q4_dequant(vc[:, :, :1], vs[:, :, :1], vb[:, :, :1], group)  # [1,Hkv,1,D] float32
    want = np.repeat(v0, Hq // Hkv, axis=1).astype(np.float16)
    assert np.array_equal(got.numpy().view(np.uint16), want.view(np.uint16))


def _dominant_case(rng, Hq, Hkv, D, group, s_cap, kv_len):
    """K codes: row r has code 15 in dimension owner[r] (at most one row owns
    a dimension) and 0 elsewhere, scale 1, bias 0.  Query head h is 4.0 in
    one dimension d(h) and 0 elsewhere, so with scale 4 its score is 240 for
    the row owning d(h) and 0 for every other row: a log2 gap of ~346, so
    that row's weight is exactly 1 and every other weight is exactly 0."""
    G = Hq // Hkv
    kcodes = np.zeros((1, Hkv, s_cap, D), np.uint8)
    dims = np.zeros((Hkv, G), np.int64)
    rows = np.zeros((Hkv, G), np.int64)
    for g in range(Hkv):
        n_own = min(kv_len, D)
        own_rows = rng.choice(kv_len, size=n_own, replace=False)
        own_dims = rng.choice(D, size=n_own, replace=False)
        kcodes[0, g, own_rows, own_dims] = 15
        pick = rng.integers(0, n_own, size=G)
        dims[g] = own_dims[pick]
        rows[g] = own_rows[pick]
    q = np.zeros((1, Hq, 1, D), np.float16)
    for h in range(Hq):
        q[0, h, 0, dims[h // G, h % G]] = 4.0
    ks = np.ones((1, Hkv, s_cap, D // group), np.float16)
    kb = np.zeros((1, Hkv, s_cap, D // group), np.float16)
    ks[:, :, kv_len:] = np.nan
    return q, gen.q4_pack_codes(kcodes), ks, kb, rows


@pytest.mark.parametrize("D,group", Q4_PAIRS)
@pytest.mark.parametrize("Hq,Hkv,s_cap", [(64, 8, 16), (14, 2, 16), (256, 256, 300), (2048, 256, 97)])
def test_q4_kernel_dominant_key_bit_exact(gpu_lib, D, group, Hq, Hkv, s_cap):
    """One key per query head has weight exactly 1: the output is that key's
    dequantized value row rounded to f16, bit for bit.  Every case runs as a
    single split (no partial merged); the last two geometries span several
    32-row steps over several waves."""
    if Hq == 2048 and D == 64:
        pytest.skip("one head dim suffices for the widest geometry")
    rng = np.random.default_rng(D * 7 + group + Hq + s_cap)
    kv_len = s_cap if s_cap <= 16 else s_cap - 3
    q, kc, ks, kb, rows = _dominant_case(rng, Hq, Hkv, D, group, s_cap, kv_len)
    vc, vs, vb = _q4_random_v(rng, Hkv, s_cap, D, group)
    qt = torch.from_numpy(q)
    note("q4 dominant key D=%d group=%d Hq=%d Hkv=%d s_cap=%d kv_len=%d" % (D, group, Hq, Hkv, s_cap, kv_len))
    got = _run_q4_raw(gpu_lib, qt, kc, ks, kb, vc, vs, vb, group, kv_len, 4.0)
    vdq = oracle.q4_dequant(vc, vs, vb, group)  # [1,Hkv,s_cap,D]
    G = Hq // Hkv
    want = np.stack([vdq[0, h // G, rows[h // G, h % G]] for h in range(Hq)])[None, :, None, :].astype(np.float16)
    # the premise holds in the oracle: attention equals that row (other weights < 1e-100)
    ref = oracle.q4_attend(qt, kc, ks, kb, vc, vs, vb, group, kv_lens=kv_len, scale=4.0)
    assert np.abs(ref - want.astype(np.float64)).max() <= np.abs(want.astype(np.float64)).max() * 2.0 ** -10
    assert np.array_equal(got.numpy().view(np.uint16), want.view(np.uint16))
