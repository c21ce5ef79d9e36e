"""GPU parity of the causal prefill entry point against the fp64 oracle.

Workloads: Qwen2.5-0.5B heads (14 query / 2 KV heads, dim 64), bf16, T in
{513, 2049, 4097} with Tq = Tk = T, and the chunk of 256 queries at offset
3841 into 4097 keys (queries aligned to the end of the keys, "Cause and
workaround" point 2 of the Fornace prefill page).  T = 513 and 2049 and the
chunk are compared on every output; T = 4097 on every output too (the oracle
takes a few seconds on all cores).  Small shapes cover ragged tiles, Tq < Tk,
D = 128, f16, several group sizes and B > 1.  Bound: max-abs 2e-2 (bf16/f16
outputs); every 16-bit comparison also reports the per-row error in units
in the last place at the row's largest |output|.  Row 0 of a square prefill
sees one key and must equal that key's value row exactly; the chunk must
match the tail of the full prefill within the bound.  Runs on two streams at
once, each with its own workspace, must equal a serial run bit for bit.

Seam cases: long rows are split into chunks of 64-key tiles merged through
the workspace, and on plain N(0,1) inputs one key more or less at a chunk
seam moves long rows by under the bound.  The seam cases plant, on each
side of every tile boundary, a key that dominates one (row, head) pair
(workloads.gen.seam_planted), so a key lost or doubled at any boundary
fails the bound (tests/test_check_power.py shows the check rejecting
exactly those mistakes on the oracle's output); their per-row error must
also stay within 2 ulps.
"""

import numpy as np
import pytest
import torch

import oracle
from tests.helpers import Guarded, assert_close, assert_workspace_ready, note
from workloads import configs as W
from workloads import gen

pytestmark = pytest.mark.gpu




def prefill_ws(gqa, q, k, Tk=None):
    B, Hq, Tq, D = q.shape
    Tk = k.shape[2] if Tk is None else Tk
    return gqa.make_prefill_workspace(B, Hq, k.shape[1], D, Tq, Tk)


def run_prefill(gqa, q, k, v, Tk=None, scale=None):
    g = Guarded(q.shape, q.dtype)
    ws = prefill_ws(gqa, q, k, Tk)
    gqa.gqa_prefill_causal(q.cuda(), k.cuda(), v.cuda(), g.t, ws, Tk=Tk, scale=scale)
    torch.cuda.synchronize()
    g.check()
    return g.t


@pytest.mark.parametrize("T", [513, 2049, 4097])
def test_prefill_0p5b(gpu_lib, T):
    w = W.by_name("prefill_0p5b")
    q, k, v = W.prefill_inputs(w, T)
    note("prefill_0p5b T=%d" % T)
    got = run_prefill(gpu_lib, q, k, v)
    want = oracle.attend(q, k, v, causal=True, scale=w.scale())
    assert_close(got, want, 2e-2, "prefill T=%d" % T)
    # row 0 sees only key 0
    g = got.cpu()
    assert torch.equal(g[0, :, 0], v[0, :, 0].repeat_interleave(w.G, dim=0))


def test_prefill_long_d128(gpu_lib):
    # T = 8193 at D = 128: 65 row blocks, the longest split into more key
    # chunks than any benchmark size, and a one-row last block
    rng = np.random.default_rng(8193)
    T, Hq, Hkv, D = 8193, 2, 1, 128
    q = torch.from_numpy(rng.standard_normal((1, Hq, T, D), dtype=np.float32)).to(torch.bfloat16)
    k = torch.from_numpy(rng.standard_normal((1, Hkv, T, D), dtype=np.float32)).to(torch.bfloat16)
    v = torch.from_numpy(rng.standard_normal((1, Hkv, T, D), dtype=np.float32)).to(torch.bfloat16)
    note("prefill long T=%d D=%d" % (T, D))
    got = run_prefill(gpu_lib, q, k, v)
    assert_close(got, oracle.attend(q, k, v, causal=True), 2e-2, "prefill T=%d" % T)


def test_prefill_chunk_at_offset(gpu_lib):
    w = W.by_name("prefill_0p5b")
    c = W.PREFILL_CHUNK
    q, k, v = W.prefill_inputs(w, c["Tk"])
    qc = q[:, :, c["offset"]:].contiguous()
    note("prefill chunk Tq=%d Tk=%d" % (c["Tq"], c["Tk"]))
    got = run_prefill(gpu_lib, qc, k, v)
    want = oracle.attend(qc, k, v, causal=True, scale=w.scale())
    assert_close(got, want, 2e-2, "chunk")
    full = run_prefill(gpu_lib, q, k, v)
    diff = (full[:, :, c["offset"]:].float() - got.float()).abs().max().item()
    note("  chunk vs tail of full prefill: %.3e" % diff)
    assert diff <= 2e-2


CASES = [
    # B, Hq, Hkv, D, Tq, Tk, s_cap
    (1, 1, 1, 64, 1, 1, 1),
    (1, 2, 1, 64, 1, 300, 300),
    (1, 14, 2, 64, 5, 5, 9),
    (2, 4, 2, 64, 127, 127, 130),
    (1, 4, 4, 64, 128, 128, 128),
    (1, 7, 1, 64, 129, 200, 256),
    (1, 8, 8, 128, 200, 200, 200),
    (2, 12, 2, 128, 65, 333, 400),
    (1, 16, 1, 128, 257, 257, 257),
    (1, 14, 2, 64, 64, 1000, 1000),
    (1, 14, 2, 64, 64, 1100, 1100),   # 18 key tiles: split into key chunks and merged
    (1, 4, 2, 64, 3, 2500, 2600),     # 40 key tiles: four key chunks merged
    (2, 4, 1, 128, 130, 1300, 1300),  # D = 128, two row blocks of 21 key tiles, each split into chunks
    (1, 4, 2, 64, 1057, 1057, 1057),  # last row block: 33 rows (waves with 32, 1, 0, 0 rows), 17 key tiles in chunks
    (1, 4, 1, 128, 1057, 1057, 1057),  # the same at D = 128
]


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
def test_prefill_small_ragged(gpu_lib, dtype):
    rng = np.random.default_rng(17 if dtype == torch.bfloat16 else 18)
    for B, Hq, Hkv, D, Tq, Tk, s_cap in CASES:
        q = torch.from_numpy(rng.standard_normal((B, Hq, Tq, D), dtype=np.float32)).to(dtype)
        k = torch.from_numpy(rng.standard_normal((B, Hkv, s_cap, D), dtype=np.float32)).to(dtype)
        v = torch.from_numpy(rng.standard_normal((B, Hkv, s_cap, D), dtype=np.float32)).to(dtype)
        k[:, :, Tk:] = float("nan")
        v[:, :, Tk:] = float("nan")
        note("prefill %s B=%d Hq=%d Hkv=%d D=%d Tq=%d Tk=%d s_cap=%d" % (dtype, B, Hq, Hkv, D, Tq, Tk, s_cap))
        got = run_prefill(gpu_lib, q, k, v, Tk=Tk)
        want = oracle.attend(q, k, v, kv_lens=Tk, causal=True)
        assert_close(got, want, 2e-2, "Tq=%d Tk=%d" % (Tq, Tk))


@pytest.mark.parametrize("div", [20.0, 50.0, -20.0])
def test_prefill_large_scores(gpu_lib, div):
    # Scores that grow along the keys: at scale 1/8 they rise by 369/div
    # log2 units per 64-key tile.  div=20: each tile outgrows the reference
    # maximum by far more than 2^8, so it is raised every tile.  div=50: ~7.4
    # units per tile, so a lane's probability sum passes the test limit
    # (the tile is formed again) while the maximum is raised only every
    # other tile.  div=-20: falling scores, the reference from the first
    # tile serves every later one.
    T, D = 300, 64
    q = torch.ones(1, 2, T, D) * 0.5
    k = (torch.arange(T, dtype=torch.float32)[:, None] / div).expand(T, D).reshape(1, 1, T, D).contiguous()
    v = torch.randn(1, 1, T, D)
    q, k, v = (t.to(torch.bfloat16) for t in (q, k, v))
    got = run_prefill(gpu_lib, q, k, v)
    want = oracle.attend(q, k, v, causal=True)
    assert_close(got, want, 2e-2, "large scores")


@pytest.mark.parametrize("T", [2049, 4097])
def test_prefill_deterministic(gpu_lib, T):
    # which key chunk of a split row block arrives last (and merges) varies
    # from run to run; the result must not: ten runs, half of them on fresh
    # workspaces, are bit-identical
    w = W.by_name("prefill_0p5b")
    q, k, v = (t.cuda() for t in W.prefill_inputs(w, T))
    ws = prefill_ws(gpu_lib, q, k)
    outs = []
    for r in range(10):
        o = torch.empty_like(q)
        gpu_lib.gqa_prefill_causal(q, k, v, o, ws if r % 2 else prefill_ws(gpu_lib, q, k))
        outs.append(o)
    torch.cuda.synchronize()
    for r in range(1, 10):
        assert torch.equal(outs[r], outs[0]), "run %d differs" % r


def test_prefill_concurrent_streams_separate_workspaces(gpu_lib):
    # The full prefill at T=4097 and the 256-query chunk at offset 3841 run
    # concurrently on two streams (default priority), each with its own
    # workspace, three calls per stream and round, five rounds.  The chunk
    # merge takes a ticket and never waits, so competing launches only change
    # which chunk merges; every output must equal a serial run bit for bit.
    w = W.by_name("prefill_0p5b")
    q, k, v = (t.cuda() for t in W.prefill_inputs(w, 4097))
    qc = q[:, :, 4097 - 256:].contiguous()
    ws_full, ws_chunk = prefill_ws(gpu_lib, q, k), prefill_ws(gpu_lib, qc, k)
    want_full, want_chunk = torch.empty_like(q), torch.empty_like(qc)
    gpu_lib.gqa_prefill_causal(q, k, v, want_full, ws_full)
    gpu_lib.gqa_prefill_causal(qc, k, v, want_chunk, ws_chunk)
    outs_full = [torch.empty_like(q) for _ in range(3)]
    outs_chunk = [torch.empty_like(qc) for _ in range(3)]
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    for r in range(5):
        note("concurrent prefill round %d" % r)
        with torch.cuda.stream(s1):
            for o in outs_full:
                gpu_lib.gqa_prefill_causal(q, k, v, o, ws_full)
        with torch.cuda.stream(s2):
            for o in outs_chunk:
                gpu_lib.gqa_prefill_causal(qc, k, v, o, ws_chunk)
        torch.cuda.synchronize()
        for i, o in enumerate(outs_full):
            assert torch.equal(o, want_full), "round %d full call %d" % (r, i)
        for i, o in enumerate(outs_chunk):
            assert torch.equal(o, want_chunk), "round %d chunk call %d" % (r, i)
    assert_workspace_ready(ws_full, "full prefill workspace after the concurrent rounds")
    assert_workspace_ready(ws_chunk, "chunk workspace after the concurrent rounds")


def test_prefill_workspace_reuse(gpu_lib):
    # The key chunks of a long row block meet through the workspace: the last
    # to arrive merges and returns the slots and the counter to zero.  Many
    # calls in a row on one workspace, with changing inputs and lengths, must
    # each match a fresh run, and leave the workspace ready for the next call.
    # The workspace is sized for the largest of the calls (the size is not
    # monotone in the lengths: a shorter prompt may be cut into more chunks).
    w = W.by_name("prefill_0p5b")
    q0, k0, v0 = (t.cuda() for t in W.prefill_inputs(w, 2049))
    Hq, Hkv, D = q0.shape[1], k0.shape[1], q0.shape[3]
    rng = np.random.default_rng(29)
    sizes = []
    for it in range(12):
        Tq = int(rng.integers(1, 2049))
        sizes.append((Tq, int(rng.integers(Tq, 2050))))
    ws = torch.zeros(max(gpu_lib.gqa_prefill_workspace_bytes(1, Hq, Hkv, D, Tq, Tk) for Tq, Tk in sizes),
                     dtype=torch.uint8, device="cuda")
    for it, (Tq, Tk) in enumerate(sizes):
        q = (q0[:, :, :Tq] * (1 + 0.1 * it)).contiguous()
        k = (k0 * (1 - 0.05 * it)).contiguous()
        note("prefill reuse it=%d Tq=%d Tk=%d" % (it, Tq, Tk))
        got = torch.empty_like(q)
        gpu_lib.gqa_prefill_causal(q, k, v0, got, ws, Tk=Tk)
        ref = torch.empty_like(q)
        gpu_lib.gqa_prefill_causal(q, k, v0, ref, prefill_ws(gpu_lib, q, k, Tk), Tk=Tk)
        torch.cuda.synchronize()
        assert torch.equal(got, ref), "it=%d" % it
        assert_workspace_ready(ws, "it=%d" % it)


def test_workspace_shared_by_decode_and_prefill(gpu_lib):
    # Decode and prefill calls of changing sizes take turns on one
    # workspace; each must match a run on a fresh workspace bit for bit.
    w = W.by_name("prefill_0p5b")
    q0, k0, v0 = (t.cuda() for t in W.prefill_inputs(w, 2049))
    Hq, Hkv, D = q0.shape[1], k0.shape[1], q0.shape[3]
    calls = [(2049, 2049, 4), (300, 1900, 1), (1500, 1500, 3), (77, 2049, 2)]
    ws = torch.zeros(max([gpu_lib.gqa_prefill_workspace_bytes(1, Hq, Hkv, D, Tq, Tk) for Tq, Tk, _ in calls] +
                         [gpu_lib.gqa_decode_workspace_bytes(4, Hq, Hkv, D, 2049)]), dtype=torch.uint8, device="cuda")
    gen = torch.Generator().manual_seed(43)
    for it, (Tq, Tk, B) in enumerate(calls):
        note("shared workspace it=%d prefill Tq=%d Tk=%d, decode B=%d" % (it, Tq, Tk, B))
        q = q0[:, :, :Tq].contiguous()
        got = torch.empty_like(q)
        gpu_lib.gqa_prefill_causal(q, k0, v0, got, ws, Tk=Tk)
        ref = torch.empty_like(q)
        gpu_lib.gqa_prefill_causal(q, k0, v0, ref, prefill_ws(gpu_lib, q, k0, Tk), Tk=Tk)
        qd = torch.randn(B, Hq, 1, D, generator=gen).to(torch.bfloat16).cuda()
        kd = torch.randn(B, Hkv, 2049, D, generator=gen).to(torch.bfloat16).cuda()
        vd = torch.randn(B, Hkv, 2049, D, generator=gen).to(torch.bfloat16).cuda()
        got_d = torch.empty_like(qd)
        gpu_lib.gqa_decode_attend(qd, kd, vd, got_d, Tk, ws)
        ref_d = torch.empty_like(qd)
        gpu_lib.gqa_decode_attend(qd, kd, vd, ref_d, Tk, gpu_lib.make_workspace(B, Hq, Hkv, D, 2049))
        torch.cuda.synchronize()
        assert torch.equal(got, ref), "prefill it=%d" % it
        assert torch.equal(got_d, ref_d), "decode it=%d" % it
        assert_workspace_ready(ws, "it=%d" % it)


@pytest.mark.parametrize("scale", [-0.125, 0.0, 0.9])
def test_prefill_scale_sign(gpu_lib, scale):
    # the running maximum is kept over sign(scale) * q.k: a negative scale
    # takes the minimum raw score, a zero scale gives the plain mean of the
    # visible value rows, a large one spreads the exponents far apart
    rng = np.random.default_rng(23)
    B, Hq, Hkv, D, Tq, Tk = 1, 4, 2, 64, 150, 260
    q = torch.from_numpy(rng.standard_normal((B, Hq, Tq, D), dtype=np.float32)).to(torch.bfloat16)
    k = torch.from_numpy(rng.standard_normal((B, Hkv, Tk, D), dtype=np.float32)).to(torch.bfloat16)
    v = torch.from_numpy(rng.standard_normal((B, Hkv, Tk, D), dtype=np.float32)).to(torch.bfloat16)
    note("prefill scale=%g" % scale)
    got = run_prefill(gpu_lib, q, k, v, scale=scale)
    want = oracle.attend(q, k, v, causal=True, scale=scale)
    assert_close(got, want, 2e-2, "scale=%g" % scale)


SEAM_CASES = [
    # B, Hq, Hkv, D, Tq, Tk, s_cap, dtype
    (1, 14, 2, 64, 4097, 4097, 4097, torch.bfloat16),   # the T=4097 workload geometry
    (1, 14, 2, 64, 256, 4097, 4097, torch.bfloat16),    # the 256-query chunk at offset 3841
    (1, 4, 2, 64, 3, 2500, 2600, torch.bfloat16),       # three rows, 40 key tiles in chunks
    (2, 4, 1, 128, 130, 1300, 1300, torch.float16),     # D = 128
    (1, 4, 2, 64, 1057, 1057, 1057, torch.float16),     # ragged last row block
]


@pytest.mark.parametrize("case", range(len(SEAM_CASES)))
def test_prefill_seams_planted(gpu_lib, case):
    B, Hq, Hkv, D, Tq, Tk, s_cap, dtype = SEAM_CASES[case]
    dt = "bf16" if dtype == torch.bfloat16 else "f16"
    q, k, v, keys = gen.seam_planted(B, Hq, Hkv, D, Tq, Tk, dt, seed=case, s_cap=s_cap)
    note("prefill seams planted B=%d Hq=%d Hkv=%d D=%d Tq=%d Tk=%d (%d planted keys)" % (B, Hq, Hkv, D, Tq, Tk,
                                                                                       len(keys)))
    got = run_prefill(gpu_lib, q, k, v, Tk=Tk)
    want = oracle.attend(q, k, v, kv_lens=Tk, causal=True)
    assert_close(got, want, 2e-2, "seams Tq=%d Tk=%d" % (Tq, Tk), max_ulps=2.0)
