"""GPU parity of the split-K decode entry points against the fp64 oracle.

Covers the single-token decode workloads (Qwen2.5-0.5B heads at KV length
128; Qwen2.5-7B heads swept 128..4096, fp32, the configuration the benchmark
times), batched decode with per-request lengths (Qwen3-4B heads, bf16,
B = 1, 2, 4, 8 in a 4096-row cache), and small ragged shapes for every dtype,
head dim and several group sizes.  Also: NaN-filled cache rows past the
valid length, guard bands around the output, run-to-run bit equality with a
reused workspace, and batched output bit-identical to per-request calls.
Bounds: max-abs 2e-5 for fp32 outputs, 2e-2 for bf16/f16.
"""

import numpy as np
import pytest
import torch

import oracle
from tests.helpers import Guarded, assert_close, assert_workspace_ready, note, tol_for
from workloads import configs as W

pytestmark = pytest.mark.gpu

DT = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


def run_decode(gqa, q, k, v, kv_len, scale=None):
    B, Hq, _, D = q.shape
    Hkv, s_cap = k.shape[1], k.shape[2]
    ws = gqa.make_workspace(B, Hq, Hkv, D, s_cap)
    g = Guarded(q.shape, q.dtype)
    gqa.gqa_decode_attend(q.cuda(), k.cuda(), v.cuda(), g.t, kv_len, ws, scale=scale)
    torch.cuda.synchronize()
    g.check()
    return g.t


def test_decode_0p5b_s128(gpu_lib):
    w = W.by_name("decode_0p5b")
    q, k, v = W.decode_inputs(w, 128, 0)
    note("decode_0p5b S=128")
    got = run_decode(gpu_lib, q, k, v, 128)
    want = oracle.attend(q, k, v, scale=w.scale())
    assert_close(got, want, 2e-5, "decode_0p5b")


@pytest.mark.parametrize("S", [128, 256, 512, 1024, 2048, 4096])
def test_decode_7b_sweep(gpu_lib, S):
    w = W.by_name("decode_7b")
    for layer in (0, 27):
        q, k, v = W.decode_inputs(w, S, layer)
        note("decode_7b S=%d layer=%d" % (S, layer))
        got = run_decode(gpu_lib, q, k, v, S)
        want = oracle.attend(q, k, v, scale=w.scale())
        assert_close(got, want, 2e-5, "decode_7b S=%d layer %d" % (S, layer))


GEOMS = [(1, 1), (4, 4), (8, 2), (12, 2), (14, 2), (32, 8), (16, 1), (10, 2), (28, 4)]
LENS = [1, 5, 31, 32, 33, 100, 777]


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("D", [64, 128])
def test_decode_small_ragged(gpu_lib, dtype, D):
    rng = np.random.default_rng({"f32": 0, "bf16": 1, "f16": 2}[dtype] * 1000 + D)
    for Hq, Hkv in GEOMS:
        for n in LENS:
            s_cap = n + int(rng.integers(0, 40))
            B = 1 + int(rng.integers(0, 2))
            q = torch.from_numpy(rng.standard_normal((B, Hq, 1, D), dtype=np.float32)).to(DT[dtype])
            k = torch.from_numpy(rng.standard_normal((B, Hkv, s_cap, D), dtype=np.float32)).to(DT[dtype])
            v = torch.from_numpy(rng.standard_normal((B, Hkv, s_cap, D), dtype=np.float32)).to(DT[dtype])
            k[:, :, n:] = float("nan")
            v[:, :, n:] = float("nan")
            note("decode %s D=%d Hq=%d Hkv=%d n=%d s_cap=%d B=%d" % (dtype, D, Hq, Hkv, n, s_cap, B))
            got = run_decode(gpu_lib, q, k, v, n)
            want = oracle.attend(q, k, v, kv_lens=n)
            assert_close(got, want, tol_for(DT[dtype]), "n=%d Hq=%d Hkv=%d" % (n, Hq, Hkv))


def test_decode_long_context(gpu_lib):
    # 65537 keys: the split plan's cap on splits makes every split stream
    # many chunks; the length is one past a multiple of every chunk size
    rng = np.random.default_rng(65537)
    Hq, Hkv, D, n, s_cap = 16, 4, 128, 65537, 65600
    q = torch.from_numpy(rng.standard_normal((1, Hq, 1, D), dtype=np.float32)).to(torch.bfloat16)
    k = torch.from_numpy(rng.standard_normal((1, Hkv, s_cap, D), dtype=np.float32)).to(torch.bfloat16)
    v = torch.from_numpy(rng.standard_normal((1, Hkv, s_cap, D), dtype=np.float32)).to(torch.bfloat16)
    k[:, :, n:] = float("nan")
    v[:, :, n:] = float("nan")
    note("decode bf16 long context n=%d" % n)
    got = run_decode(gpu_lib, q, k, v, n)
    assert_close(got, oracle.attend(q, k, v, kv_lens=n), 2e-2, "long context")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("scale", [-0.2, 0.0, 2.0])
def test_decode_scale_sign(gpu_lib, dtype, scale):
    # negative: the maximum is the smallest raw score; zero: the plain mean of
    # the value rows; 2.0: exponents far apart, so the reference maximum is
    # raised often along the keys
    rng = np.random.default_rng(31)
    B, Hq, Hkv, D, n = 2, 14, 2, 128, 1000
    q = torch.from_numpy(rng.standard_normal((B, Hq, 1, D), dtype=np.float32)).to(DT[dtype])
    k = torch.from_numpy(rng.standard_normal((B, Hkv, n, D), dtype=np.float32)).to(DT[dtype])
    v = torch.from_numpy(rng.standard_normal((B, Hkv, n, D), dtype=np.float32)).to(DT[dtype])
    note("decode %s scale=%g" % (dtype, scale))
    got = run_decode(gpu_lib, q, k, v, n, scale=scale)
    assert_close(got, oracle.attend(q, k, v, kv_lens=n, scale=scale), tol_for(DT[dtype]), "scale=%g" % scale)


def test_decode_single_key_is_value_row(gpu_lib):
    q = torch.randn(1, 28, 1, 128)
    k = torch.randn(1, 4, 64, 128)
    v = torch.randn(1, 4, 64, 128)
    got = run_decode(gpu_lib, q, k, v, 1).cpu()
    want = v[:, :, :1].repeat_interleave(7, dim=1)
    assert torch.equal(got, want)


def test_decode_deterministic_with_reused_workspace(gpu_lib):
    w = W.by_name("decode_7b")
    q, k, v = (t.cuda() for t in W.decode_inputs(w, 4096, 3))
    ws = gpu_lib.make_workspace(1, 28, 4, 128, 4096)
    outs = []
    for _ in range(3):
        o = torch.empty_like(q)
        gpu_lib.gqa_decode_attend(q, k, v, o, 4096, ws)
        outs.append(o)
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[0], outs[2])


def test_decode_workspace_shared_across_batch_sizes(gpu_lib):
    # One workspace serves calls of different batch sizes in any order (the
    # layout of the partials changes with the batch): each call must match a
    # run on a fresh workspace bit for bit and leave the workspace ready for
    # the next call, since published words are recognised by a tag bit.
    Hq, Hkv, D, S = 28, 4, 128, 1024
    ws = gpu_lib.make_workspace(8, Hq, Hkv, D, S)
    gen = torch.Generator().manual_seed(41)
    for it, B in enumerate([8, 1, 5, 2, 8, 3]):
        n = S - 37 * it
        q = torch.randn(B, Hq, 1, D, generator=gen).cuda()
        k = torch.randn(B, Hkv, S, D, generator=gen).cuda()
        v = torch.randn(B, Hkv, S, D, generator=gen).cuda()
        note("decode shared workspace it=%d B=%d kv_len=%d" % (it, B, n))
        got = torch.empty_like(q)
        gpu_lib.gqa_decode_attend(q, k, v, got, n, ws)
        ref = torch.empty_like(q)
        gpu_lib.gqa_decode_attend(q, k, v, ref, n, gpu_lib.make_workspace(B, Hq, Hkv, D, S))
        torch.cuda.synchronize()
        assert torch.equal(got, ref), "it=%d B=%d" % (it, B)
        assert_workspace_ready(ws, "it=%d" % it)


def test_binding_checks_workspace_and_devices(gpu_lib):
    # a host workspace or a host tensor is refused before anything is launched;
    # a workspace of another element type is measured in bytes
    q = torch.randn(1, 8, 1, 64, device="cuda")
    k = torch.randn(1, 2, 300, 64, device="cuda")
    v = torch.randn(1, 2, 300, 64, device="cuda")
    o = torch.empty_like(q)
    n = gpu_lib.gqa_decode_workspace_bytes(1, 8, 2, 64, 300)
    with pytest.raises(ValueError):
        gpu_lib.gqa_decode_attend(q, k, v, o, 300, torch.zeros(n, dtype=torch.uint8))
    with pytest.raises(ValueError):
        gpu_lib.gqa_decode_attend(q, k.cpu(), v, o, 300, gpu_lib.make_workspace(1, 8, 2, 64, 300))
    ws32 = torch.zeros((n + 3) // 4, dtype=torch.float32, device="cuda")
    gpu_lib.gqa_decode_attend(q, k, v, o, 300, ws32)
    torch.cuda.synchronize()
    assert_close(o, oracle.attend(q.cpu(), k.cpu(), v.cpu()), 2e-5, "float32 workspace")


def test_workspace_init_odd_size(gpu_lib):
    # every byte is cleared, including a tail shorter than a 32-bit word
    for n in (1, 3, 1027, 4096 * 1024 + 2):
        ws = torch.full((n,), 7, dtype=torch.uint8, device="cuda")
        gpu_lib.gqa_workspace_init(ws)
        torch.cuda.synchronize()
        assert int(ws.count_nonzero()) == 0, n


def test_read_probe_reads_and_writes_nothing(gpu_lib):
    # the measurement helper streams its input and leaves the sink alone
    for n in (16, 4096 + 16, 16805888):
        src = torch.arange(n // 4, dtype=torch.int32, device="cuda")
        sink = torch.full((4,), 5, dtype=torch.int32, device="cuda")
        gpu_lib.gqa_read_probe(src, sink)
        torch.cuda.synchronize()
        assert sink.tolist() == [5, 5, 5, 5], n


def test_workspace_init_entry_point(gpu_lib):
    q = torch.randn(1, 8, 1, 64, device="cuda")
    k = torch.randn(1, 2, 300, 64, device="cuda")
    v = torch.randn(1, 2, 300, 64, device="cuda")
    ws = torch.full((gpu_lib.gqa_decode_workspace_bytes(1, 8, 2, 64, 300),), 7, dtype=torch.uint8, device="cuda")
    gpu_lib.gqa_workspace_init(ws)
    o = torch.empty_like(q)
    gpu_lib.gqa_decode_attend(q, k, v, o, 300, ws)
    torch.cuda.synchronize()
    assert_close(o, oracle.attend(q.cpu(), k.cpu(), v.cpu()), 2e-5, "after workspace init")


# ---------------------------------------------------------------- batched

def run_batched(gqa, q, k, v, lens):
    B, Hq, _, D = q.shape
    Hkv, s_cap = k.shape[1], k.shape[2]
    ws = gqa.make_workspace(B, Hq, Hkv, D, s_cap)
    g = Guarded(q.shape, q.dtype)
    lens_d = torch.as_tensor(np.asarray(lens, dtype=np.int32)).cuda()
    gqa.gqa_decode_attend_batched(q.cuda(), k.cuda(), v.cuda(), g.t, lens_d, ws)
    torch.cuda.synchronize()
    g.check()
    return g.t


@pytest.mark.parametrize("B", [1, 2, 4, 8])
def test_batched_qwen3_4b(gpu_lib, B):
    w = W.by_name("batched_qwen3_4b")
    for layer in (0, 35):
        q, k, v, lens = W.batched_inputs(w, B, layer)
        note("batched B=%d layer=%d lens=%s" % (B, layer, list(lens)))
        got = run_batched(gpu_lib, q, k, v, lens)
        want = oracle.attend(q, k, v, kv_lens=lens)
        assert_close(got, want, 2e-2, "batched B=%d layer %d" % (B, layer))
        # bit-identical to one single-request call per request (same s_cap)
        qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
        for b in range(B):
            ws = gpu_lib.make_workspace(1, w.Hq, w.Hkv, w.D, w.s_cap)
            o1 = torch.empty_like(qd[b:b + 1])
            gpu_lib.gqa_decode_attend(qd[b:b + 1], kd[b:b + 1], vd[b:b + 1], o1, int(lens[b]), ws)
            torch.cuda.synchronize()
            assert torch.equal(o1, got[b:b + 1]), "request %d differs from its single call" % b
        # requests carry distinct data: no output is another's copy
        for b in range(1, B):
            assert not torch.equal(got[b], got[0])


def test_batched_long_and_short_requests(gpu_lib):
    # one request near the cache's end next to short and empty ones
    rng = np.random.default_rng(4)
    B, Hq, Hkv, D, s_cap = 4, 8, 2, 128, 65600
    q = torch.from_numpy(rng.standard_normal((B, Hq, 1, D), dtype=np.float32)).to(torch.bfloat16)
    k = torch.from_numpy(rng.standard_normal((B, Hkv, s_cap, D), dtype=np.float32)).to(torch.bfloat16)
    v = torch.from_numpy(rng.standard_normal((B, Hkv, s_cap, D), dtype=np.float32)).to(torch.bfloat16)
    lens = np.array([65537, 1, 30000, 0], np.int32)
    for b, n in enumerate(lens):
        k[b, :, n:] = float("nan")
        v[b, :, n:] = float("nan")
    note("batched long and short lens=%s" % list(lens))
    got = run_batched(gpu_lib, q, k, v, lens).cpu()
    want = oracle.attend(q, k, v, kv_lens=lens)
    assert_close(got, want, 2e-2, "long and short")
    assert torch.count_nonzero(got[3]) == 0


def test_batched_lengths_zero_clamped_and_ragged(gpu_lib):
    B, Hq, Hkv, D, s_cap = 6, 16, 4, 128, 200
    q = torch.randn(B, Hq, 1, D).to(torch.bfloat16)
    k = torch.randn(B, Hkv, s_cap, D).to(torch.bfloat16)
    v = torch.randn(B, Hkv, s_cap, D).to(torch.bfloat16)
    lens = np.array([0, 1, 33, 200, 5000, -3], np.int32)   # 5000 and -3 are clamped
    got = run_batched(gpu_lib, q, k, v, lens).cpu()
    eff = np.clip(lens, 0, s_cap)
    want = oracle.attend(q, k, v, kv_lens=eff)
    assert_close(got, want, 2e-2, "ragged batch")
    assert (got[0] == 0).all() and (got[5] == 0).all()


@pytest.mark.parametrize("B", [64, 70])
def test_batched_many_requests(gpu_lib, B):
    # Up to 64 requests, the splits that have rows are packed at the front of
    # the grid (each workgroup derives its request, head tile and split from
    # all the lengths); past 64 the grid is strided over (request, head tile,
    # split).  Both must match the oracle, with empty and full requests mixed
    # in, and each request must equal its own single-request call.  (160 rows
    # of 64: large enough for several splits per request.)
    Hq, Hkv, D, s_cap = 8, 2, 64, 160
    rng = np.random.default_rng(B)
    q = torch.from_numpy(rng.standard_normal((B, Hq, 1, D), dtype=np.float32)).to(torch.bfloat16)
    k = torch.from_numpy(rng.standard_normal((B, Hkv, s_cap, D), dtype=np.float32)).to(torch.bfloat16)
    v = torch.from_numpy(rng.standard_normal((B, Hkv, s_cap, D), dtype=np.float32)).to(torch.bfloat16)
    lens = rng.integers(0, s_cap + 1, size=B).astype(np.int32)
    lens[0], lens[1], lens[B - 1] = 0, s_cap, 1
    note("batched many requests B=%d" % B)
    got = run_batched(gpu_lib, q, k, v, lens)
    assert_close(got, oracle.attend(q, k, v, kv_lens=lens), 2e-2, "B=%d" % B)
    assert (got[0].cpu() == 0).all()
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    for b in (1, 2, B // 2, B - 1):
        if lens[b] == 0:  # (a single-request call needs a length of at least 1)
            continue
        ws = gpu_lib.make_workspace(1, Hq, Hkv, D, s_cap)
        o1 = torch.empty_like(qd[b:b + 1])
        gpu_lib.gqa_decode_attend(qd[b:b + 1], kd[b:b + 1], vd[b:b + 1], o1, int(lens[b]), ws)
        torch.cuda.synchronize()
        assert torch.equal(o1, got[b:b + 1]), "request %d differs from its single call" % b


def test_workspace_reuse_with_changing_inputs(gpu_lib):
    """Back-to-back calls on one workspace with different inputs: a merge that
    read a previous call's partials (or a counter left non-zero) would show up
    as a mismatch here.  Every call's output is checked."""
    rng = np.random.default_rng(99)
    B, Hq, Hkv, D, s_cap = 1, 28, 4, 128, 4096
    ws = gpu_lib.make_workspace(B, Hq, Hkv, D, s_cap)
    cases = []
    for i in range(24):
        n = int(rng.integers(1, s_cap + 1)) if i % 3 else s_cap
        q = torch.from_numpy(rng.standard_normal((B, Hq, 1, D), dtype=np.float32))
        k = torch.from_numpy(rng.standard_normal((B, Hkv, s_cap, D), dtype=np.float32))
        v = torch.from_numpy(rng.standard_normal((B, Hkv, s_cap, D), dtype=np.float32))
        o = torch.empty((B, Hq, 1, D), device="cuda")
        gpu_lib.gqa_decode_attend(q.cuda(), k.cuda(), v.cuda(), o, n, ws)  # no sync between calls
        cases.append((q, k, v, n, o))
    torch.cuda.synchronize()
    for q, k, v, n, o in cases:
        assert_close(o, oracle.attend(q, k, v, kv_lens=n), 2e-5, "reuse n=%d" % n)


def test_decode_concurrent_streams_separate_workspaces(gpu_lib):
    """The 7B-geometry fp32 decode at KV length 4096 and the 4-bit decode at
    KV length 16384 run concurrently on two streams (default priority), each
    with its own workspace, four calls per stream and round, ten rounds.  Each
    launch fills the device, so their workgroups compete for compute units:
    the merges must not rely on a whole launch being resident.  Every output
    is checked against the oracle; the first failure stops the test."""
    w7 = W.by_name("decode_7b")
    q7, k7, v7 = W.decode_inputs(w7, 4096, 0)
    want7 = oracle.attend(q7, k7, v7, scale=w7.scale())
    w4 = W.by_name("q4_decode")
    x4 = W.q4_inputs(w4, 16384, 0)
    names = ("k_codes", "k_scales", "k_biases", "v_codes", "v_scales", "v_biases")
    want4 = oracle.q4_attend(x4["q"], *(x4[n] for n in names), w4.group, scale=w4.scale())
    d7 = [t.cuda() for t in (q7, k7, v7)]
    d4 = {n: t.cuda() for n, t in x4.items()}
    ws7 = gpu_lib.make_workspace(1, w7.Hq, w7.Hkv, w7.D, 4096)
    ws4 = gpu_lib.make_workspace(1, w4.Hq, w4.Hkv, w4.D, 16384)
    outs7 = [torch.empty_like(d7[0]) for _ in range(4)]
    outs4 = [torch.empty_like(d4["q"]) for _ in range(4)]
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    for r in range(10):
        note("concurrent decode round %d" % r)
        with torch.cuda.stream(s1):
            for o in outs7:
                gpu_lib.gqa_decode_attend(d7[0], d7[1], d7[2], o, 4096, ws7)
        with torch.cuda.stream(s2):
            for o in outs4:
                gpu_lib.gqa_decode_attend_q4(d4["q"], *(d4[n] for n in names), o, w4.group, 16384, ws4)
        torch.cuda.synchronize()
        for i, o in enumerate(outs7):
            assert_close(o, want7, 2e-5, "round %d fp32 call %d" % (r, i))
        for i, o in enumerate(outs4):
            assert_close(o, want4, 2e-2, "round %d 4-bit call %d" % (r, i))
    assert_workspace_ready(ws7, "fp32 decode workspace after the concurrent rounds")
    assert_workspace_ready(ws4, "4-bit decode workspace after the concurrent rounds")
