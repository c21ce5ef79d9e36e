#!/usr/bin/env python3
"""Benchmark of the fused grouped-query attention library on one MI355X.

Headline workload (``value``): single-token decode attention with Qwen2.5-7B
heads (28 query / 4 KV heads, head dim 64*2 = 128), fp32 KV cache of 4096
rows per layer in the preallocated [Hkv, S, D] layout, 28 independently
seeded layers.  One step = one decode token through all 28 layers = 28 launches of
the split-K decode kernel, captured once in a HIP graph and replayed.  The
value is microseconds per layer (lower is better).

Secondary metric: causal prefill attention with Qwen2.5-0.5B heads (14 / 2,
dim 64), bf16, T = 513, 2049 and 4097, one step = 24 layers (that model's
depth) captured in a HIP graph, reported per layer as TFLOP/s and as a
fraction of the bf16 matrix-core peak.  The other configurations of the
workload set are reported the same way, each behind its own parity gate:
the 7B decode at KV lengths 128 ... 2048, decode at KV length 128 with 0.5B
heads, batched bf16 decode with Qwen3-4B heads at B = 1, 2, 4, 8, 4-bit
decode at KV length 2048 and 16384, the chunked prefill of 256 queries at
offset 3841, the cache append (dense and 4-bit) that precedes each decode
step, and the unfused torch-ROCm path the pages compare against (repeat the
KV heads, matmul, scale and mask, softmax, matmul) for the 7B decode and the
T = 4097 prefill.  --extras picks a subset, --no-extra skips them.

Protocol: inputs are generated on the host from fixed seeds and copied to
HBM before anything is timed; a parity gate compares sampled outputs with
the fp64 oracle first (no timing is reported if it fails); before each timed
step a 512 MiB buffer is read so that the 256 MB last-level cache holds none
of the step's inputs; HIP events on the launch stream bracket each step.
``cpu_baseline`` times the unmodified oracle on the host cores over a bounded
sample of the same workload.

Usage: python bench.py [--steps K] [--warmup W] [--gpus 1] [--extras a,b,...]
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2516.6      # MI355X dense bf16 matrix peak (256 CU x 2.4 GHz x 4096 FLOP/clk)
PAGES_M2_US_PER_LAYER_7B_S4096 = 264.82  # Apple M2 fused Metal SDPA (context only)
DECODE_SRCS = [os.path.join(ROOT, "prefill_split_gqa_amd", "csrc", f) for f in ("decode.hip", "common.h")]
PREFILL_SRCS = [os.path.join(ROOT, "prefill_split_gqa_amd", "csrc", f) for f in ("prefill.hip", "common.h")]
APPEND_SRCS = [os.path.join(ROOT, "prefill_split_gqa_amd", "csrc", f) for f in ("append.hip", "common.h")]
PROFILES = os.path.join(ROOT, "profiles")
PREFILL_COUNTERS_FILE = os.path.join(PROFILES, "prefill_0p5b_T4097_counters.txt")


def decode_bytes(S: int, Hq: int = 28, Hkv: int = 4, D: int = 128, elem: int = 4) -> int:
    """Algorithmic bytes of one decode launch: K and V rows read once, Q read
    once, O written once (no expanded KV, no score matrix)."""
    return 2 * Hkv * S * D * elem + 2 * Hq * D * elem


def prefill_flops(Tq: int, Tk: int, Hq: int = 14, D: int = 64) -> int:
    """Causal pairs (query row, visible key) x 4*D FLOP (QK^T and PV)."""
    off = Tk - Tq
    pairs = sum(min(i + off + 1, Tk) for i in range(Tq))
    return 4 * D * Hq * pairs


def prefill_bytes(Tq: int, Tk: int, Hq: int = 14, Hkv: int = 2, D: int = 64, elem: int = 2) -> int:
    """Compulsory HBM bytes of one prefill launch: Q read and O written once,
    K and V read once."""
    return 2 * Hq * Tq * D * elem + 2 * Hkv * Tk * D * elem


def q4r_prefill_bytes(Tq, Tk, Hq, Hkv, D, group, R) -> int:
    """Compulsory HBM bytes of a prefill chunk over a residual-window 4-bit
    cache: f16 Q read and O written once; per KV head the 4-bit rows' codes,
    scales and biases and the float16 residual rows of K and V read once."""
    n_q = Tk - Tk % R
    return 2 * Hq * Tq * D * 2 + 2 * Hkv * (n_q * (D // 2 + 2 * 2 * (D // group)) + (Tk - n_q) * D * 2)


def decode_bytes_generic(B, Hq, Hkv, D, lens, elem):
    """Algorithmic bytes of one decode launch: each request's valid K and V
    rows read once, its queries read and outputs written once."""
    return sum(2 * n * Hkv * D * elem for n in lens) + 2 * B * Hq * D * elem


def expanded_kv_bytes(S: int, Hq: int = 28, D: int = 128, elem: int = 4) -> int:
    """Bytes of the K and V copies an unfused decode writes per layer when it
    repeats every KV head once per query head (what this path never does)."""
    return 2 * Hq * S * D * elem


def score_matrix_bytes(T: int, Hq: int = 14, elem: int = 2) -> int:
    """Bytes of the [Hq, T, T] score matrix an unfused prefill writes per
    layer (what this path never does)."""
    return Hq * T * T * elem


def _code_only(text: str) -> str:
    """C/C++ source with comments removed and whitespace collapsed: what a
    counter summary must match (a comment edit does not change a kernel).
    String literals in these sources hold no comment markers."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def source_digest(paths) -> str:
    """Digest of the code (comments and whitespace aside) of the given sources."""
    h = hashlib.sha256()
    for p in paths:
        with open(p, encoding="utf-8") as f:
            h.update(_code_only(f.read()).encode())
    return h.hexdigest()[:16]


def read_summary_value(path, key, srcs, field):
    """A value from a committed rocprofv3 counter summary, or None when the
    summary is missing or was taken on a different kernel source."""
    try:
        kv = {}
        with open(path) as f:
            for ln in f:
                if ":" in ln and not ln.startswith("#"):
                    a, b = ln.split(":", 1)
                    kv[a.strip()] = b.split("#", 1)[0].strip()
        if kv.get(key) != source_digest(srcs):
            return None
        return float(kv[field])
    except (OSError, KeyError, ValueError):
        return None


def sources_of(kernel: str):
    """The source files a kernel is built from (a summary taken on other
    sources does not describe it)."""
    if "prefill" in kernel:
        return PREFILL_SRCS
    if "append" in kernel:
        return APPEND_SRCS
    return DECODE_SRCS


def attach_traffic(name: str, entry: dict) -> None:
    """Fill roofline.traffic (HBM bytes per launch, FETCH_SIZE + WRITE_SIZE
    calibrated) from the committed counter summary profiles/<name>_traffic.txt
    when it was taken on the current kernel sources; otherwise leave null."""
    rl = entry.get("roofline") if isinstance(entry, dict) else None
    if not rl or rl.get("traffic") is not None:
        return
    t = read_summary_value(os.path.join(PROFILES, name + "_traffic.txt"), "source_sha256_16",
                           sources_of(rl["kernel"]), "hbm_bytes_per_launch")
    rl["traffic"] = t
    base = rl.get("algorithmic_bytes_per_launch") or rl.get("compulsory_bytes_per_launch")
    if t is not None and base:
        rl["traffic_over_algorithmic"] = round(t / base, 3)


class Flusher:
    """Reads a buffer larger than the 256 MB last-level cache between timed
    steps, so a step's inputs come from HBM.  A read (not a write) leaves no
    dirty lines behind whose write-back would land inside the timed step."""

    def __init__(self, torch, mib=512):
        self.buf = torch.ones(mib * (1 << 20) // 4, dtype=torch.float32, device="cuda")

    def __call__(self):
        self.buf.sum()


def time_steps(torch, run_step, steps, warmup, flush):
    for _ in range(warmup):
        flush()
        run_step()
    torch.cuda.synchronize()
    pairs = []
    for _ in range(steps):
        flush()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        run_step()
        e1.record()
        pairs.append((e0, e1))
    torch.cuda.synchronize()
    return np.array([a.elapsed_time(b) for a, b in pairs])  # ms per step


def bench_decode(torch, gqa, oracle, W, S, layers, steps, warmup, flush, gate_layers):
    w = W.by_name("decode_7b")
    host = [W.decode_inputs(w, S, l) for l in range(layers)]
    dev = [tuple(t.cuda() for t in x) for x in host]
    outs = [torch.empty_like(x[0]) for x in dev]
    ws = gqa.make_workspace(1, w.Hq, w.Hkv, w.D, S)
    torch.cuda.synchronize()

    def eager():
        for (q, k, v), o in zip(dev, outs):
            gqa.gqa_decode_attend(q, k, v, o, S, ws)

    # parity gate on the eager path
    eager()
    torch.cuda.synchronize()
    gate = {}
    for l in gate_layers:
        want = oracle.attend(*host[l], scale=w.scale())
        err = float(np.abs(outs[l].cpu().double().numpy() - want).max())
        gate[l] = err
    ok = all(e <= 2e-5 for e in gate.values())
    ref = [o.clone() for o in outs]

    # one step = all layers, captured once
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        eager()  # warm the capture stream
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            eager()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()

    graph_ms = time_steps(torch, g.replay, steps, warmup, flush)
    replay_ok = all(torch.equal(a, b) for a, b in zip(outs, ref))
    eager_ms = time_steps(torch, eager, max(3, steps // 4), 2, flush)
    return {"S": S, "layers": layers, "gate_max_abs": max(gate.values()), "gate_ok": ok and replay_ok,
            "graph_ms": graph_ms, "eager_ms": eager_ms, "host": host, "scale": w.scale()}


def bench_prefill(torch, gqa, oracle, W, T, steps, warmup, flush, layers=24, n_check_rows=24):
    """One step = causal prefill attention of T tokens through `layers` layers
    (Qwen2.5-0.5B has 24), captured once in a HIP graph like the decode step.
    Layer 0 takes the seeded inputs, which gate parity on sampled rows; layer
    l > 0 takes its own device copies scaled by (1 + l/64), so every layer
    reads memory of its own after the cache flush."""
    w = W.by_name("prefill_0p5b")
    q, k, v = W.prefill_inputs(w, T)
    q0, k0, v0 = q.cuda(), k.cuda(), v.cuda()
    dev = [(q0, k0, v0)] + [tuple((x * (1.0 + l / 64.0)).contiguous() for x in (q0, k0, v0)) for l in range(1, layers)]
    outs = [torch.empty_like(q0) for _ in range(layers)]
    ws = gqa.make_prefill_workspace(1, w.Hq, w.Hkv, w.D, T, T)

    def eager():
        for (qd, kd, vd), o in zip(dev, outs):
            gqa.gqa_prefill_causal(qd, kd, vd, o, ws)

    eager()
    torch.cuda.synchronize()
    # parity gate on sampled rows of layer 0: row i is decode over keys 0..i
    rows = sorted(set([0, 1, T - 1] + list(np.random.default_rng(T).integers(0, T, n_check_rows - 3))))
    err = 0.0
    for i in rows:
        want = oracle.attend(q[:, :, i:i + 1], k[:, :, :i + 1], v[:, :, :i + 1], scale=w.scale())
        err = max(err, float(np.abs(outs[0][:, :, i:i + 1].float().cpu().double().numpy() - want).max()))
    ref = [o.clone() for o in outs]

    g = torch.cuda.CUDAGraph()
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(st):
        eager()
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=st):
            eager()
    torch.cuda.current_stream().wait_stream(st)
    torch.cuda.synchronize()
    ms = time_steps(torch, g.replay, steps, warmup, flush) / layers  # per layer
    replay_ok = all(torch.equal(a, b) for a, b in zip(outs, ref))
    return {"T": T, "layers": layers, "gate_max_abs": err, "gate_ok": err <= 2e-2 and replay_ok, "ms": ms,
            "flops": prefill_flops(T, T)}


def graph_of(torch, eager):
    """Capture eager() (every launch of one step) once in a HIP graph."""
    g = torch.cuda.CUDAGraph()
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(st):
        eager()
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=st):
            eager()
    torch.cuda.current_stream().wait_stream(st)
    torch.cuda.synchronize()
    return g


def calibration(torch, gqa, steps, warmup, flush, nbytes=16805888, layers=28, n=8192):
    """Self-calibrated ceilings, measured in the same run as the kernels.
    read_floor: the library's plain streaming-read helper over the decode
    step's bytes, launched like the decode step (a HIP graph of 28 launches,
    each reading its own 16.8 MB buffer, after the cache flush), so launch
    cost and cold-cache latency are included exactly as for decode.
    gemm_bf16: a dense n x n x n bf16 product through torch (the vendor GEMM)
    on contiguous operands, the matrix-core rate a tuned library reaches."""
    bufs = [torch.full((nbytes // 4,), l, dtype=torch.int32, device="cuda") for l in range(layers)]
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")

    def eager():
        for b in bufs:
            gqa.gqa_read_probe(b, sink)

    g = graph_of(torch, eager)
    us = float(np.median(time_steps(torch, g.replay, steps, warmup, flush))) * 1e3 / layers
    del g, bufs
    a = torch.randn(n, n, device="cuda").to(torch.bfloat16)
    b = torch.randn(n, n, device="cuda").to(torch.bfloat16)
    c = torch.empty(n, n, device="cuda", dtype=torch.bfloat16)
    for _ in range(3):
        torch.mm(a, b, out=c)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    reps = 10
    e0.record()
    for _ in range(reps):
        torch.mm(a, b, out=c)
    e1.record()
    torch.cuda.synchronize()
    gemm_s = e0.elapsed_time(e1) * 1e-3 / reps
    tf = 2.0 * n ** 3 / gemm_s / 1e12
    del a, b, c
    gbps = nbytes / (us * 1e-6) / 1e9
    return {"read_floor": {"kernel": "read_probe_kernel", "us_per_launch": round(us, 3), "GBps": round(gbps, 1),
                           "frac_hbm_peak": round(gbps / HBM_PEAK_GBS, 4), "bytes_per_launch": nbytes,
                           "launches_per_step": layers},
            "gemm_bf16": {"n": n, "TFLOPs": round(tf, 1), "frac_bf16_peak": round(tf / BF16_PEAK_TFLOPS, 4)}}


def hbm_entry(us, nbytes, gate_ok, gate_max_abs, kernel, traffic=None, **extra):
    """A secondary result for an HBM-bound configuration."""
    gbs = nbytes / (us * 1e-6) / 1e9
    d = {"us_layer": round(us, 3), "GBps": round(gbs, 1), "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
         "roofline": {"bound": "hbm", "kernel": kernel, "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                      "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": traffic,
                      "algorithmic_bytes_per_launch": nbytes, "launch_duration_us": round(us, 3)},
         "parity_ok": gate_ok, "parity_max_abs": gate_max_abs}
    d.update(extra)
    return d


EXTRAS = ("decode_7b_sweep", "prefill_0p5b_T513", "prefill_0p5b_T2049", "decode_0p5b_s128", "batched_qwen3_4b",
          "q4_decode_s2048", "q4_decode_s16384", "prefill_0p5b_chunk256_at3841", "append_7b_s4096",
          "append_q4_s16384", "q4r_decode_s16448_r128", "q4r_prefill_0p5b_chunk256_at3841_r128",
          "append_q4r_r128", "naive_decode_7b_s4096", "naive_prefill_0p5b_t4097")


def bench_extra(torch, gqa, oracle, W, steps, warmup, flush, names=EXTRAS):
    """The other configurations of the workload set (those named), each timed
    like the headline (per-layer inputs of their own, cache flushed before
    each step, one step captured in a HIP graph) after a parity gate on layer
    0 against the oracle; layers past the first are device copies of it,
    scaled (codes permuted for the 4-bit cache), so that every layer reads its
    own memory."""
    out = {}
    t0 = time.time()

    def done(what):
        sys.stderr.write("bench: %s done (%.0f s)\n" % (what, time.time() - t0))
        sys.stderr.flush()

    if "decode_7b_sweep" in names:
        out.update(extra_decode_sweep(torch, gqa, oracle, W, steps, warmup, flush))
        done("decode_7b_sweep")
    for T in (513, 2049):
        if "prefill_0p5b_T%d" % T in names:
            out["prefill_0p5b_T%d" % T] = prefill_entry(bench_prefill(torch, gqa, oracle, W, T, steps, warmup, flush))
            done("prefill_0p5b_T%d" % T)
    if "decode_0p5b_s128" in names:
        out.update(extra_decode_small(torch, gqa, oracle, W, steps, warmup, flush))
        done("decode_0p5b_s128")
    if "batched_qwen3_4b" in names:
        out.update(extra_batched(torch, gqa, oracle, W, steps, warmup, flush))
        done("batched_qwen3_4b")
    sizes = tuple(S for S in (2048, 16384) if "q4_decode_s%d" % S in names)
    if sizes:
        out.update(extra_q4(torch, gqa, oracle, W, steps, warmup, flush, sizes=sizes))
        done("q4_decode")
    if "prefill_0p5b_chunk256_at3841" in names:
        out.update(extra_chunked_prefill(torch, gqa, oracle, W, steps, warmup, flush))
        done("prefill_0p5b_chunk256_at3841")
    if "append_7b_s4096" in names:
        out.update(extra_append_dense(torch, gqa, oracle, W, steps, warmup, flush))
        done("append_7b_s4096")
    if "append_q4_s16384" in names:
        out.update(extra_append_q4(torch, gqa, oracle, W, steps, warmup, flush))
        done("append_q4_s16384")
    if "q4r_decode_s16448_r128" in names:
        out.update(extra_q4r_decode(torch, gqa, oracle, W, steps, warmup, flush))
        done("q4r_decode_s16448_r128")
    if "q4r_prefill_0p5b_chunk256_at3841_r128" in names:
        out.update(extra_q4r_prefill(torch, gqa, oracle, W, steps, warmup, flush))
        done("q4r_prefill_0p5b_chunk256_at3841_r128")
    if "append_q4r_r128" in names:
        out.update(extra_append_q4r(torch, gqa, oracle, W, steps, warmup, flush))
        done("append_q4r_r128")
    if "naive_decode_7b_s4096" in names:
        out.update(naive_decode(torch, oracle, W, steps, warmup, flush))
        done("naive_decode_7b_s4096")
    if "naive_prefill_0p5b_t4097" in names:
        out.update(naive_prefill(torch, oracle, W, max(3, steps // 2), 1, flush))
        done("naive_prefill_0p5b_t4097")
    for name, entry in out.items():
        attach_traffic(name, entry)
    return out


def extra_decode_small(torch, gqa, oracle, W, steps, warmup, flush):
    """Decode, Qwen2.5-0.5B heads, KV length 128, fp32; 28 layers per step
    (one launch alone would be mostly the graph's own launch cost)."""
    out = {}
    # (one launch alone would be mostly the graph's own launch cost)
    w = W.by_name("decode_0p5b")
    q, k, v = W.decode_inputs(w, 128, 0)
    d0 = (q.cuda(), k.cuda(), v.cuda())
    dev = [d0] + [tuple((x * (1.0 + l / 64.0)).contiguous() for x in d0) for l in range(1, 28)]
    outs = [torch.empty_like(d0[0]) for _ in dev]
    ws = gqa.make_workspace(1, w.Hq, w.Hkv, w.D, 128)

    def eager_small():
        for (qq, kk, vv), oo in zip(dev, outs):
            gqa.gqa_decode_attend(qq, kk, vv, oo, 128, ws)

    eager_small()
    torch.cuda.synchronize()
    err = float(np.abs(outs[0].cpu().double().numpy() - oracle.attend(q, k, v)).max())
    ref = [t.clone() for t in outs]
    g = graph_of(torch, eager_small)
    us = float(np.median(time_steps(torch, g.replay, steps, warmup, flush))) * 1e3 / len(dev)
    ok = err <= 2e-5 and all(torch.equal(a, b) for a, b in zip(outs, ref))
    out["decode_0p5b_s128"] = hbm_entry(us, decode_bytes_generic(1, w.Hq, w.Hkv, w.D, [128], 4), ok, err,
                                        "decode_mfma_kernel<float,64,7>",
                                        layers_per_step=len(dev))
    return out


def extra_batched(torch, gqa, oracle, W, steps, warmup, flush):
    """Batched decode, Qwen3-4B heads, bf16, per-request lengths, 36 layers."""
    out = {}
    w = W.by_name("batched_qwen3_4b")
    for B in (1, 2, 4, 8):
        q, k, v, lens = W.batched_inputs(w, B, 0)
        d0 = (q.cuda(), k.cuda(), v.cuda())
        dev = [d0] + [tuple((x * (1.0 + l / 64.0)).contiguous() for x in d0) for l in range(1, w.layers)]
        outs = [torch.empty_like(d0[0]) for _ in dev]
        lens_d = torch.as_tensor(lens.astype(np.int32)).cuda()
        ws = gqa.make_workspace(B, w.Hq, w.Hkv, w.D, w.s_cap)

        def eager(dev=dev, outs=outs, lens_d=lens_d, ws=ws):
            for (qq, kk, vv), oo in zip(dev, outs):
                gqa.gqa_decode_attend_batched(qq, kk, vv, oo, lens_d, ws)

        eager()
        torch.cuda.synchronize()
        err = float(np.abs(outs[0].float().cpu().double().numpy() - oracle.attend(q, k, v, kv_lens=lens)).max())
        ref = [x.clone() for x in outs]
        g = graph_of(torch, eager)
        us = float(np.median(time_steps(torch, g.replay, steps, warmup, flush))) * 1e3 / w.layers
        ok = err <= 2e-2 and all(torch.equal(a, b) for a, b in zip(outs, ref))
        out["batched_qwen3_4b_B%d" % B] = hbm_entry(
            us, decode_bytes_generic(B, w.Hq, w.Hkv, w.D, [int(x) for x in lens], 2), ok, err,
            "decode_mfma_kernel<bf16_t,128,4>",
            layers_per_step=w.layers, kv_lens=[int(x) for x in lens])
        del dev, outs, ref, g
        torch.cuda.empty_cache()
    return out


def extra_q4(torch, gqa, oracle, W, steps, warmup, flush, sizes=(2048, 16384)):
    """4-bit decode, 64 query / 8 KV heads, group 64, f16 queries, 80 layers."""
    out = {}
    w = W.by_name("q4_decode")
    names = ("k_codes", "k_scales", "k_biases", "v_codes", "v_scales", "v_biases")
    for S in sizes:
        x = W.q4_inputs(w, S, 0)
        d0 = {n: t.cuda() for n, t in x.items()}
        dev = [d0]
        for l in range(1, w.layers):
            dl = {"q": (d0["q"] * (1.0 + l / 64.0)).contiguous()}
            for n in names:
                t = d0[n]
                dl[n] = (t ^ (l & 0xFF)) if t.dtype == torch.uint8 else (t * (1.0 + l / 64.0)).contiguous()
            dev.append(dl)
        outs = [torch.empty_like(d0["q"]) for _ in dev]
        ws = gqa.make_workspace(1, w.Hq, w.Hkv, w.D, S)

        def eager(dev=dev, outs=outs, ws=ws, S=S):
            for dl, oo in zip(dev, outs):
                gqa.gqa_decode_attend_q4(dl["q"], *(dl[n] for n in names), oo, w.group, S, ws)

        eager()
        torch.cuda.synchronize()
        want = oracle.q4_attend(x["q"], *(x[n] for n in names), w.group)
        err = float(np.abs(outs[0].float().cpu().double().numpy() - want).max())
        ref = [t.clone() for t in outs]
        g = graph_of(torch, eager)
        us = float(np.median(time_steps(torch, g.replay, steps, warmup, flush))) * 1e3 / w.layers
        ok = err <= 2e-2 and all(torch.equal(a, b) for a, b in zip(outs, ref))
        nbytes = S * w.Hkv * 2 * (w.D // 2 + 2 * 2 * (w.D // w.group)) + 2 * w.Hq * w.D * 2
        out["q4_decode_s%d" % S] = hbm_entry(us, nbytes, ok, err, "decode_q4_kernel<128,64,8>",
                                             layers_per_step=w.layers)
        del dev, outs, ref, g
        torch.cuda.empty_cache()
    return out


def extra_chunked_prefill(torch, gqa, oracle, W, steps, warmup, flush):
    """Chunked prefill: the last 256 queries of T=4097 against all 4097 keys,
    24 layers."""
    out = {}
    w = W.by_name("prefill_0p5b")
    q, k, v = W.prefill_inputs(w, 4097)
    qc = q[:, :, 4097 - 256:].contiguous()
    d0 = (qc.cuda(), k.cuda(), v.cuda())
    dev = [d0] + [tuple((x * (1.0 + l / 64.0)).contiguous() for x in d0) for l in range(1, 24)]
    outs = [torch.empty_like(d0[0]) for _ in dev]
    ws = gqa.make_prefill_workspace(1, w.Hq, w.Hkv, w.D, 256, 4097)

    def eager_pf():
        for (qq, kk, vv), oo in zip(dev, outs):
            gqa.gqa_prefill_causal(qq, kk, vv, oo, ws)

    eager_pf()
    torch.cuda.synchronize()
    rows = sorted(set([0, 1, 255] + list(np.random.default_rng(256).integers(0, 256, 13))))
    err = 0.0
    for i in rows:  # chunk row i sees keys 0 .. 3841 + i
        want = oracle.attend(qc[:, :, i:i + 1], k[:, :, :3842 + i], v[:, :, :3842 + i], scale=w.scale())
        err = max(err, float(np.abs(outs[0][:, :, i:i + 1].float().cpu().double().numpy() - want).max()))
    ref = [t.clone() for t in outs]
    g = graph_of(torch, eager_pf)
    us = float(np.median(time_steps(torch, g.replay, steps, warmup, flush))) * 1e3 / len(dev)
    flops = prefill_flops(256, 4097)
    tf = flops / (us * 1e-6) / 1e12
    out["prefill_0p5b_chunk256_at3841"] = {
        "us": round(us, 2), "layers_per_step": len(dev), "TFLOPs": round(tf, 2),
        "frac_bf16_peak": round(tf / BF16_PEAK_TFLOPS, 4),
        "roofline": {"bound": "mfma", "kernel": "prefill_causal_kernel<bf16_t,64,false>", "achieved": round(tf, 1),
                     "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": round(tf / BF16_PEAK_TFLOPS, 4),
                     "traffic": None, "algorithmic_flop_per_launch": flops,
                     "compulsory_bytes_per_launch": prefill_bytes(256, 4097), "launch_duration_us": round(us, 2)},
        "parity_ok": err <= 2e-2 and all(torch.equal(a, b) for a, b in zip(outs, ref)), "parity_max_abs": err}
    return out


def prefill_entry(p, traffic=None, counters=None, gemm=None):
    """The result entry of one prefill configuration."""
    us = float(np.median(p["ms"])) * 1e3
    tf = p["flops"] / (us * 1e-6) / 1e12
    d = {"us": round(us, 2), "layers_per_step": p["layers"], "TFLOPs": round(tf, 2),
         "score_matrix_bytes_avoided": score_matrix_bytes(p["T"]),
         "frac_bf16_peak": round(tf / BF16_PEAK_TFLOPS, 4),
         "roofline": {"bound": "mfma", "kernel": "prefill_causal_kernel<bf16_t,64,false>",
                      "achieved": round(tf, 1), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                      "frac": round(tf / BF16_PEAK_TFLOPS, 4), "traffic": traffic,
                      "algorithmic_flop_per_launch": p["flops"],
                      "compulsory_bytes_per_launch": prefill_bytes(p["T"], p["T"]), "launch_duration_us": round(us, 2)},
         "parity_ok": p["gate_ok"], "parity_max_abs": p["gate_max_abs"]}
    if counters is not None:
        d["roofline"]["mfma_busy_counter_frac"] = counters
    if gemm:
        d["frac_of_gemm_bf16"] = round(tf / gemm, 4)
    return d


def extra_decode_sweep(torch, gqa, oracle, W, steps, warmup, flush, sizes=(128, 256, 512, 1024, 2048)):
    """The 7B-geometry fp32 decode at the other KV lengths of the pages'
    table, each timed like the headline (28 seeded layers, graph, flush)."""
    out = {}
    for S in sizes:
        d = bench_decode(torch, gqa, oracle, W, S, 28, steps, warmup, flush, gate_layers=(0,))
        us = float(np.median(d["graph_ms"])) * 1e3 / 28
        out["decode_7b_s%d" % S] = hbm_entry(us, decode_bytes(S), d["gate_ok"], d["gate_max_abs"],
                                             "decode_mfma_kernel<float,128,7>",
                                             layers_per_step=28,
                                             eager_us_layer=round(float(np.median(d["eager_ms"])) * 1e3 / 28, 3))
    return out


def extra_append_dense(torch, gqa, oracle, W, steps, warmup, flush, S=4096):
    """The dense append before a 7B-geometry fp32 decode step: one new
    token's K and V rows (4 KV heads x 128) written at row S-1 of each of 28
    layers' preallocated 4096-row caches; device lengths in and out.  Parity:
    the caches after the append equal the oracle's placement bit for bit."""
    w = W.by_name("decode_7b")
    layers = 28
    rng = np.random.default_rng(4096)
    caches = [(torch.zeros((1, w.Hkv, S, w.D), device="cuda"), torch.zeros((1, w.Hkv, S, w.D), device="cuda"))
              for _ in range(layers)]
    new = [(torch.from_numpy(rng.standard_normal((1, w.Hkv, 1, w.D), dtype=np.float32)).cuda(),
            torch.from_numpy(rng.standard_normal((1, w.Hkv, 1, w.D), dtype=np.float32)).cuda()) for _ in range(layers)]
    lens = torch.tensor([S - 1], dtype=torch.int32, device="cuda")
    new_lens = torch.zeros(1, dtype=torch.int32, device="cuda")

    def eager():
        for (kc, vc), (kn, vn) in zip(caches, new):
            gqa.gqa_kv_append(kn, vn, kc, vc, lens, new_lens)

    eager()
    torch.cuda.synchronize()
    want, wl = oracle.kv_append(np.zeros((1, w.Hkv, S, w.D), np.float32), new[0][0].cpu().numpy(), [S - 1])
    ok = bool(np.array_equal(caches[0][0].cpu().numpy(), want)) and int(new_lens.cpu()[0]) == int(wl[0])
    g = graph_of(torch, eager)
    us = float(np.median(time_steps(torch, g.replay, steps, warmup, flush))) * 1e3 / layers
    nbytes = 2 * 2 * w.Hkv * w.D * 4  # new K and V rows read and written
    return {"append_7b_s4096": hbm_entry(us, nbytes, ok, 0.0 if ok else None, "kv_append_kernel",
                                         layers_per_step=layers, bit_exact=ok)}


def extra_append_q4(torch, gqa, oracle, W, steps, warmup, flush, S=16384):
    """The 4-bit append before a decode step of the 64/8-head workload: one
    new token's f16 K and V rows (8 KV heads x 128) quantized into row S-1 of
    each of 80 layers' 16384-row caches (codes, f16 scale and bias per group
    of 64).  Parity: codes, scales and biases equal the oracle's quantizer
    bit for bit."""
    w = W.by_name("q4_decode")
    layers = w.layers
    rng = np.random.default_rng(16384)
    G = w.D // w.group

    def cache():
        return [torch.zeros((1, w.Hkv, S, w.D // 2), dtype=torch.uint8, device="cuda"),
                torch.zeros((1, w.Hkv, S, G), dtype=torch.float16, device="cuda"),
                torch.zeros((1, w.Hkv, S, G), dtype=torch.float16, device="cuda")]

    caches = [(cache(), cache()) for _ in range(layers)]
    new = [(torch.from_numpy(rng.standard_normal((1, w.Hkv, 1, w.D), dtype=np.float32)).half().cuda(),
            torch.from_numpy(rng.standard_normal((1, w.Hkv, 1, w.D), dtype=np.float32)).half().cuda())
           for _ in range(layers)]
    lens = torch.tensor([S - 1], dtype=torch.int32, device="cuda")

    def eager():
        for (kc, vc), (kn, vn) in zip(caches, new):
            gqa.gqa_kv_append_q4(kn, vn, *kc, *vc, w.group, lens)

    eager()
    torch.cuda.synchronize()
    c, sc, bi = oracle.q4_quantize(new[0][0].cpu(), w.group)
    kc = caches[0][0]
    ok = (np.array_equal(kc[0][:, :, S - 1:].cpu().numpy(), c)
          and np.array_equal(kc[1][:, :, S - 1:].cpu().numpy().view(np.uint16), sc.view(np.uint16))
          and np.array_equal(kc[2][:, :, S - 1:].cpu().numpy().view(np.uint16), bi.view(np.uint16)))
    g = graph_of(torch, eager)
    us = float(np.median(time_steps(torch, g.replay, steps, warmup, flush))) * 1e3 / layers
    nbytes = 2 * w.Hkv * (w.D * 2 + w.D // 2 + 2 * 2 * G)  # f16 rows read; codes, scales, biases written
    return {"append_q4_s16384": hbm_entry(us, nbytes, bool(ok), 0.0 if ok else None, "kv_append_q4_kernel<f16_t,128,64>",
                                          layers_per_step=layers, bit_exact=bool(ok))}


Q4R_NAMES = ("k_codes", "k_scales", "k_biases", "v_codes", "v_scales", "v_biases", "k_res", "v_res")


def _q4r_layers(torch, d0, layers):
    """Device copies of one residual-window cache state, one per layer
    (codes permuted, float values scaled), so that every layer reads its own
    memory."""
    dev = [d0]
    for l in range(1, layers):
        dl = {}
        for n, t in d0.items():
            dl[n] = (t ^ (l & 0xFF)) if t.dtype == torch.uint8 else (t * (1.0 + l / 64.0)).contiguous()
        dev.append(dl)
    return dev


def extra_q4r_decode(torch, gqa, oracle, W, steps, warmup, flush, n=16448, R=128):
    """Decode over a 4-bit cache with a float16 residual window (the 64/8-head
    workload, group 64, 80 layers): 16448 tokens = 16384 4-bit rows (the
    q4_decode_s16384 cache) plus 64 float16 residual rows (R = 128).  One
    launch per layer: the 4-bit kernel, whose last split streams the
    residual rows and is merged with the others."""
    w = W.by_name("q4_decode")
    rng = np.random.default_rng(16448)
    n_q, n_r = oracle.q4r_split(n, R)
    s_cap = n_q + R  # capacity for the request's positions; rows past n_q are never read
    x = W.q4_inputs(w, n_q, 0, s_cap=s_cap)
    st = {k: x[k] for k in Q4R_NAMES[:6]}
    st["k_res"] = torch.from_numpy(rng.standard_normal((1, w.Hkv, R, w.D)).astype(np.float16))
    st["v_res"] = torch.from_numpy(rng.standard_normal((1, w.Hkv, R, w.D)).astype(np.float16))
    q = x["q"]
    dev = _q4r_layers(torch, {k: v.cuda() for k, v in st.items()}, w.layers)
    qs = [(q.cuda() * (1.0 + l / 64.0)).contiguous() for l in range(w.layers)]
    outs = [torch.empty_like(qs[0]) for _ in dev]
    lens = torch.tensor([n], dtype=torch.int32, device="cuda")
    ws = gqa.make_q4r_workspace(1, w.Hq, w.Hkv, w.D, s_cap, R)

    def eager():
        for dl, qq, oo in zip(dev, qs, outs):
            gqa.gqa_decode_attend_q4r(qq, *(dl[k] for k in Q4R_NAMES), oo, w.group, lens, ws)

    eager()
    torch.cuda.synchronize()
    stn = {k: v.numpy() for k, v in st.items()}
    want = oracle.q4r_attend(q, stn, [n], w.group, R)
    err = float(np.abs(outs[0].float().cpu().double().numpy() - want).max())
    ref = [t.clone() for t in outs]
    g = graph_of(torch, eager)
    us = float(np.median(time_steps(torch, g.replay, steps, warmup, flush))) * 1e3 / w.layers
    ok = err <= 2e-2 and all(torch.equal(a, b) for a, b in zip(outs, ref))
    nbytes = (n_q * w.Hkv * 2 * (w.D // 2 + 2 * 2 * (w.D // w.group)) + n_r * w.Hkv * 2 * w.D * 2
              + 2 * w.Hq * w.D * 2)
    return {"q4r_decode_s16448_r128": hbm_entry(
        us, nbytes, ok, err, "decode_q4_kernel<128,64,8,1>",
        layers_per_step=w.layers, n_q=n_q, n_r=n_r, launches_per_layer=1)}


def extra_q4r_prefill(torch, gqa, oracle, W, steps, warmup, flush, Tk=4097, Tq=256, R=128, group=32):
    """Chunked prefill over a residual-window 4-bit cache: the last 256 queries
    of a 4097-token prompt on the 0.5B geometry (14/2 heads, D = 64, f16),
    the cache holding 4096 4-bit rows (group 32) and 1 float16 residual row;
    24 layers.  Parity: sampled chunk rows against the oracle over the
    cache's values."""
    w = W.by_name("prefill_0p5b")
    rng = np.random.default_rng(3841)
    k = rng.standard_normal((1, w.Hkv, Tk, w.D)).astype(np.float16)
    v = rng.standard_normal((1, w.Hkv, Tk, w.D)).astype(np.float16)
    st = {"k_codes": np.zeros((1, w.Hkv, Tk, w.D // 2), np.uint8), "v_codes": np.zeros((1, w.Hkv, Tk, w.D // 2), np.uint8),
          "k_scales": np.zeros((1, w.Hkv, Tk, w.D // group), np.float16),
          "k_biases": np.zeros((1, w.Hkv, Tk, w.D // group), np.float16),
          "v_scales": np.zeros((1, w.Hkv, Tk, w.D // group), np.float16),
          "v_biases": np.zeros((1, w.Hkv, Tk, w.D // group), np.float16),
          "k_res": np.zeros((1, w.Hkv, R, w.D), np.float16), "v_res": np.zeros((1, w.Hkv, R, w.D), np.float16)}
    st, _ = oracle.kv_append_q4r(st, k, v, [0], group, R)
    q = rng.standard_normal((1, w.Hq, Tq, w.D)).astype(np.float16)
    dev = _q4r_layers(torch, {n: torch.from_numpy(t).cuda() for n, t in st.items()}, 24)
    qs = [(torch.from_numpy(q).cuda() * (1.0 + l / 64.0)).contiguous() for l in range(24)]
    outs = [torch.empty_like(qs[0]) for _ in dev]
    ws = gqa.make_prefill_workspace(1, w.Hq, w.Hkv, w.D, Tq, Tk)

    def eager():
        for dl, qq, oo in zip(dev, qs, outs):
            gqa.gqa_prefill_causal_q4r(qq, *(dl[n] for n in Q4R_NAMES), oo, group, Tk, ws)

    eager()
    torch.cuda.synchronize()
    kv, vv = oracle.q4r_view(st, [Tk], group, R)
    rows = sorted(set([0, 1, Tq - 1] + list(np.random.default_rng(257).integers(0, Tq, 13))))
    err = 0.0
    for i in rows:
        n_vis = Tk - Tq + i + 1
        want = oracle.attend(q[:, :, i:i + 1], kv[:, :, :n_vis], vv[:, :, :n_vis], scale=w.scale())
        err = max(err, float(np.abs(outs[0][:, :, i:i + 1].float().cpu().double().numpy() - want).max()))
    ref = [t.clone() for t in outs]
    g = graph_of(torch, eager)
    us = float(np.median(time_steps(torch, g.replay, steps, warmup, flush))) * 1e3 / len(dev)
    flops = prefill_flops(Tq, Tk)
    tf = flops / (us * 1e-6) / 1e12
    return {"q4r_prefill_0p5b_chunk256_at3841_r128": {
        "us": round(us, 2), "layers_per_step": len(dev), "TFLOPs": round(tf, 2),
        "frac_bf16_peak": round(tf / BF16_PEAK_TFLOPS, 4),
        "roofline": {"bound": "mfma", "kernel": "prefill_causal_kernel<f16_t,64,false,true>", "achieved": round(tf, 1),
                     "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": round(tf / BF16_PEAK_TFLOPS, 4),
                     "traffic": None, "algorithmic_flop_per_launch": flops,
                     "compulsory_bytes_per_launch": q4r_prefill_bytes(Tq, Tk, w.Hq, w.Hkv, w.D, group, R),
                     "launch_duration_us": round(us, 2)},
        "parity_ok": err <= 2e-2 and all(torch.equal(a, b) for a, b in zip(outs, ref)), "parity_max_abs": err}}


def extra_append_q4r(torch, gqa, oracle, W, steps, warmup, flush, R=128):
    """The residual-window 4-bit append before a decode step of the 64/8-head
    workload, 80 layers, one new f16 token per layer: at 16447 tokens (the
    row joins the residual, no encoding) and at 16511 tokens (the residual
    fills: its 128 rows are encoded as a block).  Parity: every array equals
    the oracle's append bit for bit (layer 0)."""
    w = W.by_name("q4_decode")
    rng = np.random.default_rng(16511)
    G = w.D // w.group
    s_cap = 16640
    out = {}
    for name, n in (("append_q4r_r128", 16447), ("append_q4r_r128_flush", 16511)):
        st = {"k_codes": rng.integers(0, 256, (1, w.Hkv, s_cap, w.D // 2), dtype=np.uint8),
              "v_codes": rng.integers(0, 256, (1, w.Hkv, s_cap, w.D // 2), dtype=np.uint8),
              "k_scales": rng.random((1, w.Hkv, s_cap, G)).astype(np.float16),
              "k_biases": rng.random((1, w.Hkv, s_cap, G)).astype(np.float16),
              "v_scales": rng.random((1, w.Hkv, s_cap, G)).astype(np.float16),
              "v_biases": rng.random((1, w.Hkv, s_cap, G)).astype(np.float16),
              "k_res": rng.standard_normal((1, w.Hkv, R, w.D)).astype(np.float16),
              "v_res": rng.standard_normal((1, w.Hkv, R, w.D)).astype(np.float16)}
        kn = rng.standard_normal((1, w.Hkv, 1, w.D)).astype(np.float16)
        vn = rng.standard_normal((1, w.Hkv, 1, w.D)).astype(np.float16)
        want, _ = oracle.kv_append_q4r(st, kn, vn, [n], w.group, R)
        dev = _q4r_layers(torch, {k: torch.from_numpy(v).cuda() for k, v in st.items()}, w.layers)
        knd, vnd = torch.from_numpy(kn).cuda(), torch.from_numpy(vn).cuda()
        lens = torch.tensor([n], dtype=torch.int32, device="cuda")
        new_lens = torch.zeros(1, dtype=torch.int32, device="cuda")

        def eager(dev=dev):
            for dl in dev:
                gqa.gqa_kv_append_q4r(knd, vnd, *(dl[k] for k in Q4R_NAMES), w.group, lens, new_lens)

        eager()
        torch.cuda.synchronize()
        ok = all(np.array_equal(dev[0][k].cpu().numpy().view(np.uint8), want[k].view(np.uint8)) for k in Q4R_NAMES)
        ok = ok and int(new_lens.cpu()[0]) == n + 1
        g = graph_of(torch, eager)
        us = float(np.median(time_steps(torch, g.replay, steps, warmup, flush))) * 1e3 / w.layers
        n_q0, n_r0 = oracle.q4r_split(n, R)
        n_q1, _ = oracle.q4r_split(n + 1, R)
        aged = n_q1 - n_q0
        # new f16 rows read; aged rows read from the residual and encoded; kept rows written
        nbytes = 2 * w.Hkv * (w.D * 2 + aged * (w.D * 2 + w.D // 2 + 2 * 2 * G) + (1 if aged == 0 else 0) * w.D * 2)
        out[name] = hbm_entry(us, nbytes, bool(ok), 0.0 if ok else None, "kv_append_q4r_kernel<128,64>",
                              layers_per_step=w.layers, bit_exact=bool(ok), tokens_before=n, rows_encoded=aged)
        del dev
        torch.cuda.empty_cache()
    return out


def time_eager(torch, run, steps, warmup, flush):
    """Median ms per step of an eager sequence of launches, flush before each."""
    return float(np.median(time_steps(torch, run, steps, warmup, flush)))


def naive_decode(torch, oracle, W, steps, warmup, flush, S=4096):
    """The unfused decode the Candle page replaces ("7x KV expansion" plus
    matmul, softmax and matmul dispatches), in torch-ROCm on the same GPU:
    repeat each KV head for its 7 query heads, Q K^T, scale, softmax, P V;
    fp32, 28 seeded layers, eager, the cache flushed before each step."""
    w = W.by_name("decode_7b")
    layers = 28
    dev = [tuple(t.cuda() for t in W.decode_inputs(w, S, l)) for l in range(layers)]
    scale = w.scale()

    def run():
        outs = []
        for q, k, v in dev:
            kr = k.repeat_interleave(w.G, dim=1)
            vr = v.repeat_interleave(w.G, dim=1)
            p = torch.softmax(torch.matmul(q, kr.transpose(-1, -2)) * scale, dim=-1)
            outs.append(torch.matmul(p, vr))
        return outs

    outs = run()
    torch.cuda.synchronize()
    err = float(np.abs(outs[0].cpu().double().numpy() - oracle.attend(*(t.cpu() for t in dev[0]), scale=scale)).max())
    ms = time_eager(torch, run, steps, warmup, flush)
    us = ms * 1e3 / layers
    return {"naive_decode_7b_s4096": {
        "us_layer": round(us, 3), "path": "torch repeat_interleave, matmul, scale, softmax, matmul (fp32, eager)",
        "layers_per_step": layers, "algorithmic_bytes_per_layer": decode_bytes(S),
        "expanded_kv_bytes_written_per_layer": expanded_kv_bytes(S),
        "GBps_algorithmic": round(decode_bytes(S) / (us * 1e-6) / 1e9, 1), "max_abs_vs_oracle": err}}


def naive_prefill(torch, oracle, W, steps, warmup, flush, T=4097, layers=24):
    """The unfused prefill the Fornace page replaces: repeat_kv, a matmul
    writing the [14, T, T] scores, scale, causal mask, softmax, a second
    matmul, each its own kernel; bf16 in torch-ROCm on the same GPU, 24
    layers (layer l: the seeded inputs scaled by 1 + l/64), eager."""
    w = W.by_name("prefill_0p5b")
    q, k, v = W.prefill_inputs(w, T)
    q0, k0, v0 = q.cuda(), k.cuda(), v.cuda()
    dev = [(q0, k0, v0)] + [tuple((x * (1.0 + l / 64.0)).contiguous() for x in (q0, k0, v0)) for l in range(1, layers)]
    mask = torch.ones((T, T), dtype=torch.bool, device="cuda").tril()
    scale = w.scale()

    def run():
        outs = []
        for qq, kk, vv in dev:
            kr = kk.repeat_interleave(w.G, dim=1)
            vr = vv.repeat_interleave(w.G, dim=1)
            s_ = torch.matmul(qq, kr.transpose(-1, -2).contiguous()) * scale
            s_.masked_fill_(~mask, float("-inf"))
            outs.append(torch.matmul(torch.softmax(s_, dim=-1), vr))
        return outs[:1]

    outs = run()
    torch.cuda.synchronize()
    err = 0.0
    for i in (0, T // 2, T - 1):  # sampled rows: row i is decode over keys 0..i
        want = oracle.attend(q[:, :, i:i + 1], k[:, :, :i + 1], v[:, :, :i + 1], scale=scale)
        err = max(err, float(np.abs(outs[0][:, :, i:i + 1].float().cpu().double().numpy() - want).max()))
    ms = time_eager(torch, run, steps, warmup, flush)
    us = ms * 1e3 / layers
    flops = prefill_flops(T, T)
    return {"naive_prefill_0p5b_t4097": {
        "us": round(us, 1), "path": "torch repeat_interleave, matmul, scale, masked_fill, softmax, matmul (bf16, eager)",
        "layers_per_step": layers, "TFLOPs_algorithmic": round(flops / (us * 1e-6) / 1e12, 2),
        "score_matrix_bytes_per_layer": score_matrix_bytes(T), "max_abs_vs_oracle_sampled_rows": err}}


def cpu_baseline(oracle, host, scale, seconds, nthreads=0):
    """Time the oracle, as it stands, on the host cores (all of them, or
    `nthreads`) over whole layers of the headline workload until about
    `seconds` have elapsed."""
    import torch

    layers_f64 = [tuple(t.to(torch.float64).numpy() for t in x) for x in host]
    n_done = 0
    t0 = time.perf_counter()
    while True:
        q, k, v = layers_f64[n_done % len(layers_f64)]
        oracle.attend(q, k, v, scale=scale, nthreads=nthreads)
        n_done += 1
        el = time.perf_counter() - t0
        if el >= seconds and n_done >= 1:
            break
    return el / n_done * 1e6, n_done


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--S", type=int, default=4096, help="KV length of the headline decode workload")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--extras", default=",".join(EXTRAS),
                    help="comma-separated extra configurations to time (default: all of " + ", ".join(EXTRAS) + ")")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the other configurations (decode S=128, batched, 4-bit, chunked prefill)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-calibration", action="store_true",
                    help="skip the self-calibrated read floor and GEMM rate")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--calibration-copy", type=int, default=0, metavar="MIB",
                    help="also run one plain device copy of MIB MiB (reference for memory counters)")
    args = ap.parse_args()

    extra_names = tuple(x for x in args.extras.split(",") if x)
    unknown = [x for x in extra_names if x not in EXTRAS]
    if unknown:
        sys.exit("bench.py: unknown --extras %s (known: %s)" % (",".join(unknown), ",".join(EXTRAS)))
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        sys.stderr.write("bench.py measures one GPU: this build has no multi-GPU path "
                         "(--gpus %d requested)\n" % args.gpus)
        sys.exit(2)

    import torch

    import oracle
    import prefill_split_gqa_amd as gqa
    from workloads import configs as W

    gqa.load()
    torch.cuda.set_device(0)
    flush = Flusher(torch)
    if args.calibration_copy:
        src = torch.ones(args.calibration_copy * (1 << 20) // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        flush()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    layers = 28

    d = bench_decode(torch, gqa, oracle, W, args.S, layers, args.steps, args.warmup, flush,
                     gate_layers=(0, layers // 2, layers - 1))
    result = {"metric": "decode attn us/layer + HBM GB/s (% peak); prefill attn TFLOP/s (% MFMA)",
              "unit": "us/layer", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
              "higher_is_better": False, "scaling": "weak", "dtype": "f32", "data": "synthetic",
              "config": {"workload": "decode_7b_s%d" % args.S, "B": 1, "Hq": 28, "Hkv": 4, "D": 128,
                         "S": args.S, "layers": layers, "kv_cache": "preallocated [Hkv,S,D] fp32",
                         "inputs": "seeded N(0,1)", "timing": "HIP graph of 28 launches per step, "
                         "512 MiB read before each step evicts the last-level cache"}}
    if not d["gate_ok"]:
        result.update({"value": None, "ms_per_step": None, "vs_baseline": None,
                       "error": "parity gate failed: max-abs %.3e" % d["gate_max_abs"]})
        print(json.dumps(result), flush=True)
        sys.exit(1)

    ms_step = float(np.median(d["graph_ms"]))
    us_layer = ms_step * 1e3 / layers
    nbytes = decode_bytes(args.S)
    achieved = nbytes / (us_layer * 1e-6) / 1e9
    result.update({
        "value": round(us_layer, 3),
        "ms_per_step": round(ms_step, 4),
        "vs_baseline": round(us_layer / PAGES_M2_US_PER_LAYER_7B_S4096, 5) if args.S == 4096 else None,
        "baseline_context": "pages' fused Metal figure 264.82 us/layer on an Apple M2 10-core GPU "
                            "(same geometry and context); lower ratio = faster",
        "roofline": {"bound": "hbm", "kernel": "decode_mfma_kernel<float,128,7>",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": None, "algorithmic_bytes_per_launch": nbytes,
                     "launch_duration_us": round(us_layer, 3)},
        "decode_detail": {"expanded_kv_bytes_avoided": expanded_kv_bytes(args.S),
                          "p10_us_layer": round(float(np.percentile(d["graph_ms"], 10)) * 1e3 / layers, 3),
                          "p90_us_layer": round(float(np.percentile(d["graph_ms"], 90)) * 1e3 / layers, 3),
                          "eager_us_layer": round(float(np.median(d["eager_ms"])) * 1e3 / layers, 3),
                          "parity_max_abs": d["gate_max_abs"]},
    })

    attach_traffic("decode_7b_s%d" % args.S, result)

    if not args.no_calibration:
        try:  # auxiliary: a failure here must not cost the benchmark line
            cal = calibration(torch, gqa, args.steps, args.warmup, flush)
            result["calibration"] = cal
            result["decode_detail"]["frac_of_read_floor"] = round(achieved / cal["read_floor"]["GBps"], 4)
        except Exception as e:  # noqa: BLE001
            result["calibration"] = {"error": "%s: %s" % (type(e).__name__, e)}

    secondary = {}
    if not args.no_prefill:
        p = bench_prefill(torch, gqa, oracle, W, 4097, max(5, args.steps // 2), 2, flush)
        gemm = result.get("calibration", {}).get("gemm_bf16", {}).get("TFLOPs")
        secondary["prefill_0p5b_T4097"] = prefill_entry(
            p, counters=read_summary_value(PREFILL_COUNTERS_FILE, "source_sha256_16", PREFILL_SRCS,
                                           "mfma_busy_over_simd_cycles"), gemm=gemm)
        attach_traffic("prefill_0p5b_T4097", secondary["prefill_0p5b_T4097"])
        sys.stderr.write("bench: prefill_0p5b_T4097 done\n")
        sys.stderr.flush()
    if not args.no_extra:
        secondary.update(bench_extra(torch, gqa, oracle, W, max(5, args.steps // 2), 2, flush, extra_names))
    # the pages' headline ratios on this GPU: the unfused torch path against the fused kernels
    if "naive_decode_7b_s4096" in secondary:
        nd = secondary["naive_decode_7b_s4096"]
        nd["fused_speedup_graph"] = round(nd["us_layer"] / us_layer, 2)
        nd["fused_speedup_eager"] = round(nd["us_layer"] / result["decode_detail"]["eager_us_layer"], 2)
    if "naive_prefill_0p5b_t4097" in secondary and "prefill_0p5b_T4097" in secondary:
        npf = secondary["naive_prefill_0p5b_t4097"]
        npf["fused_speedup"] = round(npf["us"] / secondary["prefill_0p5b_T4097"]["us"], 2)
    if secondary:
        result["secondary"] = secondary

    if not args.no_cpu_baseline:
        us_cpu, n = cpu_baseline(oracle, d["host"], d["scale"], args.cpu_seconds)
        us_1, n_1 = cpu_baseline(oracle, d["host"], d["scale"], max(1.0, args.cpu_seconds / 4), nthreads=1)
        result["cpu_baseline"] = {"value": round(us_cpu, 1), "unit": "us/layer", "cores": oracle.max_threads(),
                                  "kind": "oracle",
                                  "sample": "%d whole layers of the same workload (S=%d), fp64 oracle, "
                                            "inputs widened before timing" % (n, args.S),
                                  "one_thread": {"value": round(us_1, 1), "layers": n_1},
                                  "cpu": cpu_model()}
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
