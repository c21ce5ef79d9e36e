"""The benchmark's byte and FLOP model against the arithmetic the pages print
(no GPU needed).

* "2x faster Qwen2 decode on Metal in Candle", section "Why It Matters: 7x KV
  Expansion on Every Decode Step": at 7B geometry, fp32 and 2048 tokens, K
  and V of one layer take 8 MiB as stored; copied up to the 28 query heads
  they take 56 MiB per layer, 1.53 GiB for the 28 layers.
* "Fused attention makes a 4,096-token Qwen2 prefill on Metal 4.5x
  faster...", section "Why it matters": the unfused prefill writes a
  [14, T, T] score matrix of 470 MB at T = 4096.
* Same Candle page, "Isolated Decode Attention Microbenchmark": the printed
  tables (tests/golden/candle_decode_microbench.txt) are self-consistent
  (speedup = upstream / fused, time saved = (upstream - fused) x layers), and
  the fused 7B figure at 4096 tokens is the one the benchmark quotes as
  context for its headline.
"""

import os

import pytest

import bench

MiB = 1 << 20
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "candle_decode_microbench.txt")


def test_unexpanded_kv_cache_is_8_mib():
    q_and_o = 2 * 28 * 128 * 4
    assert bench.decode_bytes(2048) - q_and_o == 8 * MiB
    # the same with the generic model (one request, its own length)
    assert bench.decode_bytes_generic(1, 28, 4, 128, [2048], 4) == bench.decode_bytes(2048)


def test_repeated_kv_heads_write_56_mib_per_layer_and_1p53_gib_per_token():
    assert bench.expanded_kv_bytes(2048) == 56 * MiB
    # the generic decode model with every KV head repeated reads the same bytes
    q_and_o = 2 * 28 * 128 * 4
    assert bench.decode_bytes_generic(1, 28, 28, 128, [2048], 4) - q_and_o == 56 * MiB
    assert round(28 * bench.expanded_kv_bytes(2048) / (1 << 30), 2) == 1.53
    # the expansion factor is the group size
    assert bench.expanded_kv_bytes(2048) == 7 * (bench.decode_bytes(2048) - q_and_o)


def test_score_matrix_is_470_mb_at_4096():
    assert round(bench.score_matrix_bytes(4096) / 1e6) == 470


def test_prefill_flops_count_the_causal_triangle():
    # one visible pair costs 4*D FLOP (QK^T and PV); square prompt: T(T+1)/2 pairs per head
    for T in (1, 2, 513, 4097):
        assert bench.prefill_flops(T, T) == 4 * 64 * 14 * T * (T + 1) // 2
    # a chunk of 256 queries at offset 3841 sees 3842 .. 4097 keys
    assert bench.prefill_flops(256, 4097) == 4 * 64 * 14 * sum(range(3842, 4098))


def _rows():
    rows = []
    for line in open(GOLDEN):
        if line.startswith("#") or not line.strip():
            continue
        g, layers, ctx, up, fused, speed, saved = line.split()
        rows.append((g, int(layers), int(ctx), float(up), float(fused), float(speed), float(saved)))
    return rows


def test_microbench_tables_are_self_consistent():
    rows = _rows()
    assert len(rows) == 12
    for g, layers, ctx, up, fused, speed, saved in rows:
        assert abs(up / fused - speed) <= 0.006, (g, ctx)
        assert abs((up - fused) * layers / 1000.0 - saved) <= 0.0015, (g, ctx)


def test_headline_context_figure_is_the_pages_7b_4096_row():
    row = [r for r in _rows() if r[0] == "7B" and r[2] == 4096]
    assert len(row) == 1
    assert bench.PAGES_M2_US_PER_LAYER_7B_S4096 == pytest.approx(row[0][4], abs=0)
