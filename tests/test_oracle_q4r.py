"""Pins for the oracle's residual-window 4-bit cache (no GPU).

Reading (VeloxQuant posts, "What this means in practice" and Part 4's
caveats: a production KIVI cache keeps recent tokens in float16): with
residual capacity R, n tokens are held as n_q = R * floor(n / R) 4-bit rows
and n - n_q exact float16 rows, position p >= n_q at residual slot p - n_q.

Pins, each independent of the append code's own arithmetic:
* the view equals the float16 inputs exactly on residual positions and
  equals q4_dequant(q4_quantize(row)) of the input row on 4-bit positions
  (q4_quantize and q4_dequant are pinned on their own);
* path independence: appending a request's tokens one at a time, in ragged
  blocks or all at once leaves identical bytes in every array (an error in
  the flush bookkeeping breaks this);
* incremental equals full re-encoding: the 4-bit rows equal quantizing the
  whole history [0, n_q) at once (the pages' harness re-quantized the full
  history every step);
* with R >= n nothing is quantized and the attention is the plain oracle's
  over the float16 rows;
* capacity: rows at or past s_cap are dropped and lengths capped;
* a planted off-by-one in the flush (oracle copy, CPU only) is caught.
"""

import numpy as np
import pytest

import oracle


def _empty_state(B, H, s_cap, D, group, R):
    return {
        "k_codes": np.zeros((B, H, s_cap, D // 2), np.uint8),
        "v_codes": np.zeros((B, H, s_cap, D // 2), np.uint8),
        "k_scales": np.zeros((B, H, s_cap, D // group), np.float16),
        "k_biases": np.zeros((B, H, s_cap, D // group), np.float16),
        "v_scales": np.zeros((B, H, s_cap, D // group), np.float16),
        "v_biases": np.zeros((B, H, s_cap, D // group), np.float16),
        "k_res": np.zeros((B, H, R, D), np.float16),
        "v_res": np.zeros((B, H, R, D), np.float16),
    }


def _rows(rng, B, H, T, D):
    return (rng.standard_normal((B, H, T, D)) * rng.uniform(0.5, 2.0)).astype(np.float16)


def _append_in_blocks(state, k, v, sizes, group, R):
    lens = np.zeros(k.shape[0], np.int32)
    t = 0
    for m in sizes:
        state, lens = oracle.kv_append_q4r(state, k[:, :, t:t + m], v[:, :, t:t + m], lens, group, R)
        t += m
    return state, lens


@pytest.mark.parametrize("D,group,R", [(64, 32, 64), (128, 64, 128), (128, 128, 64)])
def test_view_is_exact_residual_and_encoded_history(D, group, R):
    rng = np.random.default_rng(D + group + R)
    B, H, s_cap, T = 2, 2, 512, 300
    k, v = _rows(rng, B, H, T, D), _rows(rng, B, H, T, D)
    st, lens = _append_in_blocks(_empty_state(B, H, s_cap, D, group, R), k, v, [1, 7, 64, 100, 1, 127], group, R)
    assert list(lens) == [T, T]
    kv, vv = oracle.q4r_view(st, lens, group, R)
    n_q, n_r = oracle.q4r_split(T, R)
    assert n_q == R * (T // R) and n_q + n_r == T and 0 <= n_r < R
    for src, view in ((k, kv), (v, vv)):
        assert np.array_equal(view[:, :, n_q:T], src[:, :, n_q:T].astype(np.float32))
        c, s, b = oracle.q4_quantize(src[:, :, :n_q].astype(np.float32), group)
        assert np.array_equal(view[:, :, :n_q], oracle.q4_dequant(c, s, b, group))
        assert not view[:, :, T:].any()


@pytest.mark.parametrize("R", [64, 128])
def test_append_is_path_independent(R):
    rng = np.random.default_rng(R)
    B, H, s_cap, D, group, T = 1, 2, 640, 64, 32, 400
    k, v = _rows(rng, B, H, T, D), _rows(rng, B, H, T, D)
    ways = [[T], [1] * T, [R - 1, 1, 2 * R + 5, T - 3 * R - 5], [3, R, R, R + 7, T - 3 * R - 10]]
    states = [_append_in_blocks(_empty_state(B, H, s_cap, D, group, R), k, v, w, group, R) for w in ways]
    n_q, n_r = oracle.q4r_split(T, R)
    for st, lens in states[1:]:
        assert list(lens) == list(states[0][1])
        for key in st:
            a, b = st[key], states[0][0][key]
            if key.endswith("_res"):  # slots past the residual's length are not part of the state
                a, b = a[:, :, :n_r], b[:, :, :n_r]
            assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), key


def test_incremental_equals_full_requantization():
    rng = np.random.default_rng(5)
    B, H, s_cap, D, group, R = 2, 1, 1024, 128, 32, 128
    T = 1000
    k, v = _rows(rng, B, H, T, D), _rows(rng, B, H, T, D)
    st, lens = _append_in_blocks(_empty_state(B, H, s_cap, D, group, R), k, v, [17] * 58 + [T - 17 * 58], group, R)
    n_q, _ = oracle.q4r_split(T, R)
    for name, src in (("k", k), ("v", v)):
        c, s, b = oracle.q4_quantize(src[:, :, :n_q].astype(np.float32), group)
        assert np.array_equal(st[name + "_codes"][:, :, :n_q], c)
        assert np.array_equal(st[name + "_scales"][:, :, :n_q].view(np.uint16), s.view(np.uint16))
        assert np.array_equal(st[name + "_biases"][:, :, :n_q].view(np.uint16), b.view(np.uint16))
        # rows past n_q are untouched by the encoder
        assert not st[name + "_codes"][:, :, n_q:].any()


def test_short_requests_are_plain_float16_attention():
    rng = np.random.default_rng(9)
    B, Hq, H, s_cap, D, group, R = 2, 4, 2, 256, 64, 64, 128
    T = 100  # < R: nothing quantized
    k, v = _rows(rng, B, H, T, D), _rows(rng, B, H, T, D)
    st, lens = _append_in_blocks(_empty_state(B, H, s_cap, D, group, R), k, v, [T], group, R)
    assert not st["k_codes"].any() and not st["v_scales"].any()
    q = rng.standard_normal((B, Hq, 1, D)).astype(np.float16)
    got = oracle.q4r_attend(q, st, lens, group, R)
    want = oracle.attend(q, k, v, kv_lens=T)
    assert np.array_equal(got, want)
    # a chunk of 16 queries at the end, causal
    qc = rng.standard_normal((B, Hq, 16, D)).astype(np.float16)
    assert np.array_equal(oracle.q4r_attend(qc, st, lens, group, R, causal=True),
                          oracle.attend(qc, k, v, kv_lens=T, causal=True))


def test_capacity_drops_rows_past_s_cap():
    rng = np.random.default_rng(3)
    B, H, s_cap, D, group, R = 2, 1, 192, 64, 32, 64
    k, v = _rows(rng, B, H, 50, D), _rows(rng, B, H, 50, D)
    st = _empty_state(B, H, s_cap, D, group, R)
    st, lens = oracle.kv_append_q4r(st, k, v, np.array([150, 190], np.int32), group, R)
    assert list(lens) == [192, 192]
    # request 1 kept 2 rows (190, 191); positions [128, 192) were flushed
    # from the residual, which then is empty
    n_q, n_r = oracle.q4r_split(192, R)
    assert (n_q, n_r) == (192, 0)
    c, s, b = oracle.q4_quantize(k[1, :, :2].astype(np.float32), group)
    assert np.array_equal(st["k_codes"][1, :, 190:192], c)


def _append_off_by_one(state, k_new, v_new, kv_lens, group, R):
    """The oracle's append with the flush taken one row late (planted mistake)."""
    st = {key: np.array(val, copy=True) for key, val in state.items()}
    for b in range(k_new.shape[0]):
        n = int(kv_lens[b])
        m = k_new.shape[2]
        nq_old, nr_old = oracle.q4r_split(n, R)
        nq_new = R * ((n + m - 1) // R)  # wrong: one row late
        for name, new in (("k", k_new), ("v", v_new)):
            recent = np.concatenate([st[name + "_res"][b, :, :nr_old], new[b]], axis=1)
            aged = recent[:, :nq_new - nq_old]
            if aged.shape[1] > 0:
                c, s, bi = oracle.q4_quantize(aged.astype(np.float32), group)
                st[name + "_codes"][b, :, nq_old:nq_new] = c
                st[name + "_scales"][b, :, nq_old:nq_new] = s
                st[name + "_biases"][b, :, nq_old:nq_new] = bi
            keep = recent[:, nq_new - nq_old:]
            st[name + "_res"][b, :, :keep.shape[1]] = keep[:, :R]
    return st


def _view_matches_inputs(st, lens, k, v, group, R):
    """The check of test_view_is_exact_residual_and_encoded_history."""
    T = int(lens[0])
    n_q, _ = oracle.q4r_split(T, R)
    kv, vv = oracle.q4r_view(st, lens, group, R)
    for src, view in ((k, kv), (v, vv)):
        if not np.array_equal(view[:, :, n_q:T], src[:, :, n_q:T].astype(np.float32)):
            return False
        c, s, b = oracle.q4_quantize(src[:, :, :n_q].astype(np.float32), group)
        if not np.array_equal(view[:, :, :n_q], oracle.q4_dequant(c, s, b, group)):
            return False
    return True


@pytest.mark.parametrize("T", [64, 128, 129, 200])
def test_planted_flush_error_is_caught(T):
    rng = np.random.default_rng(11)
    B, H, s_cap, D, group, R = 1, 1, 256, 64, 32, 64
    k, v = _rows(rng, B, H, T, D), _rows(rng, B, H, T, D)
    good, lens = _append_in_blocks(_empty_state(B, H, s_cap, D, group, R), k, v, [T], group, R)
    assert _view_matches_inputs(good, lens, k, v, group, R)
    if T % R == 0:  # the late flush differs exactly when the length reaches a block boundary
        bad = _append_off_by_one(_empty_state(B, H, s_cap, D, group, R), k, v, np.zeros(1, np.int32), group, R)
        assert not _view_matches_inputs(bad, lens, k, v, group, R)
