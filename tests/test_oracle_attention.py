"""Pins for the fp64 attention oracle (no GPU).

The oracle (oracle/gqa_oracle.c) is checked against things other than itself:

* a numpy brute force that expands the KV heads with ``np.repeat`` (the
  repeat_kv step of the unfused path in "Fused attention makes a 4,096-token
  Qwen2 prefill on Metal 4.5x faster", section "Cause and workaround", its
  paragraph on the cause), builds the full
  score matrix, adds a -inf mask and applies scipy's softmax;
* torch's CPU ``scaled_dot_product_attention`` in float64 on repeated K/V
  with an explicit bottom-right boolean mask (the end-alignment of the same
  page's "Cause and workaround", point 2);
* closed forms: one visible key gives that key's value row; equal scores give
  the mean of the visible value rows; constant V gives that constant; the
  two-key softmax;
* invariants: probability rows sum to 1, masked weights are 0, linearity in
  V, decode equals the last prefill row, a chunk at an offset equals the tail
  of the full prefill, per-request lengths equal separate calls, NaN padding
  never leaks, and a power-of-two scale can move into Q.

A sensitivity check shows the brute force would catch an interleaved
(h mod Hkv) head mapping.
"""

import itertools

import numpy as np
import pytest
import scipy.special
import torch

import oracle

RNG = np.random.default_rng(1234)


def brute_force(q, k, v, lens, causal, scale, mapping="contiguous"):
    """Repeat-KV, full score matrix, additive -inf mask, library softmax."""
    B, Hq, Tq, D = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    if mapping == "contiguous":
        kr = np.repeat(k, G, axis=1)
        vr = np.repeat(v, G, axis=1)
    else:  # interleaved mapping, used only to show the pin is sensitive to it
        kr = np.tile(k, (1, G, 1, 1))
        vr = np.tile(v, (1, G, 1, 1))
    out = np.zeros_like(q)
    S = k.shape[2]
    for b in range(B):
        n = int(lens[b])
        scores = scale * np.einsum("hid,hjd->hij", q[b], kr[b])  # [Hq, Tq, S]
        j = np.arange(S)[None, :]
        i = np.arange(Tq)[:, None]
        visible = j < n
        if causal:
            visible = visible & (j <= i + (n - Tq))
        mask = np.where(visible, 0.0, -np.inf)
        p = scipy.special.softmax(scores + mask[None], axis=-1)
        p = np.where(visible[None], p, 0.0)
        out[b] = np.einsum("hij,hjd->hid", p, np.nan_to_num(vr[b]))
    return out


def rand(*shape):
    return RNG.standard_normal(shape)


SHAPES = [(1, 1), (2, 1), (4, 2), (7, 1), (14, 2)]


@pytest.mark.parametrize("hq,hkv", SHAPES)
@pytest.mark.parametrize("D", [1, 2, 3, 8])
@pytest.mark.parametrize("causal", [False, True])
def test_brute_force_sweep(hq, hkv, D, causal):
    for tq, tk in [(1, 1), (1, 5), (2, 2), (3, 7), (5, 9), (9, 9)]:
        B = 2
        S = 10
        q = rand(B, hq, tq, D)
        k = rand(B, hkv, S, D)
        v = rand(B, hkv, S, D)
        lens = np.array([tk, max(tq, tk - 1)], dtype=np.int32)
        scale = 0.37
        got = oracle.attend(q, k, v, kv_lens=lens, causal=causal, scale=scale)
        want = brute_force(q, k, v, lens, causal, scale)
        np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


def test_interleaved_mapping_is_detected():
    q = rand(1, 14, 3, 8)
    k = rand(1, 2, 9, 8)
    v = rand(1, 2, 9, 8)
    lens = np.array([9], np.int32)
    got = oracle.attend(q, k, v, kv_lens=lens, causal=True, scale=0.3)
    wrong = brute_force(q, k, v, lens, True, 0.3, mapping="interleaved")
    assert np.abs(got - wrong).max() > 1e-3


@pytest.mark.parametrize("hq,hkv", SHAPES)
@pytest.mark.parametrize("tq,tk", [(1, 6), (4, 4), (3, 8), (8, 8)])
def test_torch_sdpa_bottom_right(hq, hkv, tq, tk):
    D = 8
    q = torch.from_numpy(rand(1, hq, tq, D))
    k = torch.from_numpy(rand(1, hkv, tk, D))
    v = torch.from_numpy(rand(1, hkv, tk, D))
    G = hq // hkv
    kr = k.repeat_interleave(G, dim=1)
    vr = v.repeat_interleave(G, dim=1)
    i = torch.arange(tq)[:, None]
    j = torch.arange(tk)[None, :]
    mask = j <= i + (tk - tq)  # True = may attend
    want = torch.nn.functional.scaled_dot_product_attention(q, kr, vr, attn_mask=mask, scale=0.25)
    got = oracle.attend(q, k, v, causal=True, scale=0.25)
    np.testing.assert_allclose(got, want.numpy(), rtol=0, atol=1e-12)


def test_probabilities_are_a_distribution():
    q = rand(2, 4, 5, 8)
    k = rand(2, 2, 12, 8)
    v = rand(2, 2, 12, 8)
    lens = np.array([12, 7], np.int32)
    out, p = oracle.attend(q, k, v, kv_lens=lens, causal=True, scale=0.5, return_probs=True)
    assert (p >= 0).all()
    np.testing.assert_allclose(p.sum(-1), 1.0, rtol=0, atol=1e-14)
    for b, n in enumerate(lens):
        for i in range(5):
            last = i + (n - 5)
            assert (p[b, :, i, last + 1:] == 0).all()
            assert (p[b, :, i, : last + 1] > 0).all()
    # and the output is P @ V (G = 2: head h reads kv head h // 2)
    for b in range(2):
        for h in range(4):
            np.testing.assert_allclose(out[b, h], p[b, h] @ v[b, h // 2], rtol=0, atol=1e-12)


def test_single_visible_key_returns_value_row_exactly():
    q = rand(1, 7, 1, 64)
    k = rand(1, 1, 4, 64)
    v = rand(1, 1, 4, 64)
    out = oracle.attend(q, k, v, kv_lens=1, scale=0.125)
    assert np.array_equal(out[0, :, 0], np.broadcast_to(v[0, 0, 0], (7, 64)))
    # causal prefill row 0 with Tq == Tk sees only key 0
    q2 = rand(1, 7, 4, 64)
    out2 = oracle.attend(q2, k, v, causal=True, scale=0.125)
    assert np.array_equal(out2[0, :, 0], np.broadcast_to(v[0, 0, 0], (7, 64)))


def test_equal_scores_give_mean_of_values():
    v = rand(1, 2, 11, 16)
    k = rand(1, 2, 11, 16)
    q = np.zeros((1, 4, 1, 16))
    out = oracle.attend(q, k, v, kv_lens=9, scale=1.0)
    want = np.repeat(v[:, :, :9].mean(axis=2, keepdims=True), 2, axis=1)
    np.testing.assert_allclose(out, want, rtol=0, atol=1e-14)
    # equal key rows also make every score equal
    k_eq = np.broadcast_to(rand(1, 2, 1, 16), (1, 2, 11, 16)).copy()
    out2 = oracle.attend(rand(1, 4, 1, 16), k_eq, v, kv_lens=9, scale=1.0)
    np.testing.assert_allclose(out2, want, rtol=0, atol=1e-14)


def test_constant_values():
    c = rand(16)
    v = np.broadcast_to(c, (1, 1, 20, 16)).copy()
    out = oracle.attend(rand(1, 3, 4, 16), rand(1, 1, 20, 16), v, causal=True, scale=0.7)
    np.testing.assert_allclose(out, np.broadcast_to(c, out.shape), rtol=1e-15, atol=1e-15)


def test_two_key_closed_form():
    # scores a, b for keys 0, 1: o = (v0 + e^(b-a) v1) / (1 + e^(b-a))
    D = 4
    q = np.zeros((1, 1, 1, D))
    q[..., 0] = 1.0
    k = np.zeros((1, 1, 2, D))
    k[0, 0, 0, 0] = 0.5   # a = scale * 0.5
    k[0, 0, 1, 0] = 2.0   # b = scale * 2.0
    v = rand(1, 1, 2, D)
    scale = 0.8
    a, b = scale * 0.5, scale * 2.0
    r = np.exp(b - a)
    want = (v[0, 0, 0] + r * v[0, 0, 1]) / (1 + r)
    out = oracle.attend(q, k, v, scale=scale)
    np.testing.assert_allclose(out[0, 0, 0], want, rtol=1e-14, atol=1e-15)


def test_linearity_in_values():
    q = rand(1, 6, 3, 8)
    k = rand(1, 3, 10, 8)
    v1 = rand(1, 3, 10, 8)
    v2 = rand(1, 3, 10, 8)
    o12 = oracle.attend(q, k, v1 + v2, causal=True, scale=0.4)
    o1 = oracle.attend(q, k, v1, causal=True, scale=0.4)
    o2 = oracle.attend(q, k, v2, causal=True, scale=0.4)
    np.testing.assert_allclose(o12, o1 + o2, rtol=0, atol=1e-12)


def test_group_members_with_identical_queries_agree_and_gqa_reduces_to_mha():
    q = rand(1, 8, 2, 8)
    q[0, 1] = q[0, 0]  # heads 0 and 1 are in the same group (G = 4)
    k = rand(1, 2, 6, 8)
    v = rand(1, 2, 6, 8)
    out = oracle.attend(q, k, v, causal=True, scale=0.5)
    assert np.array_equal(out[0, 0], out[0, 1])
    # MHA (G = 1) on repeated K/V equals GQA on the grouped K/V
    kr = np.repeat(k, 4, axis=1)
    vr = np.repeat(v, 4, axis=1)
    mha = oracle.attend(q, kr, vr, causal=True, scale=0.5)
    assert np.array_equal(out, mha)
    # MQA: one KV head serves every query head
    mqa = oracle.attend(q, k[:, :1], v[:, :1], causal=True, scale=0.5)
    np.testing.assert_allclose(mqa, brute_force(q, k[:, :1], v[:, :1], [6], True, 0.5), atol=1e-12, rtol=0)


def test_decode_equals_last_prefill_row():
    T = 33
    q = rand(1, 14, T, 64)
    k = rand(1, 2, T, 64)
    v = rand(1, 2, T, 64)
    full = oracle.attend(q, k, v, causal=True, scale=0.125)
    dec = oracle.attend(q[:, :, T - 1:], k, v, causal=False, scale=0.125)
    assert np.array_equal(dec[:, :, 0], full[:, :, T - 1])


def test_chunk_at_offset_equals_tail_of_full_prefill():
    Tk, Tq = 97, 16
    off = Tk - Tq
    q = rand(1, 14, Tk, 64)
    k = rand(1, 2, Tk, 64)
    v = rand(1, 2, Tk, 64)
    full = oracle.attend(q, k, v, causal=True, scale=0.125)
    chunk = oracle.attend(q[:, :, off:], k, v, causal=True, scale=0.125)
    assert np.array_equal(chunk, full[:, :, off:])


def test_per_request_lengths_equal_separate_calls_and_padding_never_leaks():
    B, S = 3, 40
    lens = np.array([40, 17, 1], np.int32)
    q = rand(B, 8, 1, 16)
    k = rand(B, 2, S, 16)
    v = rand(B, 2, S, 16)
    for b in range(B):
        k[b, :, lens[b]:] = np.nan
        v[b, :, lens[b]:] = np.nan
    out = oracle.attend(q, k, v, kv_lens=lens, scale=0.25)
    assert np.isfinite(out).all()
    for b in range(B):
        n = int(lens[b])
        one = oracle.attend(q[b:b + 1], k[b:b + 1, :, :n], v[b:b + 1, :, :n], scale=0.25)
        assert np.array_equal(out[b:b + 1], one)


def test_zero_length_request_gives_zeros():
    out = oracle.attend(rand(2, 4, 1, 8), rand(2, 2, 5, 8), rand(2, 2, 5, 8),
                        kv_lens=np.array([0, 5], np.int32), scale=0.5)
    assert (out[0] == 0).all()
    assert np.abs(out[1]).sum() > 0


def test_power_of_two_scale_moves_into_queries():
    q = rand(1, 4, 3, 64)
    k = rand(1, 2, 9, 64)
    v = rand(1, 2, 9, 64)
    a = oracle.attend(q, k, v, causal=True, scale=0.125)
    b = oracle.attend(q * 0.125, k, v, causal=True, scale=1.0)
    assert np.array_equal(a, b)
    c = oracle.attend(q, k, v, causal=True, scale=1.0)
    assert np.abs(a - c).max() > 1e-3


def test_default_scale_is_float32_inverse_sqrt():
    q = rand(1, 2, 1, 128)
    k = rand(1, 1, 5, 128)
    v = rand(1, 1, 5, 128)
    s32 = float(np.float32(1.0) / np.sqrt(np.float32(128)))
    assert np.array_equal(oracle.attend(q, k, v), oracle.attend(q, k, v, scale=s32))


def test_bf16_inputs_are_widened_exactly():
    q = torch.randn(1, 4, 2, 8).to(torch.bfloat16)
    k = torch.randn(1, 2, 6, 8).to(torch.bfloat16)
    v = torch.randn(1, 2, 6, 8).to(torch.bfloat16)
    a = oracle.attend(q, k, v, causal=True, scale=0.5)
    b = oracle.attend(q.double().numpy(), k.double().numpy(), v.double().numpy(), causal=True, scale=0.5)
    assert np.array_equal(a, b)


def test_argument_validation():
    with pytest.raises(ValueError):
        oracle.attend(rand(1, 3, 1, 8), rand(1, 2, 4, 8), rand(1, 2, 4, 8))  # Hq % Hkv != 0
    with pytest.raises(ValueError):
        oracle.attend(rand(1, 2, 1, 8), rand(1, 2, 4, 8), rand(1, 2, 4, 8), kv_lens=5)  # > s_cap


@pytest.mark.parametrize("nthreads", [1, 3])
def test_thread_count_does_not_change_results(nthreads):
    q = rand(2, 8, 5, 16)
    k = rand(2, 2, 20, 16)
    v = rand(2, 2, 20, 16)
    a = oracle.attend(q, k, v, causal=True, scale=0.3, nthreads=nthreads)
    b = oracle.attend(q, k, v, causal=True, scale=0.3, nthreads=0)
    assert np.array_equal(a, b)


def test_exhaustive_tiny_causal_masks():
    # every (Tq, Tk) with 1 <= Tq <= Tk <= 6, checked against the brute force
    for tq, tk in itertools.product(range(1, 7), range(1, 7)):
        if tq > tk:
            continue
        q = rand(1, 2, tq, 3)
        k = rand(1, 1, tk, 3)
        v = rand(1, 1, tk, 3)
        got = oracle.attend(q, k, v, causal=True, scale=1.1)
        want = brute_force(q, k, v, [tk], True, 1.1)
        np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)
