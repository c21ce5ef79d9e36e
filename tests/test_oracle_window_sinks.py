"""Pins for the oracle's sliding window and attention sinks (no GPU).

Readings (the Fornace prefill page, "What this does not prove": the fused
kernel applies no sliding window, other models need one; the VeloxQuant-MLX
"attention" posts, "Part 4": the SDPA call the fused decode intercepts
carries `sinks`):
* window W: a query row sees only the W most recent keys up to its own
  position -- key j with last - W < j <= last, last = i + (n - Tq);
* sinks: one logit per query head, in the units of the scaled scores, that
  joins the softmax normaliser and adds no value row.

Pins:
* a numpy brute force with explicitly repeated KV heads, a full score
  matrix, a banded mask and the sink appended as one more softmax column;
* torch's float64 scaled_dot_product_attention with an explicit banded
  boolean mask (window, no sinks; a library routine);
* special cases: a window at least as long as the keys changes nothing (bit
  for bit); a window of 1 returns the diagonal key's value row exactly; a
  sink of -inf changes nothing (bit for bit); with all scores equal the
  output is sum(V) / (n + e^sink) over the n visible keys;
* decode with a window equals the last row of prefill with that window, bit
  for bit.
"""

import numpy as np
import pytest
import torch

import oracle


def brute(q, k, v, kv_lens, causal, scale, window, sinks):
    B, Hq, Tq, D = q.shape
    Hkv, S = k.shape[1], k.shape[2]
    G = Hq // Hkv
    kr = np.repeat(k, G, axis=1)
    vr = np.repeat(v, G, axis=1)
    out = np.zeros((B, Hq, Tq, D))
    for b in range(B):
        n = int(kv_lens[b])
        i = np.arange(Tq)[:, None]
        j = np.arange(S)[None, :]
        last = i + (n - Tq) if causal else np.full((Tq, 1), n - 1)
        vis = (j < n) & (j <= last)
        if window > 0:
            vis &= j > last - window
        sc = scale * np.einsum("hid,hjd->hij", q[b], kr[b])
        sc = np.where(vis[None], sc, -np.inf)
        sk = np.full((Hq, Tq, 1), -np.inf) if sinks is None else np.broadcast_to(np.asarray(sinks)[:, None, None],
                                                                                   (Hq, Tq, 1))
        full = np.concatenate([sc, sk], axis=-1)
        mx = full.max(-1, keepdims=True)
        e = np.exp(full - mx)
        p = e / e.sum(-1, keepdims=True)
        out[b] = np.einsum("hij,hjd->hid", p[..., :S], vr[b])
    return out


GEOMS = [(1, 2, 1, 3), (2, 6, 2, 4), (1, 4, 4, 2), (1, 8, 1, 5)]


@pytest.mark.parametrize("B,Hq,Hkv,D", GEOMS)
def test_window_and_sinks_match_brute_force(B, Hq, Hkv, D):
    rng = np.random.default_rng(B * 100 + Hq * 10 + D)
    S = 9
    for Tq in (1, 3, 9):
        for window in (0, 1, 2, 5, 9, 20):
            for use_sinks in (False, True):
                q = rng.standard_normal((B, Hq, Tq, D))
                k = rng.standard_normal((B, Hkv, S, D))
                v = rng.standard_normal((B, Hkv, S, D))
                lens = rng.integers(Tq, S + 1, size=B)
                sinks = rng.standard_normal(Hq) * 2 if use_sinks else None
                for causal in ((True, False) if Tq == 1 else (True,)):
                    got = oracle.attend(q, k, v, kv_lens=lens, causal=causal, scale=0.7, window=window, sinks=sinks)
                    want = brute(q, k, v, lens, causal, 0.7, window, sinks)
                    assert np.abs(got - want).max() <= 1e-12


def test_window_matches_torch_sdpa_with_banded_mask():
    rng = np.random.default_rng(11)
    B, Hq, Hkv, Tq, S, D, W = 1, 6, 2, 5, 12, 8, 4
    q = rng.standard_normal((B, Hq, Tq, D))
    k = rng.standard_normal((B, Hkv, S, D))
    v = rng.standard_normal((B, Hkv, S, D))
    i = torch.arange(Tq)[:, None] + (S - Tq)
    j = torch.arange(S)[None, :]
    mask = (j <= i) & (j > i - W)
    G = Hq // Hkv
    want = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(np.repeat(k, G, 1)), torch.from_numpy(np.repeat(v, G, 1)),
        attn_mask=mask, scale=0.3).numpy()
    got = oracle.attend(q, k, v, causal=True, scale=0.3, window=W)
    assert np.abs(got - want).max() <= 1e-12


def test_special_cases():
    rng = np.random.default_rng(12)
    B, Hq, Hkv, Tq, S, D = 2, 4, 2, 6, 10, 8
    q = rng.standard_normal((B, Hq, Tq, D))
    k = rng.standard_normal((B, Hkv, S, D))
    v = rng.standard_normal((B, Hkv, S, D))
    base = oracle.attend(q, k, v, causal=True, scale=0.5)
    assert np.array_equal(oracle.attend(q, k, v, causal=True, scale=0.5, window=S), base)
    assert np.array_equal(oracle.attend(q, k, v, causal=True, scale=0.5, window=10 ** 6), base)
    assert np.array_equal(oracle.attend(q, k, v, causal=True, scale=0.5, sinks=np.full(Hq, -np.inf)), base)
    one = oracle.attend(q, k, v, causal=True, scale=0.5, window=1)
    diag = np.repeat(v, Hq // Hkv, axis=1)[:, :, S - Tq:]
    assert np.array_equal(one, diag)
    # equal scores: sum of the visible values over (n + e^sink)
    z = np.zeros_like(q)
    sinks = np.array([0.0, 1.5, -2.0, 3.0])
    for W in (0, 3):
        got = oracle.attend(z, k, v, causal=True, scale=0.5, window=W, sinks=sinks)
        vr = np.repeat(v, Hq // Hkv, axis=1)
        for i in range(Tq):
            last = i + S - Tq
            lo = 0 if W == 0 else max(0, last - W + 1)
            n = last + 1 - lo
            want = vr[:, :, lo:last + 1].sum(2) / (n + np.exp(sinks))[None, :, None]
            assert np.abs(got[:, :, i] - want).max() <= 1e-13


def test_decode_with_window_is_the_last_prefill_row():
    rng = np.random.default_rng(13)
    B, Hq, Hkv, T, D = 1, 6, 3, 40, 16
    q = rng.standard_normal((B, Hq, T, D))
    k = rng.standard_normal((B, Hkv, T, D))
    v = rng.standard_normal((B, Hkv, T, D))
    sinks = rng.standard_normal(Hq)
    for W in (1, 7, 40, 100):
        full = oracle.attend(q, k, v, causal=True, window=W, sinks=sinks)
        dec = oracle.attend(q[:, :, -1:], k, v, causal=False, window=W, sinks=sinks)
        assert np.array_equal(dec[:, :, 0], full[:, :, -1])
