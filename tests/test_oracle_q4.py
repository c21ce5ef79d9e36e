"""Pins for the oracle's 4-bit group-affine functions (no GPU).

Layout and formula (VeloxQuant-MLX "attention" posts: the fused group-affine
decode kernel takes codes, per-group scales and biases and the group size):
element 2j of a row sits in the low nibble of byte j, element 2j+1 in the
high nibble; the value of code c in a group with f16 scale s and bias b is
s*c + b rounded once to float32.

Pins:
* nibble order: a hand-written fixture (tests/golden/q4_nibbles.txt) and a
  round trip against the input generator's independent numpy packer over all
  256 byte values;
* f16 -> f32 widening: numpy's own float16 cast over all 65536 bit patterns;
* dequant: an independent route (numpy float64 product and sum, one cast to
  float32 -- exact in float64 for every input used here, so the cast is the
  only rounding) bit for bit, including codes 0 and 15 and zero scales;
* the encoder + dequant round trip stays within half a quantization step
  (plus the f16 rounding of the bias and scale).
"""

import os

import numpy as np
import pytest

import oracle
from workloads import gen

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "q4_nibbles.txt")


def test_nibble_fixture():
    with open(GOLDEN) as f:
        rows = [ln.split() for ln in f if ln.strip() and not ln.startswith("#")]
    for byte_hex, lo, hi in rows:
        codes = oracle.q4_unpack(np.array([[int(byte_hex, 16)]], np.uint8))
        assert codes.tolist() == [[int(lo), int(hi)]]


def test_unpack_all_bytes_round_trip():
    allbytes = np.arange(256, dtype=np.uint8).reshape(1, 256)
    codes = oracle.q4_unpack(allbytes)
    assert codes.shape == (1, 512)
    assert codes.max() <= 15
    assert np.array_equal(gen.q4_pack_codes(codes), allbytes)


def test_unpack_random_codes_round_trip():
    rng = np.random.default_rng(7)
    codes = rng.integers(0, 16, size=(5, 3, 128), dtype=np.uint8)
    assert np.array_equal(oracle.q4_unpack(gen.q4_pack_codes(codes)), codes)


def test_f16_widening_matches_numpy_for_every_bit_pattern():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    h = bits.view(np.float16)
    got = oracle.f16_to_f32(h)
    want = h.astype(np.float32)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), want[~nan].view(np.uint32))


def _independent_dequant(codes, scales, biases, group):
    s = scales.astype(np.float64)
    b = biases.astype(np.float64)
    D = codes.shape[-1]
    sg = np.repeat(s, group, axis=-1)[..., :D]
    bg = np.repeat(b, group, axis=-1)[..., :D]
    return (sg * codes.astype(np.float64) + bg).astype(np.float32)


@pytest.mark.parametrize("group", [64, 32, 128])
def test_dequant_bit_exact_against_independent_route(group):
    rng = np.random.default_rng(11)
    D = 128
    codes = rng.integers(0, 16, size=(4, 8, D), dtype=np.uint8)
    codes[0, 0, :] = 0
    codes[0, 1, :] = 15
    scales = (rng.random((4, 8, D // group)) * 0.6).astype(np.float16)
    biases = (rng.standard_normal((4, 8, D // group)) * 2).astype(np.float16)
    scales[1, 2, 0] = 0.0
    got = oracle.q4_dequant(gen.q4_pack_codes(codes), scales, biases, group)
    want = _independent_dequant(codes, scales, biases, group)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
    # code 0 returns the bias itself; a zero scale returns the bias everywhere
    assert np.array_equal(got[0, 0], np.repeat(biases[0, 0].astype(np.float32), group))
    assert np.array_equal(got[1, 2, :group], np.full(group, np.float32(biases[1, 2, 0])))


def test_encoder_round_trip_error_bound():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((2, 8, 50, 128)).astype(np.float32)
    packed, scales, biases = gen.q4_encode(x, 64)
    xh = oracle.q4_dequant(packed, scales, biases, 64)
    s = np.repeat(scales.astype(np.float32), 64, axis=-1)
    mn = np.repeat(x.reshape(2, 8, 50, 2, 64).min(-1), 64, axis=-1)
    b = np.repeat(biases.astype(np.float32), 64, axis=-1)
    # half a step, the bias rounding, and the f16 rounding of the step
    # (up to 15 steps of relative error 2^-11)
    bound = 0.5 * s + np.abs(mn - b) + 15 * s * 2.0 ** -11 + 1e-6
    assert (np.abs(x - xh) <= bound).all()


def test_encoder_degenerate_group():
    x = np.full((1, 1, 1, 64), 0.3, np.float32)
    packed, scales, biases = gen.q4_encode(x, 64)
    assert scales[0, 0, 0, 0] == 0
    xh = oracle.q4_dequant(packed, scales, biases, 64)
    assert np.array_equal(xh, np.full((1, 1, 1, 64), np.float32(np.float16(0.3))))


def test_q4_attend_equals_attend_on_dequantized_cache():
    rng = np.random.default_rng(5)
    kx = rng.standard_normal((1, 2, 30, 128)).astype(np.float32)
    vx = rng.standard_normal((1, 2, 30, 128)).astype(np.float32)
    kc, ks, kb = gen.q4_encode(kx, 64)
    vc, vs, vb = gen.q4_encode(vx, 64)
    q = rng.standard_normal((1, 16, 1, 128)).astype(np.float16)
    got = oracle.q4_attend(q, kc, ks, kb, vc, vs, vb, 64, kv_lens=21)
    k = oracle.q4_dequant(kc, ks, kb, 64)
    v = oracle.q4_dequant(vc, vs, vb, 64)
    want = oracle.attend(q.astype(np.float64), k[:, :, :21], v[:, :, :21])
    assert np.array_equal(got, want)
