"""Pins for the oracle's min-max 4-bit quantizer and its float16 rounding (no GPU).

The quantizer (oracle.q4_quantize, gqa_oracle_q4_quantize in C) encodes a
new cache row the way the incremental append does (VeloxQuant-MLX
"attention" posts, "Part 4": only newly aged rows are quantized): per group,
scale = f16((max - min) / 15), bias = f16(min), code = clamp(rint((x -
bias) / scale), 0, 15) in float32, ties to even, code 0 for a zero scale.

Pins:
* float32 -> float16 rounding against numpy's cast (a library routine):
  every float16 value round-trips; random values across the whole range and
  both signs; every midpoint between neighbouring float16 values (ties to
  even); the subnormal range; the overflow threshold;
* hand-computed groups (tests/golden/q4_quantize.txt): exact ramps, negative
  values, a shuffled order, a constant group, ties to even, a wide range;
* invariants on random inputs: codes are monotone in x within a group, the
  decoded value is within half a step (plus the f16 rounding of scale and
  bias) of x, the group minimum gets code 0 when its bias is exact;
* agreement with a float32 numpy route written here from the same steps.
"""

import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "q4_quantize.txt")


def test_f16_rounding_round_trips_every_f16_value():
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16).view(np.float16)
    x = h.astype(np.float32)
    got = oracle.f32_to_f16(x)
    finite = np.isfinite(x)
    assert np.array_equal(got[finite].view(np.uint16), h[finite].view(np.uint16))
    assert np.isnan(got[np.isnan(x)]).all()


def test_f16_rounding_matches_numpy_on_random_and_edge_values():
    rng = np.random.default_rng(0)
    mag = np.exp2(rng.uniform(-30, 17, 200000)).astype(np.float32)
    x = np.concatenate([mag, -mag])
    # every midpoint between consecutive finite positive float16 values
    h = np.arange(0, 0x7BFF, dtype=np.uint16).view(np.float16).astype(np.float64)
    mids = ((h[:-1] + h[1:]) / 2).astype(np.float32)
    edges = np.array([65504, 65519.996, 65520, 65536, 1e9, 2.0 ** -24, 2.0 ** -25, 3 * 2.0 ** -26, 2.0 ** -26,
                      6.0975552e-05, 6.1035156e-05, 0.0, -0.0, np.inf, -np.inf], np.float32)
    x = np.concatenate([x, mids, -mids, edges])
    with np.errstate(over="ignore"):
        want = x.astype(np.float16)
    got = oracle.f32_to_f16(x)
    assert np.array_equal(got.view(np.uint16), want.view(np.uint16))


def _golden():
    for ln in open(GOLDEN):
        if not ln.strip() or ln.startswith("#"):
            continue
        name, xs, sc, bi, cs = [f.strip() for f in ln.split("|")]
        yield (name, np.array(xs.split(), np.float32), float(sc), float(bi), np.array(cs.split(), np.uint8))


@pytest.mark.parametrize("case", list(_golden()), ids=lambda c: c[0])
def test_hand_computed_groups(case):
    name, x, sc, bi, codes = case
    packed, s, b = oracle.q4_quantize(x[None, :], 16)
    assert float(s[0, 0]) == sc and float(b[0, 0]) == bi
    assert np.array_equal(oracle.q4_unpack(packed)[0], codes)


def test_invariants_on_random_rows():
    rng = np.random.default_rng(1)
    for group in (32, 64, 128):
        x = (rng.standard_normal((300, 128)) * rng.uniform(0.01, 50, (300, 1))).astype(np.float16).astype(np.float32)
        packed, s, b = oracle.q4_quantize(x, group)
        c = oracle.q4_unpack(packed).astype(np.int64)
        xg = x.reshape(300, -1, group)
        cg = c.reshape(300, -1, group)
        s32 = s.astype(np.float32)[..., None]
        b32 = b.astype(np.float32)[..., None]
        # monotone codes within a group
        order = np.argsort(xg, axis=-1, kind="stable")
        assert (np.diff(np.take_along_axis(cg, order, -1), axis=-1) >= 0).all()
        # decoded value within half a step plus the f16 rounding of scale and bias
        lo = xg.min(-1, keepdims=True)
        hi = xg.max(-1, keepdims=True)
        step = (hi - lo) / 15
        dec = s32 * cg + b32
        slack = 0.5 * s32 + np.abs(lo - b32) + 15 * np.abs(s32 - step) + 1e-6 * np.abs(xg)
        assert (np.abs(xg - dec) <= slack).all()
        # the minimum gets code 0 where the bias is exact
        exact = (b32 == lo)[..., 0]
        mins = np.take_along_axis(cg, np.argmin(xg, -1)[..., None], -1)[..., 0]
        assert (mins[exact] == 0).all()


def test_matches_a_float32_numpy_route():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((500, 128)).astype(np.float16).astype(np.float32)
    x[0, :64] = 0.75  # a degenerate group
    group = 64
    xg = x.reshape(500, 2, group)
    lo, hi = xg.min(-1), xg.max(-1)
    s16 = ((hi - lo) / np.float32(15)).astype(np.float16)
    b16 = lo.astype(np.float16)
    s32, b32 = s16.astype(np.float32)[..., None], b16.astype(np.float32)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        c = np.rint((xg - b32) / s32)
    c = np.clip(np.where(s32 == 0, 0, c), 0, 15).astype(np.uint8).reshape(500, 128)
    packed, s, b = oracle.q4_quantize(x, group)
    assert np.array_equal(s.view(np.uint16), s16.view(np.uint16))
    assert np.array_equal(b.view(np.uint16), b16.view(np.uint16))
    assert np.array_equal(oracle.q4_unpack(packed), c)


def test_kv_append_definition():
    cache = np.arange(2 * 3 * 6 * 2, dtype=np.float32).reshape(2, 3, 6, 2)
    new = -np.arange(2 * 3 * 4 * 2, dtype=np.float32).reshape(2, 3, 4, 2) - 1
    out, lens = oracle.kv_append(cache, new, [1, 4])
    assert lens.tolist() == [5, 6]
    assert np.array_equal(out[0, :, 1:5], new[0])
    assert np.array_equal(out[1, :, 4:6], new[1, :, :2])   # rows past the capacity are dropped
    assert np.array_equal(out[0, :, :1], cache[0, :, :1]) and np.array_equal(out[0, :, 5:], cache[0, :, 5:])
    assert np.array_equal(out[1, :, :4], cache[1, :, :4])
    out2, lens2 = oracle.kv_append(cache, new, [-3, 99])   # lengths clamp to [0, capacity]
    assert lens2.tolist() == [4, 6] and np.array_equal(out2[0, :, :4], new[0]) and np.array_equal(out2[1], cache[1])


def test_signed_zeros_have_one_encoding():
    # a group of zeros of both signs: scale and bias are +0, codes 0; a group
    # whose minimum is -0 stores its bias as +0
    x = np.zeros((2, 16), np.float32)
    x[0, ::2] = -0.0
    x[1] = np.arange(16, dtype=np.float32)
    x[1, 0] = -0.0
    packed, s, b = oracle.q4_quantize(x, 16)
    assert s.view(np.uint16).tolist() == [[0], [np.float16(1.0).view(np.uint16)]]
    assert b.view(np.uint16).tolist() == [[0], [0]]
    assert oracle.q4_unpack(packed).tolist() == [[0] * 16, list(range(16))]
