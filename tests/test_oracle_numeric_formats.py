"""Pins for the oracle's FP8 E4M3 codec and bfloat16 rounding.

E4M3 is pinned to the OCP OFP8 specification's fixed points (tests/golden)
and to an independent bit-level formulation written here; bfloat16 rounding
is pinned to PyTorch's CPU conversion.
"""

import json
import os

import numpy as np
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_e4m3_spec_points():
    spec = json.load(open(os.path.join(GOLDEN, "ofp8_e4m3_points.json")))
    for code, value in spec["points"]:
        got = oracle.e4m3_decode(int(code, 16))
        assert got == value and np.signbit(got) == np.signbit(value), code
    for code in spec["nan_codes"]:
        assert np.isnan(oracle.e4m3_decode(int(code, 16)))


def test_e4m3_decode_structure():
    pos = oracle.e4m3_decode(np.arange(0x7F))
    assert np.all(np.diff(pos) > 0), "positive codes are monotone"
    neg = oracle.e4m3_decode(np.arange(0x80, 0xFF))
    np.testing.assert_array_equal(neg, -pos)
    # every finite value is exactly representable in float32
    assert np.array_equal(pos.astype(np.float32).astype(np.float64), pos)


def test_e4m3_encode_round_trip_and_ties():
    codes = np.arange(0x7F)
    vals = oracle.e4m3_decode(codes)
    np.testing.assert_array_equal(oracle.e4m3_encode_rne(vals), codes)
    mids = (vals[:-1] + vals[1:]) / 2
    got = oracle.e4m3_encode_rne(mids)
    lower, upper = codes[:-1], codes[1:]
    expect = np.where(lower % 2 == 0, lower, upper)
    np.testing.assert_array_equal(got, expect)
    below = np.nextafter(mids, -np.inf)
    above = np.nextafter(mids, np.inf)
    np.testing.assert_array_equal(oracle.e4m3_encode_rne(below), lower)
    np.testing.assert_array_equal(oracle.e4m3_encode_rne(above), upper)


def _e4m3_bits_rne(x32):
    """Independent E4M3 encoder for float32 x in [0, 448] by integer rounding."""
    bits = x32.view(np.uint32).astype(np.int64)
    exp = (bits >> 23) & 0xFF
    out = np.empty(x32.shape, dtype=np.int64)
    normal = exp >= 127 - 6                      # x >= 2^-6
    # normal range: drop 20 mantissa bits with round-half-even, rebias 127 -> 7
    b = bits[normal]
    kept = b >> 20
    rem = b & 0xFFFFF
    up = (rem > 0x80000) | ((rem == 0x80000) & ((kept & 1) == 1))
    out[normal] = (kept + up) - ((127 - 7) << 3)
    # subnormal range: value = m * 2^-9, m = round-half-even(x * 2^9)
    sub = ~normal
    out[sub] = np.rint(x32[sub].astype(np.float64) * 512.0).astype(np.int64)
    return out.astype(np.uint8)


def test_e4m3_encode_matches_bit_rounding_on_unit_interval():
    rng = np.random.default_rng(1234)
    xs = [rng.random(200_000, dtype=np.float64).astype(np.float32),
          np.exp2(rng.uniform(-12, 0, 200_000)).astype(np.float32)]
    # every float32 in the subnormal-E4M3 range and just above it, densely
    lo = np.float32(2.0 ** -12).view(np.uint32)
    hi = np.float32(2.0 ** -5).view(np.uint32)
    xs.append(np.arange(lo, hi, 37, dtype=np.uint32).view(np.float32))
    x = np.concatenate(xs)
    x = x[(x > 0) & (x <= 1)]
    np.testing.assert_array_equal(oracle.e4m3_encode_rne(x), _e4m3_bits_rne(x))


def test_e4m3_relative_error_bound_in_normal_range():
    rng = np.random.default_rng(7)
    x = np.exp2(rng.uniform(-6, 0, 100_000))
    back = oracle.e4m3_decode(oracle.e4m3_encode_rne(x))
    assert np.max(np.abs(back - x) / x) <= 2.0 ** -4


def test_bf16_round_matches_torch():
    rng = np.random.default_rng(3)
    bits = rng.integers(0, 2 ** 32, 1_000_000, dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32)
    x = x[np.isfinite(x)]
    # add exact ties (low 16 bits == 0x8000) with odd and even kept parts
    ties = ((rng.integers(0, 2 ** 16, 10_000).astype(np.uint32) << 16) | 0x8000).view(np.float32)
    x = np.concatenate([x, ties[np.isfinite(ties)]])
    x = x[np.abs(x) < 3.3e38]  # keep away from overflow to infinity
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    np.testing.assert_array_equal(oracle.bf16_round(x).view(np.uint32), ref.view(np.uint32))
