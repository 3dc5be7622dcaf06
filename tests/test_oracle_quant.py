"""Pins for the oracle's quantiser, double quantisation, dequantisation and
storage arithmetic.

Independent formulations used here: the level table from scipy's ndtri, the
nearest level by counting fp64 midpoints below x (instead of the oracle's
argmin of distances), exhaustive enumeration of bfloat16 inputs, the pages'
storage figures (tests/golden/pages_storage_figures.json) and invariants the
method implies.
"""

import json
import os

import numpy as np
import pytest
from scipy import special

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _scipy_levels32():
    d = oracle.DELTA
    pos = [special.ndtri(0.5 + j * (d - 0.5) / 8) for j in range(1, 9)]
    neg = [-special.ndtri(0.5 + j * (d - 0.5) / 7) for j in range(1, 8)]
    top = special.ndtri(d)
    return np.array(sorted([0.0] + [v / top for v in pos + neg])).astype(np.float32)


Q = _scipy_levels32()
MID = (Q[:-1].astype(np.float64) + Q[1:].astype(np.float64)) / 2


def _codes_by_midpoints(w, c):
    """Number of midpoints strictly below x = fp32(w / c); a tie goes down."""
    x = (w.astype(np.float32) / np.float32(c)).astype(np.float32).astype(np.float64)
    return np.searchsorted(MID, x, side="left").astype(np.uint8)


def _all_bf16_values():
    bits = (np.arange(1 << 16, dtype=np.uint32) << 16)
    v = bits.view(np.float32)
    return v[np.isfinite(v)]


def _blocks_with_max(c, values):
    """Blocks of 64 whose first element is c, filled with ``values``."""
    per = 63
    nb = -(-values.size // per)
    fill = np.zeros(nb * per, dtype=np.float32)
    fill[:values.size] = values
    blocks = np.concatenate([np.full((nb, 1), c, dtype=np.float32), fill.reshape(nb, per)], axis=1)
    return blocks.ravel()


@pytest.mark.parametrize("c", [1.0, 0.0078125, 0.02001953125, 3.140625, 1.5e-3, 57344.0, -0.6875])
def test_codes_exhaustive_over_bf16_inputs(c):
    allv = _all_bf16_values()
    cabs = np.float32(abs(c))
    vals = allv[np.abs(allv) <= cabs]
    w = _blocks_with_max(np.float32(c), vals)
    packed, c2, c1 = oracle.quantize_nf4_dq(w)
    codes = oracle.unpack_codes(packed, w.size)
    np.testing.assert_array_equal(codes, _codes_by_midpoints(w, cabs))


def test_invariants_on_gaussian_blocks():
    rng = np.random.default_rng(11)
    w = oracle.bf16_round((rng.standard_normal(64 * 1000) * 0.02).astype(np.float32))
    packed, c2, c1 = oracle.quantize_nf4_dq(w)
    codes = oracle.unpack_codes(packed, w.size).reshape(-1, 64)
    blocks = w.reshape(-1, 64)
    absmax = np.abs(blocks).max(axis=1)
    # the element that sets the absmax maps to an end of the range
    at_max = np.abs(blocks) == absmax[:, None]
    assert np.all(np.isin(codes[at_max], [0, 15]))
    assert np.all(codes[(blocks == absmax[:, None])] == 15)
    assert np.all(codes[(blocks == -absmax[:, None])] == 0)
    # codes are monotone in w inside every block
    for b in range(0, 1000, 97):
        order = np.argsort(blocks[b], kind="stable")
        assert np.all(np.diff(codes[b][order].astype(int)) >= 0)
    # the chosen level is never further than half the widest gap
    x = (blocks / absmax[:, None]).astype(np.float32)
    assert np.max(np.abs(x - Q[codes])) <= np.max(np.diff(Q)) / 2 + 1e-7
    # zero weights take the exact zero
    assert np.all(codes[blocks == 0] == 7)


def test_nibble_order_and_hand_example():
    # block absmax 1: x = w. 0.5 lies between 0.4407 (code 12) and 0.5626
    # (code 13) and is closer to the first.
    w = np.zeros(64, dtype=np.float32)
    w[:6] = [1.0, -1.0, 0.0, 0.5, -0.5, 0.25]
    packed, c2, c1 = oracle.quantize_nf4_dq(w)
    assert packed[0] == (15 | (0 << 4))
    assert packed[1] == (7 | (12 << 4))
    # -0.5: between -0.5251 (code 2) and -0.3949 (code 3); 0.0251 vs 0.1051
    # 0.25: between 0.2461 (code 10) and 0.3379 (code 11)
    assert packed[2] == (2 | (10 << 4))
    assert np.all(packed[3:] == 0x77)
    assert c1[0] == 1.0 and c2[0] == 0x38  # ratio 1 -> E4M3 1.0


def test_short_final_block_and_group():
    rng = np.random.default_rng(5)
    for n in [1, 2, 63, 65, 127, 16383, 16385, 16384 + 64 * 3 + 1]:
        w = oracle.bf16_round(rng.standard_normal(n).astype(np.float32))
        packed, c2, c1 = oracle.quantize_nf4_dq(w)
        nb = -(-n // 64)
        assert packed.size == -(-n // 2) and c2.size == nb and c1.size == -(-nb // 256)
        if n % 2:
            assert packed[-1] >> 4 == 0, "pad nibble is zero"
        codes = oracle.unpack_codes(packed, n)
        tail = w[(nb - 1) * 64:]
        cm = np.abs(tail).max()
        np.testing.assert_array_equal(codes[(nb - 1) * 64:], _codes_by_midpoints(tail, cm))
        # the short group's constant is the max over the blocks present
        last_group = np.abs(w[(c1.size - 1) * 16384:]).max()
        assert c1[-1] == last_group


def test_double_quantisation_constants():
    rng = np.random.default_rng(9)
    n = 16384 * 3
    w = oracle.bf16_round((rng.standard_normal(n) * 0.02).astype(np.float32))
    w[16384:2 * 16384] = 0.0                       # an all-zero group
    w[2 * 16384: 2 * 16384 + 64] = 0.0             # an all-zero block in a live group
    packed, c2, c1 = oracle.quantize_nf4_dq(w)
    absmax = np.abs(w).reshape(-1, 64).max(axis=1)
    np.testing.assert_array_equal(c1, absmax.reshape(3, 256).max(axis=1))
    assert c1[1] == 0 and np.all(c2[256:512] == 0)
    assert c2[512] == 0
    codes = oracle.unpack_codes(packed, n)
    assert np.all(codes[16384:2 * 16384 + 64] == 7)
    live = absmax > 0
    chat = oracle.e4m3_decode(c2) * np.repeat(c1, 256)
    with np.errstate(invalid="ignore", divide="ignore"):
        ratio = absmax / np.repeat(c1, 256)
    normal = live & (ratio >= 2.0 ** -6)
    assert np.all(np.abs(chat[normal] - absmax[normal]) <= 2.0 ** -4 * absmax[normal])
    # the block holding the group maximum stores exactly 1.0
    for g in (0, 2):
        b = g * 256 + np.argmax(absmax[g * 256:(g + 1) * 256])
        assert c2[b] == 0x38


def test_storage_arithmetic_matches_pages():
    figs = json.load(open(os.path.join(GOLDEN, "pages_storage_figures.json")))
    n = 64 * 256 * 1000
    assert 32.0 / oracle.NF4_BLOCK == figs["fp32_constants_block64_bits_per_param"]["value"]
    dq_overhead = oracle.storage_bits_per_param(n) - 4.0
    saving = figs["fp32_constants_block64_bits_per_param"]["value"] - dq_overhead
    f = figs["dq_saving_bits_per_param"]
    assert abs(saving - f["value"]) <= f["tolerance"]
    assert saving == 0.5 - (8.0 / 64 + 32.0 / (64 * 256))
    g = figs["dq_saving_bytes_65b"]
    assert abs(g["params"] * saving / 8 - g["value"]) <= g["tolerance"]
    h = figs["finetune_65b_single_gpu_bytes_upper"]
    assert h["params"] * oracle.storage_bits_per_param(n) / 8 < h["value"]
    k = figs["weights_7b_4bit_bytes_about"]
    assert abs(k["params"] * oracle.storage_bits_per_param(n) / 8 - k["value"]) <= k["tolerance"]


def test_dequant_exact_with_power_of_two_constants():
    # every block has absmax 2^-3, so c2 = E4M3(1.0), c1 = 2^-3 and every
    # dequantised weight is exactly level * 2^-3
    rng = np.random.default_rng(2)
    n = 16384
    w = oracle.bf16_round((rng.uniform(-1, 1, n) * 0.125).astype(np.float32))
    w[::64] = 0.125
    packed, c2, c1 = oracle.quantize_nf4_dq(w)
    assert np.all(c2 == 0x38) and c1[0] == 0.125
    W = oracle.dequant(packed, c2, c1, n)
    codes = oracle.unpack_codes(packed, n)
    np.testing.assert_array_equal(W, Q[codes] * np.float32(0.125))


def test_dequant_requantise_is_idempotent_and_error_band():
    rng = np.random.default_rng(4)
    n = 16384 * 4
    w = oracle.bf16_round((rng.standard_normal(n) * 0.02).astype(np.float32))
    packed, c2, c1 = oracle.quantize_nf4_dq(w)
    W = oracle.dequant(packed, c2, c1, n)
    Wt = oracle.bf16_round(W)
    packed2, _, _ = oracle.quantize_nf4_dq(Wt)
    np.testing.assert_array_equal(packed2, packed)
    rel = np.sqrt(np.mean((W - w) ** 2) / np.mean(w ** 2))
    assert 0.07 < rel < 0.12, rel
    # the block maximum is reconstructed as +-c_hat
    chat = (oracle.e4m3_decode(c2).astype(np.float32) * np.repeat(c1, 256)).astype(np.float32)
    blocks = W.reshape(-1, 64)
    np.testing.assert_array_equal(np.abs(blocks).max(axis=1), chat)
