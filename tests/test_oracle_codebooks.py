"""Pins of the oracle's other 4-bit data types and of the format without
double quantisation.

The pages compare NF4 with 4-bit Integers and 4-bit Floats ("QLoRA: Efficient
Finetuning of Quantized LLMs", Introduction, contribution (1)) without
defining them, and price the format without double quantisation at 32/64 =
0.5 bit per weight ("Method", paragraph "Double Quantization"). What pins the
oracle here is fixed outside it: the OCP microscaling specification's E2M1
value table (typed below), textbook integer rounding, brute force over the
exact value grid, the pages' storage figures (tests/golden) and the pages'
ordering claim.
"""

import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")

# OCP Microscaling Formats (MX) v1.0, FP4 E2M1: value of each bit pattern
# 0b0000 .. 0b1111 (sign, 2 exponent bits, 1 mantissa bit).
E2M1_TABLE = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0,
              -0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0]


def _bf16_normal(n, sigma, seed):
    rng = np.random.default_rng(seed)
    return oracle.bf16_round((rng.standard_normal(n) * sigma).astype(np.float32))


def test_int4_levels_closed_form():
    q = oracle.int4_levels()
    assert q.dtype == np.float32 and q.size == 16
    for k in range(15):
        assert q[k] == np.float32((k - 7) / 7.0)
        assert abs(7.0 * float(q[k]) - (k - 7)) <= 2.0 ** -21
        assert q[14 - k] == -q[k]
    assert q[7] == 0.0 and not np.signbit(q[7])
    assert q[14] == 1.0 and q[15] == 1.0 and q[0] == -1.0
    assert np.all(np.diff(q[:15]) > 0)


def test_e2m1_decode_matches_ocp_table():
    for code in range(16):
        v = oracle.e2m1_decode(code)
        assert v == E2M1_TABLE[code]
        assert np.signbit(v) == np.signbit(E2M1_TABLE[code])


def test_fp4_levels_are_the_e2m1_grid_over_6():
    q = oracle.fp4_levels()
    assert q.dtype == np.float32 and q.size == 16
    grid = sorted({v + 0.0 for v in E2M1_TABLE})
    assert len(grid) == 15
    for k in range(15):
        assert q[k] == np.float32(grid[k] / 6.0)
    assert q[7] == 0.0 and not np.signbit(q[7])
    assert q[15] == q[14] == 1.0 and q[0] == -1.0


@pytest.mark.parametrize("name", ["nf4", "int4", "fp4"])
def test_codebook_lookup(name):
    q = oracle.codebook_levels(name)
    assert q[7] == 0.0 and q[0] == -1.0 and q[15] == 1.0
    with pytest.raises(ValueError):
        oracle.codebook_levels("int8")


def _weights_with_edge_blocks(seed):
    w = _bf16_normal(64 * 300 + 37, 0.02, seed)
    w[64:128] = 0.0                       # all-zero block
    w[128:192] = np.float32(0.0625)       # constant block: every x = 1
    w[192:256] = -np.abs(w[192:256])      # one-signed block
    return w


def test_int4_codes_are_textbook_integer_rounding():
    w = _weights_with_edge_blocks(1)
    packed, absmax = oracle.quantize_blockwise(w, oracle.int4_levels())
    codes = oracle.unpack_codes(packed, w.size).astype(np.int64)
    # textbook absmax integer quantisation: round(7 w / absmax) in [-7, 7]
    blk = np.arange(w.size) // 64
    c = np.abs(np.pad(w, (0, (-w.size) % 64)).reshape(-1, 64)).max(axis=1)[blk]
    live = c > 0
    x = np.zeros_like(w)
    x[live] = (w[live] / c[live]).astype(np.float32)
    ref = np.clip(np.rint(7.0 * x.astype(np.float64)), -7, 7).astype(np.int64) + 7
    # away from the half-integer boundaries the two definitions agree exactly
    frac = np.abs(7.0 * x.astype(np.float64) - np.floor(7.0 * x.astype(np.float64)) - 0.5)
    clear = frac > 1e-5
    assert clear.mean() > 0.99
    assert np.array_equal(codes[clear], ref[clear])
    assert np.all(codes[~live] == 7)
    assert not np.any(codes == 15)


def test_fp4_codes_nearest_on_exact_grid():
    w = _weights_with_edge_blocks(2)
    packed, absmax = oracle.quantize_blockwise(w, oracle.fp4_levels())
    codes = oracle.unpack_codes(packed, w.size)
    grid = np.array(sorted({v + 0.0 for v in E2M1_TABLE})) / 6.0  # exact in float64
    blk = np.arange(w.size) // 64
    c = absmax[blk]
    live = c > 0
    x = np.zeros(w.size, dtype=np.float64)
    x[live] = (w[live] / c[live]).astype(np.float32)
    d = np.abs(x[:, None] - grid[None, :])
    order = np.sort(d, axis=1)
    clear = (order[:, 1] - order[:, 0]) > 1e-6
    assert np.array_equal(codes[clear], np.argmin(d, axis=1)[clear])
    assert np.all(codes[~live] == 7)
    assert not np.any(codes == 15)


@pytest.mark.parametrize("name", ["int4", "fp4"])
def test_extremes_map_to_plus_minus_one(name):
    lv = oracle.codebook_levels(name)
    w = np.zeros(128, dtype=np.float32)
    w[5] = 0.5                  # block 0: max at +0.5
    w[70] = -0.25               # block 1: max magnitude negative
    packed, absmax = oracle.quantize_blockwise(w, lv)
    codes = oracle.unpack_codes(packed, 128)
    assert codes[5] == 14 and codes[70] == 0
    assert np.all(np.delete(codes, [5, 70]) == 7)
    assert absmax[0] == 0.5 and absmax[1] == 0.25


@pytest.mark.parametrize("name", ["nf4", "int4", "fp4"])
def test_blockwise_absmax_is_brute_force_max(name):
    w = _weights_with_edge_blocks(3)
    _, absmax = oracle.quantize_blockwise(w, oracle.codebook_levels(name))
    for b in range(absmax.size):
        blk = w[64 * b: 64 * (b + 1)]
        assert absmax[b] == max(abs(float(v)) for v in blk)


@pytest.mark.parametrize("name", ["nf4", "int4", "fp4"])
def test_blockwise_dequant_exact_and_round_trip(name):
    lv = oracle.codebook_levels(name)
    rng = np.random.default_rng(4)
    n = 64 * 40
    codes = rng.integers(0, 15, n).astype(np.uint8)
    packed = (codes[0::2] | (codes[1::2] << 4)).astype(np.uint8)
    absmax = np.exp2(rng.integers(-20, 5, n // 64)).astype(np.float32)
    d = oracle.dequant_blockwise(packed, absmax, n, lv)
    # power-of-two constants: the product is exact
    assert np.array_equal(d.astype(np.float64), lv[codes].astype(np.float64) * absmax[np.arange(n) // 64])
    # quantising the dequantised weights of a real quantisation reproduces its codes
    w = _bf16_normal(64 * 50 + 9, 0.02, 5)
    p1, a1 = oracle.quantize_blockwise(w, lv)
    d1 = oracle.dequant_blockwise(p1, a1, w.size, lv)
    p2, a2 = oracle.quantize_blockwise(d1, lv)
    assert np.array_equal(p1, p2) and np.array_equal(a1, a2)


def test_blockwise_codes_equal_double_quant_codes():
    # double quantisation only changes how the constants are stored
    w = _weights_with_edge_blocks(6)
    for name in ("nf4", "int4", "fp4"):
        lv = oracle.codebook_levels(name)
        p1, _ = oracle.quantize_blockwise(w, lv)
        p2, _, _ = oracle.quantize_nf4_dq(w, levels=lv)
        assert np.array_equal(p1, p2)


def test_storage_without_double_quant_matches_pages():
    figs = json.load(open(os.path.join(GOLDEN, "pages_storage_figures.json")))
    n = 64 * 256 * 40
    const_bits = oracle.storage_bits_per_param(n, double_quant=False) - 4.0
    assert const_bits == figs["fp32_constants_block64_bits_per_param"]["value"]
    saving = oracle.storage_bits_per_param(n, double_quant=False) - oracle.storage_bits_per_param(n)
    f = figs["dq_saving_bits_per_param"]
    assert abs(saving - f["value"]) <= f["tolerance"]


@pytest.mark.parametrize("double_quant", [False, True])
def test_nf4_error_lower_than_int4_and_fp4_on_normal_weights(double_quant):
    # the pages' claim: NF4 is the better 4-bit type for zero-centred normal weights
    w = _bf16_normal(1 << 16, 0.02, 7)
    mse = {}
    for name in ("nf4", "int4", "fp4"):
        lv = oracle.codebook_levels(name)
        if double_quant:
            p, c2, c1 = oracle.quantize_nf4_dq(w, levels=lv)
            d = oracle.dequant(p, c2, c1, w.size, levels=lv)
        else:
            p, a = oracle.quantize_blockwise(w, lv)
            d = oracle.dequant_blockwise(p, a, w.size, lv)
        mse[name] = float(np.mean((d.astype(np.float64) - w) ** 2))
    assert mse["nf4"] < mse["fp4"] and mse["nf4"] < mse["int4"]
