"""Pins for the oracle's NF4 level table.

The construction is in "QLoRA: Efficient Finetuning of Quantized LLMs"
(inquiringlines.com), Method, paragraph "4-bit NormalFloat Quantization":
quantiles of N(0, 1), normalised into [-1, 1], asymmetric with 2^(k-1)
negative-side and 2^(k-1)+1 positive-side quantiles sharing one zero. The
checks below use library routines (scipy's ndtri/ndtr, mpmath's erfinv) that
share nothing with the oracle's bisection.
"""

import math

import mpmath
import numpy as np
import pytest
from scipy import special

import oracle

Q = oracle.nf4_levels()
Q64 = oracle.nf4_levels_f64()


def test_sixteen_values_exact_zero_and_range():
    assert Q.dtype == np.float32 and Q.shape == (16,)
    assert np.all(np.diff(Q) > 0), "strictly increasing"
    assert Q[0] == np.float32(-1.0) and Q[15] == np.float32(1.0)
    assert Q[7] == 0.0 and np.count_nonzero(Q == 0.0) == 1
    assert np.count_nonzero(Q < 0) == 7, "2^(k-1) negative-side quantiles, one zero removed"
    assert np.count_nonzero(Q > 0) == 8


def _levels_from(ppf):
    d = oracle.DELTA
    pos = [ppf(0.5 + j * (d - 0.5) / 8) for j in range(1, 9)]
    neg = [-ppf(0.5 + j * (d - 0.5) / 7) for j in range(1, 8)]
    top = ppf(d)
    return np.array(sorted([0.0] + [v / top for v in pos + neg]), dtype=np.float64)


def test_matches_scipy_ndtri():
    ref = _levels_from(lambda p: float(special.ndtri(p)))
    assert np.max(np.abs(ref - Q64)) <= 1e-14
    assert np.array_equal(ref.astype(np.float32), Q)


def test_matches_mpmath_high_precision_and_float32_is_unambiguous():
    mpmath.mp.dps = 50
    ppf = lambda p: mpmath.sqrt(2) * mpmath.erfinv(2 * mpmath.mpf(p) - 1)  # noqa: E731
    d = mpmath.mpf(1) - (mpmath.mpf(1) / 32 + mpmath.mpf(1) / 30) / 2
    pos = [ppf(mpmath.mpf(1) / 2 + j * (d - mpmath.mpf(1) / 2) / 8) for j in range(1, 9)]
    neg = [-ppf(mpmath.mpf(1) / 2 + j * (d - mpmath.mpf(1) / 2) / 7) for j in range(1, 8)]
    top = ppf(d)
    exact = sorted([mpmath.mpf(0)] + [v / top for v in pos + neg])
    for i, e in enumerate(exact):
        assert abs(float(e) - Q64[i]) <= 1e-15
        # The float32 rounding is far from a tie, so any accurate inverse CDF
        # yields this same float32 table.
        if e != 0 and abs(e) != 1:
            f = np.float32(float(e))
            ulp = float(np.spacing(np.float32(abs(f))))
            frac = abs(float(e) - float(f)) / ulp
            assert frac < 0.49, (i, frac)
        assert np.float32(float(e)) == Q[i]


def test_equal_probability_spacing_with_forward_cdf():
    """Phi(q * Phi^-1(delta)) is equally spaced: 8 steps above zero, 7 below."""
    z = float(special.ndtri(oracle.DELTA))
    p = special.ndtr(Q64 * z)
    d = oracle.DELTA - 0.5
    np.testing.assert_allclose(p[7:], 0.5 + np.arange(9) * d / 8, rtol=0, atol=1e-14)
    np.testing.assert_allclose(p[:8], 0.5 - np.arange(7, -1, -1) * d / 7, rtol=0, atol=1e-14)


@pytest.mark.parametrize("p", [0.5, 0.5000001, 0.6, 0.75, 0.9, 0.9677083333333334, 0.999, 1 - 1e-12])
def test_phi_inv_against_ndtri(p):
    # a perturbation of p by one ulp moves the quantile by ulp(p) / pdf(x)
    x = float(special.ndtri(p))
    pdf = math.exp(-x * x / 2) / math.sqrt(2 * math.pi)
    tol = 4 * np.spacing(p) / pdf + 1e-15
    assert abs(oracle.phi_inv(p) - x) <= tol


def test_phi_inv_is_an_inverse():
    for x in np.linspace(0.0, 5.0, 51):
        p = 0.5 * math.erfc(-x / math.sqrt(2))
        pdf = math.exp(-x * x / 2) / math.sqrt(2 * math.pi)
        assert abs(oracle.phi_inv(p) - x) <= 4 * np.spacing(p) / pdf + 1e-15
