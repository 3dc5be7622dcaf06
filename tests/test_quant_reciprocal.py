"""The quantiser's per-block reciprocal (csrc/quantize.hip, rcp_bf16).

The kernel forms RN32(w / c) by Markstein's correction, which needs r =
RN32(1 / c) exactly. It takes the hardware reciprocal y0 (within 1 ulp of
1 / c) and one Newton step with fused multiply-adds: e = RN32(1 - c y0),
r = RN32(y0 + e y0). The block max c is a bf16 value in [2^-100, 2^100], so
it has at most 8 significant bits, and the step commutes with power-of-two
scaling there: checking the 128 significands in [1, 2) with exact rational
arithmetic covers every c, for any start within 2 ulps (a wider band than the
hardware's guarantee). Host arithmetic only; no GPU.
"""

import math
from fractions import Fraction as F


def _exponent(q):
    e = math.floor(math.log2(q))
    while F(2) ** e > q:
        e -= 1
    while F(2) ** (e + 1) <= q:
        e += 1
    return e


def _rn32(q):
    """Round a nonzero rational to the nearest binary32 value (ties to even), normal range."""
    if q < 0:
        return -_rn32(-q)
    ulp = F(2) ** (_exponent(q) - 23)
    m = q / ulp
    fl = math.floor(m)
    rem = m - fl
    if rem > F(1, 2) or (rem == F(1, 2) and fl % 2 == 1):
        fl += 1
    return fl * ulp


def _fma32(a, b, c):
    """binary32 fused multiply-add: one rounding of the exact a b + c."""
    t = a * b + c
    return F(0) if t == 0 else _rn32(t)


def _ulp(y):
    return F(2) ** (_exponent(y) - 23)


def test_refined_reciprocal_is_correctly_rounded_for_every_bf16_significand():
    bad = []
    for s in range(128, 256):
        c = F(s, 128)
        exact = 1 / c
        r = _rn32(exact)
        starts = {r}
        y = r
        for _ in range(2):  # two binary32 neighbours on each side
            y = y + _ulp(y)
            starts.add(y)
        y = r
        for _ in range(2):
            y = y - _ulp(y - _ulp(y) / 2)
            starts.add(y)
        for y0 in starts:
            e = _fma32(-c, y0, F(1))
            y1 = _fma32(e, y0, y0)
            if y1 != r:
                bad.append((s, float(y0)))
    assert not bad, bad[:5]


def test_the_two_starts_within_one_ulp_are_among_those_checked():
    # 1 / c for c = 1 + 1/128 lies strictly between two binary32 values; both
    # are within 1 ulp and both must be in the checked set above
    c = F(129, 128)
    exact = 1 / c
    r = _rn32(exact)
    lo = r if r < exact else r - _ulp(r - _ulp(r) / 2)
    hi = lo + _ulp(lo)
    assert lo < exact < hi and hi - lo == _ulp(lo)
    for y0 in (lo, hi):
        assert _fma32(_fma32(-c, y0, F(1)), y0, y0) == r
