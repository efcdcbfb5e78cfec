"""Fractions at and around every rounding tie of an area slice, and the
slice coordinate they must give, found by search.

An area fraction f of an extent n lands on a tie when f*n is an exact half,
f = (2k+1)/(2n).  Such a fraction is a float64 only when 2n divides a power of
two times 2k+1; otherwise the float64 values next to it fall just below and
just above the tie.  For every tie with k < n this yields the float64 nearest
to it and its two float64 neighbours.
"""
from __future__ import annotations

import math
from fractions import Fraction


def near_tie_fractions(n: int):
    out = []
    for k in range(n):
        t = Fraction(2 * k + 1, 2 * n)
        f = float(t)
        out += [math.nextafter(f, -math.inf), f, math.nextafter(f, math.inf)]
    return out


def nearest_by_search(f: float, n: int) -> int:
    """The integer m with m - 1/2 <= f*n < m + 1/2 (f*n taken exactly): the
    nearest integer, a tie going to the larger one.  Found by bisection over
    the candidates -1 .. n + 1 for the first m with f*n < m + 1/2 (a monotone
    test in m), then checked against the lower bound."""
    v = Fraction(f) * n
    num, den = v.numerator, v.denominator
    lo, hi = -1, n + 1                      # f*n < hi + 1/2 holds for f < 1
    assert 2 * num < (2 * hi + 1) * den and not 2 * num < (2 * (lo - 1) + 1) * den
    while lo < hi:
        mid = (lo + hi) // 2
        if 2 * num < (2 * mid + 1) * den:
            hi = mid
        else:
            lo = mid + 1
    assert (2 * lo - 1) * den <= 2 * num < (2 * lo + 1) * den
    return lo
