"""Exact-arithmetic helpers for pinning the oracle: rational values rounded
correctly to binary32, and functions evaluated with ``decimal`` at 60 digits.
None of this shares code with the oracle or the GPU library."""
from __future__ import annotations

import decimal
from fractions import Fraction

import numpy as np

_D = decimal.Context(prec=60)
F32 = np.float32


def _neighbors(v: np.float32):
    return (np.nextafter(v, F32(-np.inf), dtype=F32), v,
            np.nextafter(v, F32(np.inf), dtype=F32))


def f32_nearest(q: Fraction) -> np.float32:
    """The binary32 value nearest to the rational ``q`` (ties to even)."""
    c = F32(float(q))
    best = None
    for v in _neighbors(c):
        if not np.isfinite(v):
            continue
        dist = abs(Fraction(float(v)) - q)
        even = int(np.array(v, F32).view(np.uint32)) & 1 == 0
        key = (dist, not even)
        if best is None or key < best[0]:
            best = (key, v)
    return best[1]


def near_f32_midpoint(q: Fraction, rel: float = 1e-12) -> bool:
    """True when ``q`` lies within ``rel`` (relative) of a point halfway
    between two binary32 neighbours -- where a binary64 intermediate may
    legitimately round the other way."""
    v = f32_nearest(q)
    lo, _, hi = _neighbors(v)
    for n in (lo, hi):
        mid = (Fraction(float(v)) + Fraction(float(n))) / 2
        if q == 0:
            continue
        if abs(mid - q) <= abs(q) * Fraction(rel):
            return True
    return False


def matches_f32(got, q: Fraction) -> bool:
    """``got`` is the correctly rounded binary32 of ``q``, or ``q`` is so close
    to a rounding midpoint that a binary64 evaluation may round either way."""
    want = f32_nearest(q)
    return F32(got) == want or near_f32_midpoint(q)


def dec(x) -> decimal.Decimal:
    return _D.create_decimal_from_float(float(x))


def sigmoid_exact(l) -> Fraction:
    """1/(1+exp(-l)) to 60 significant digits, as a Fraction."""
    z = _D.divide(decimal.Decimal(1), _D.add(decimal.Decimal(1), _D.exp(-dec(l))))
    return Fraction(z)


def silu_exact(g) -> Fraction:
    z = dec(g)
    return Fraction(_D.divide(z, _D.add(decimal.Decimal(1), _D.exp(-z))))
