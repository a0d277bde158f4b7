"""Definitional bf16 rounding with exact rationals, for pinning the oracle.

Independent of the oracle's procedure: instead of scaling by an ulp, this
lists every finite non-negative bf16 value as an exact ``Fraction``, finds
the two neighbours of |x| by bisection and picks one by the mode's rule
(IEEE-754 roundTiesToEven, roundTiesToAway, roundTowardZero).
"""
from __future__ import annotations

import bisect
import math
from fractions import Fraction

import numpy as np

MAX_FINITE = 0x7F7F


def _bf16_value(bits: int) -> Fraction:
    """Exact value of a non-negative finite bf16 pattern via float32 (exact)."""
    f = np.array([bits << 16], dtype=np.uint32).view(np.float32)[0]
    return Fraction(float(f))


_TABLE_BITS = list(range(0, MAX_FINITE + 1))
_TABLE_VALS = [_bf16_value(b) for b in _TABLE_BITS]
# the value one ulp past the largest finite bf16 (used for overflow ties)
_OVER = Fraction(2) ** 128


def round_exact(x, mode: str) -> int:
    """bf16 bits of the exact value ``x`` (Fraction, int or float) in ``mode``."""
    if isinstance(x, float):
        if math.isnan(x):
            return 0x7FC0
        if math.isinf(x):
            return 0x7F80 if x > 0 else 0xFF80
        neg = math.copysign(1.0, x) < 0
        x = Fraction(x)
    else:
        x = Fraction(x)
        neg = x < 0
    a = abs(x)
    sign = 0x8000 if neg else 0
    vals = _TABLE_VALS
    i = bisect.bisect_left(vals, a)
    if i < len(vals) and vals[i] == a:
        return sign | _TABLE_BITS[i]
    if i == len(vals):  # beyond the largest finite value
        lo_bits, lo = MAX_FINITE, vals[-1]
        hi_bits, hi = 0x7F80, _OVER
    else:
        lo_bits, lo = _TABLE_BITS[i - 1], vals[i - 1]
        hi_bits, hi = _TABLE_BITS[i], vals[i]
    if mode == "rtz":
        return sign | lo_bits
    mid = (lo + hi) / 2
    if a < mid:
        pick = lo_bits
    elif a > mid:
        pick = hi_bits
    elif mode == "rtna":
        pick = hi_bits
    else:  # rtne: the neighbour whose last significand bit is 0 (2^128 counts as even)
        pick = lo_bits if (lo_bits & 1) == 0 else hi_bits
    return sign | pick


def tie_distance(x: Fraction) -> Fraction:
    """Relative distance of |x| to the nearest rounding midpoint (for flagging near-ties)."""
    a = abs(Fraction(x))
    if a == 0:
        return Fraction(1)
    vals = _TABLE_VALS
    i = bisect.bisect_left(vals, a)
    cands = []
    for j in (i - 1, i):
        if 0 <= j < len(vals) - 1:
            cands.append((vals[j] + vals[j + 1]) / 2)
    if i >= len(vals) - 1:
        cands.append((vals[-1] + _OVER) / 2)
    return min(abs(a - m) for m in cands) / a


def ord_bf16(bits: np.ndarray) -> np.ndarray:
    """Monotone integer image of bf16 patterns (both zeros map to 0)."""
    b = np.asarray(bits).astype(np.int32)
    return np.where(b & 0x8000, -(b & 0x7FFF), b)
