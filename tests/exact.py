"""Exact-arithmetic helpers for pinning the oracle (tests only).

Nothing here is shared with the oracle or the HIP library.  bf16 values come
from numpy's float32 interpretation of the bit pattern shifted into the high
half (a library routine); sums are exact Python Fractions; rounding picks the
nearest bf16 from the sorted table of all finite values, ties to the even
pattern (IEEE 754 roundTiesToEven).
"""
import bisect
from fractions import Fraction

import numpy as np


def widen(bits):
    """bf16 bit patterns -> float64 via numpy float32 (exact)."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):
        return u.view(np.float32).astype(np.float64)


_POS_BITS = np.arange(0, 0x7F80, dtype=np.uint32).astype(np.uint16)   # +0 .. max finite
_POS_VALS = None


def _table():
    global _POS_VALS
    if _POS_VALS is None:
        _POS_VALS = [Fraction(float(v)) for v in widen(_POS_BITS)]
    return _POS_VALS


def round_exact(x):
    """Nearest-even bf16 bit pattern of an exact rational (or int/float)."""
    x = Fraction(x)
    sign = 0x8000 if x < 0 else 0
    ax = -x if x < 0 else x
    vals = _table()
    top = vals[-1]
    inf_mid = (top + Fraction(2) ** 128) / 2
    if ax >= inf_mid:
        # at the midpoint the even neighbour is 2^128, i.e. infinity
        return sign | 0x7F80
    i = bisect.bisect_left(vals, ax)
    if i < len(vals) and vals[i] == ax:
        return sign | i
    lo, hi = i - 1, i          # vals[lo] < ax < vals[hi]
    if hi >= len(vals):
        return sign | lo
    dlo, dhi = ax - vals[lo], vals[hi] - ax
    if dlo < dhi:
        k = lo
    elif dhi < dlo:
        k = hi
    else:
        k = lo if lo % 2 == 0 else hi
    return sign | k


def exact_dot(a_bits, b_bits):
    av = widen(a_bits)
    bv = widen(b_bits)
    s = Fraction(0)
    sa = Fraction(0)
    for x, y in zip(av.tolist(), bv.tolist()):
        p = Fraction(x) * Fraction(y)
        s += p
        sa += abs(p)
    return s, sa
