"""Exact-arithmetic helpers for pinning the oracle (tests only).

An fp16 round-to-nearest-even written from the IEEE binary16 definition with
Python Fractions, independent of numpy's conversion routines.
"""
from bisect import bisect_left
from fractions import Fraction

import numpy as np


def _half_value(bits: int) -> Fraction:
    e, m = bits >> 10, bits & 0x3FF
    if e == 0:
        return Fraction(m, 1 << 24)
    return Fraction(1024 + m) * Fraction(2) ** (e - 25)


# Non-negative finite binary16 values, ascending (bit patterns 0 .. 0x7BFF).
_POS = [_half_value(b) for b in range(0x7C00)]


def half_to_fraction(h) -> Fraction:
    bits = int(np.asarray(h, dtype=np.float16).view(np.uint16))
    v = _half_value(bits & 0x7FFF)
    return -v if bits & 0x8000 else v


def round_to_half_bits(x: Fraction) -> int:
    """binary16 bit pattern of x rounded to nearest, ties to even (finite range only)."""
    neg = x < 0
    a = -x if neg else x
    i = bisect_left(_POS, a)
    if i < len(_POS) and _POS[i] == a:
        b = i
    else:
        lo, hi = i - 1, i
        if hi >= len(_POS):
            raise OverflowError("beyond the finite binary16 range")
        dlo, dhi = a - _POS[lo], _POS[hi] - a
        if dlo < dhi:
            b = lo
        elif dhi < dlo:
            b = hi
        else:
            b = lo if lo % 2 == 0 else hi
    return b | (0x8000 if neg else 0)  # IEEE: a negative value that rounds to 0 gives -0


def round_to_half(x: Fraction) -> np.float16:
    return np.array([round_to_half_bits(x)], dtype=np.uint16).view(np.float16)[0]
