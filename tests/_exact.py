"""Exact bf16 helpers for the tests, independent of the oracle's code.

`is_nearest_bf16(v, bits)` decides whether a bf16 bit pattern is the
round-to-nearest-even image of a high-precision real `v` by comparing
distances to the two neighbouring bf16 values (no scaling, no rounding
arithmetic of its own).
"""
import mpmath
import numpy as np


def bits_to_float(bits):
    """Exact value of finite bf16 bits as a Python float."""
    return float((np.array([int(bits) << 16], dtype=np.uint32)).view(np.float32)[0])


def _value_order_neighbours(bits):
    """bf16 bit patterns just below and just above `bits` in value order
    (None past the largest finite magnitude)."""
    bits = int(bits)
    mag = bits & 0x7FFF
    neg = bool(bits & 0x8000)
    if mag == 0:
        return 0x8001, 0x0001
    bigger = mag + 1 if mag + 1 < 0x7F80 else None
    smaller = mag - 1
    smaller_bits = (0x8000 if neg else 0) | smaller if smaller > 0 else (0x8000 if neg else 0)
    bigger_bits = None if bigger is None else ((0x8000 if neg else 0) | bigger)
    if neg:
        return bigger_bits, smaller_bits
    return smaller_bits, bigger_bits


def is_nearest_bf16(v, bits):
    """True iff finite bf16 `bits` is RNE(v) for the mpmath real `v`.

    Ties (equal distances) must land on the even significand.
    """
    bits = int(bits)
    if (bits & 0x7F80) == 0x7F80:
        return False
    here = mpmath.mpf(bits_to_float(bits))
    d_here = abs(v - here)
    for nb in _value_order_neighbours(bits):
        if nb is None:
            continue
        d_nb = abs(v - mpmath.mpf(bits_to_float(nb)))
        if d_nb < d_here:
            return False
        if d_nb == d_here and (bits & 1):
            return False
    if v != 0 and here == 0:
        # a zero result must carry the sign of the value it rounds
        return bool(bits & 0x8000) == (v < 0)
    return True
