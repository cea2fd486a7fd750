"""The parity checker itself: a planted one-bit difference is reported as
exactly one mismatch, and the transcendental bar accepts one ulp but not
two (runs without a GPU)."""
import numpy as np
import pytest

import oracle
import workloads as W
from _compare import assert_bitexact, assert_ulp_bar


def _oracle_output():
    o = oracle.get()
    x = W.normal_bf16((1, 16, 2, 64), 4242)
    cos, sin = o.rope_cossin(W.freqs_unpaired(16, 1, 64, 4243))
    return o.rope_rotate_half(x, cos, sin)


def test_one_flipped_bit_is_one_mismatch():
    want = _oracle_output()
    assert_bitexact(want.copy(), want, "unchanged")
    for bit in (0, 7, 14, 15):
        got = want.copy()
        got.flat[357] ^= np.uint16(1 << bit)         # element (0, 2, 1, 37)
        with pytest.raises(AssertionError, match=r": 1 mismatches, first at \[\[0, 2, 1, 37\]\]"):
            assert_bitexact(got, want, f"bit {bit}")


def test_ulp_bar_accepts_one_ulp_and_rejects_two():
    want = np.full(100000, 0x3F80, np.uint16)        # 1.0
    got = want.copy()
    got[5] = 0x3F81                                  # one ulp up
    assert_ulp_bar(got, want, "one ulp")
    got[5] = 0x3F82                                  # two ulps
    with pytest.raises(AssertionError, match="max ulp 2"):
        assert_ulp_bar(got, want, "two ulps")
    zeros = np.zeros(10, np.uint16)
    signed = zeros.copy()
    signed[0] = 0x8000                                # -0 vs +0: 0 ulp, not identical
    with pytest.raises(AssertionError, match="not bit-identical"):
        assert_ulp_bar(signed, zeros, "signed zero in a small array")
    got = want.copy()
    got[:20] = 0x3F81                                 # 20 of 1e5 differ: over 0.01%
    with pytest.raises(AssertionError, match="not bit-identical"):
        assert_ulp_bar(got, want, "too many")
