"""The comparisons every parity test uses, shared by the GPU tests and the
CPU test that checks the checker.

Bars: bit-exact (every element's bits equal), or the transcendental bar (at
most 1 bf16 ulp apart, at least 99.99% bit-identical).  The ulp distance is
|ord(a) - ord(b)| with ord(bits) = bits for a positive sign and
-(bits & 0x7FFF) otherwise, so +0 and -0 are 0 ulp apart but still count as
not bit-identical.
"""
import numpy as np


def say(*a):
    print(*a, flush=True)


def ordered(bits):
    b = np.asarray(bits, np.int64)
    return np.where(b & 0x8000, -(b & 0x7FFF), b)


def assert_bitexact(got, want, what):
    got, want = np.asarray(got), np.asarray(want)
    assert got.shape == want.shape, f"{what}: shape {got.shape} vs {want.shape}"
    bad = np.count_nonzero(got != want)
    say(f"{what}: {got.size} elements, {bad} not bit-identical")
    if bad:
        idx = np.argwhere(got != want)[:5]
        raise AssertionError(f"{what}: {bad} mismatches, first at {idx.tolist()}: "
                             f"{[hex(int(got[tuple(i)])) for i in idx]} vs "
                             f"{[hex(int(want[tuple(i)])) for i in idx]}")


def assert_ulp_bar(got, want, what):
    got, want = np.asarray(got), np.asarray(want)
    assert got.shape == want.shape, f"{what}: shape {got.shape} vs {want.shape}"
    d = np.abs(ordered(got) - ordered(want))
    bad = np.count_nonzero(got != want)
    say(f"{what}: {got.size} elements, {bad} not bit-identical, max {int(d.max(initial=0))} ulp")
    assert d.max(initial=0) <= 1, f"{what}: max ulp {d.max()}"
    assert bad <= 1e-4 * got.size, f"{what}: {bad} of {got.size} not bit-identical"
