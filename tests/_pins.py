"""Parity pins of the CPU oracle.

Each `check_*` function takes an `oracle.Oracle` and raises AssertionError if
the oracle disagrees with something other than itself: a library routine that
computes a step by another route (torch's bf16 cast and bf16 arithmetic,
numpy's permute), mpmath at 256-bit precision, hand-derived worked vectors,
textbook normal-CDF values, or an invariant of exact arithmetic.  The same
functions run against deliberately broken copies of the oracle in
test_oracle_mutants.py, where at least one of them must fail.

Method passages: [ERNIE-fuse] = "[sglang] ERNIE-Image의 RoPE와 GELU-mul 융합 및
RoPE cos/sin 호이스팅을 통한 성능 최적화" (blog.secrett2633.cloud, sglang PR
34306 analysis); §1 cos/sin hoist, §2 rotate-half, §3 GEGLU.
"""
import os

import mpmath
import numpy as np
import torch

import workloads
from _exact import bits_to_float, is_nearest_bf16

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
mpmath.mp.prec = 256


def _read_hex_table(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            body = line.split("#", 1)[0].split()
            if body:
                rows.append([int(t, 16) for t in body])
    return rows


def _torch_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16)).view(
        torch.bfloat16)


def _bits(t):
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def _same_bits_or_both_nan(a, b):
    a = np.asarray(a, np.uint16)
    b = np.asarray(b, np.uint16)
    nan_a = (a & 0x7F80) == 0x7F80
    nan_a &= (a & 0x007F) != 0
    nan_b = (b & 0x7F80) == 0x7F80
    nan_b &= (b & 0x007F) != 0
    return (a == b) | (nan_a & nan_b)


# ---------------------------------------------------------------------------
# rounding helper
# ---------------------------------------------------------------------------

def check_rounding_vs_torch(o):
    """double -> bf16 RNE agrees with torch's float32 -> bf16 cast on float inputs,
    including exact midpoints, subnormals and the overflow boundary; the sticky
    argument agrees with the cast of the neighbouring float."""
    rng = np.random.Generator(np.random.PCG64(11))
    bits32 = rng.integers(0, 2**32, size=6000, dtype=np.uint64).astype(np.uint32)
    mids = (rng.integers(0, 65536, size=3000, dtype=np.uint32) << 16) | 0x8000
    edge = np.array([0x00000000, 0x80000000, 0x00008000, 0x00018000, 0x00000001, 0x7F7F7FFF,
                     0x7F7F8000, 0x7F7F8001, 0xFF7F8000, 0x007F8000, 0x00800000, 0x3F808000,
                     0x3F818000, 0x3F7FFFFF, 0x00FF8000], dtype=np.uint32)
    allb = np.concatenate([bits32, mids, edge])
    f = allb.view(np.float32)
    keep = np.isfinite(f)
    f = f[keep]
    want = workloads.f32_to_bf16_bits(f)
    got = np.array([o.double_to_bf16(float(v), 0) for v in f], dtype=np.uint16)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, f"rounding differs from torch at {f[bad[:5]]}: {got[bad[:5]]} vs {want[bad[:5]]}"

    # sticky: a midpoint nudged by an infinitesimal rounds like the next float
    m = mids.view(np.float32)
    m = m[np.isfinite(m) & (m != 0)][:800]
    up = np.nextafter(m, np.float32(np.inf))
    dn = np.nextafter(m, np.float32(-np.inf))
    want_up = workloads.f32_to_bf16_bits(up)
    want_dn = workloads.f32_to_bf16_bits(dn)
    got_up = np.array([o.double_to_bf16(float(v), +1) for v in m], dtype=np.uint16)
    got_dn = np.array([o.double_to_bf16(float(v), -1) for v in m], dtype=np.uint16)
    assert np.array_equal(got_up, want_up), "sticky=+1 at a midpoint must round toward +inf"
    assert np.array_equal(got_dn, want_dn), "sticky=-1 at a midpoint must round toward -inf"

    # every finite bf16 value maps to itself
    allbf = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    finite = (allbf & 0x7F80) != 0x7F80
    vals = workloads.bf16_bits_to_f32(allbf[finite])
    back = np.array([o.double_to_bf16(float(v), 0) for v in vals], dtype=np.uint16)
    assert np.array_equal(back, allbf[finite])


# ---------------------------------------------------------------------------
# Rotate-half
# ---------------------------------------------------------------------------

def check_rope_worked_vectors(o):
    """Hand-derived vectors (tests/golden/rope_worked_vectors.txt)."""
    for v in _read_hex_table("rope_worked_vectors.txt"):
        x = np.array([[[[v[0], v[1]]]]], np.uint16)
        c = np.array([[v[2], v[4]]], np.uint16)
        s = np.array([[v[3], v[5]]], np.uint16)
        out = o.rope_rotate_half(x, c, s).ravel()
        assert out[0] == v[6] and out[1] == v[7], (
            f"worked vector {[hex(t) for t in v]}: got {hex(out[0])} {hex(out[1])}")


def eager_rope_chain(x_bits, cos_bits, sin_bits):
    """The eager bf16 operator chain the page describes [ERNIE-fuse §2], run
    by PyTorch on the CPU: split the leading R columns into halves, build the
    rotate-half partner (negated second half, then first half), two bf16
    products and one bf16 sum, then append the untouched columns."""
    B, S, H, D = x_bits.shape
    R = cos_bits.shape[1]
    x = _torch_bf16(x_bits)
    c = _torch_bf16(cos_bits).view(B, S, 1, R)
    s = _torch_bf16(sin_bits).view(B, S, 1, R)
    head, rest = x[..., :R], x[..., R:]
    lo, hi = head.chunk(2, dim=-1)
    partner = torch.cat((-hi, lo), dim=-1)
    turned = head * c + partner * s
    return _bits(torch.cat((turned, rest), dim=-1))


def check_rope_vs_eager_chain(o):
    """Bit-exact against the eager bf16 chain, on normal and edge-case data,
    with halves of the cos/sin rows that differ and with rotary tails."""
    cases = [  # B, S, H, D, R, data kind, table kind
        (1, 7, 3, 16, 16, "normal", "unpaired"),
        (2, 5, 2, 24, 16, "special", "unpaired"),
        (3, 4, 2, 32, 8, "special", "special"),
        (1, 9, 1, 12, 4, "special", "special"),
        (2, 3, 4, 10, 10, "normal", "special"),
        (1, 6, 2, 8, 2, "special", "special"),
    ]
    for i, (B, S, H, D, R, kind, tkind) in enumerate(cases):
        seed = 500 + 10 * i
        if kind == "normal":
            x = workloads.normal_bf16((B, S, H, D), seed)
        else:
            x = workloads.special_bf16((B, S, H, D), seed)
        if tkind == "unpaired":
            cos, sin = o.rope_cossin(workloads.freqs_unpaired(S, B, R, seed + 1))
        else:
            cos = workloads.special_bf16((B * S, R), seed + 2)
            sin = workloads.special_bf16((B * S, R), seed + 3)
        want = eager_rope_chain(x, cos, sin)
        got = o.rope_rotate_half(x, cos, sin)
        ok = _same_bits_or_both_nan(got, want)
        assert ok.all(), f"case {i}: {np.count_nonzero(~ok)} mismatches vs eager chain"


def check_rope_zero_angle(o):
    """freqs = 0 gives cos 1, sin 0, and the rotation returns x bit for bit,
    except that a -0 may come back as +0."""
    B, S, H, D, R = 2, 8, 3, 32, 24
    x = workloads.special_bf16((B, S, H, D), 77)
    cos, sin = o.rope_cossin(np.zeros((S, B, 1, R), np.float32))
    assert (cos == 0x3F80).all() and (sin == 0x0000).all()
    out = o.rope_rotate_half(x, cos, sin)
    neg_zero = x == 0x8000
    assert np.array_equal(out[~neg_zero], x[~neg_zero])
    assert np.isin(out[neg_zero], [0x0000, 0x8000]).all()


def check_rope_exact_invariants(o):
    """Exact-arithmetic policy with paired angles, freqs = cat(f, f):
    a unit vector in column j < R/2 goes to (cos, sin) in columns (j, j + R/2)
    (the textbook plane rotation by +theta); each pair keeps its norm; rotating
    twice by theta is rotating once by 2*theta."""
    rng = np.random.Generator(np.random.PCG64(21))
    B, S, H, D, R = 2, 5, 3, 20, 16
    h = R // 2
    theta = rng.uniform(-4, 4, size=(B * S, h))
    c = np.cos(np.concatenate([theta, theta], 1))
    s = np.sin(np.concatenate([theta, theta], 1))
    c2 = np.cos(np.concatenate([2 * theta, 2 * theta], 1))
    s2 = np.sin(np.concatenate([2 * theta, 2 * theta], 1))

    for j in (0, h - 1):
        e = np.zeros((B, S, H, D))
        e[..., j] = 1.0
        out = o.rope_rotate_half_exact(e, c, s).reshape(B * S, H, D)
        np.testing.assert_allclose(out[:, :, j], np.repeat(c[:, j:j + 1], H, 1), rtol=0, atol=1e-15)
        np.testing.assert_allclose(out[:, :, j + h], np.repeat(s[:, j:j + 1], H, 1), rtol=0,
                                   atol=1e-15)

    x = rng.standard_normal((B, S, H, D))
    y = o.rope_rotate_half_exact(x, c, s)
    n_in = x[..., :h] ** 2 + x[..., h:R] ** 2
    n_out = y[..., :h] ** 2 + y[..., h:R] ** 2
    np.testing.assert_allclose(n_out, n_in, rtol=1e-12)
    np.testing.assert_array_equal(y[..., R:], x[..., R:])
    twice = o.rope_rotate_half_exact(y, c, s)
    once = o.rope_rotate_half_exact(x, c2, s2)
    np.testing.assert_allclose(twice, once, rtol=1e-12, atol=1e-12)


def check_rope_rows_form(o):
    """The rows entry point equals the tensor entry point row by row."""
    B, S, H, D, R = 2, 6, 3, 24, 16
    x = workloads.normal_bf16((B, S, H, D), 31)
    cos, sin = o.rope_cossin(workloads.freqs_unpaired(S, B, R, 32))
    full = o.rope_rotate_half(x, cos, sin)
    tok = np.repeat(np.arange(B * S), H)
    rows = o.rope_rows(x.reshape(-1, D), cos[tok], sin[tok])
    assert np.array_equal(rows, full.reshape(-1, D))


# ---------------------------------------------------------------------------
# Cos/sin tables
# ---------------------------------------------------------------------------

def _check_table_vs_mpmath(freq_values, cos_bits, sin_bits):
    for f, cb, sb in zip(freq_values, cos_bits, sin_bits):
        x = mpmath.mpf(float(f))
        assert is_nearest_bf16(mpmath.cos(x), cb), f"cos({float(f)!r}) -> {hex(cb)}"
        assert is_nearest_bf16(mpmath.sin(x), sb), f"sin({float(f)!r}) -> {hex(sb)}"


def check_cossin_vs_mpmath(o):
    """Every distinct angle of the tiny, rope_qk and partial workloads, plus
    special angles, rounds to the nearest bf16 of mpmath's cos/sin."""
    angles = [np.array([0.0, 1e-30, -1e-30, 0.5, 1.0, np.pi, 100.0, 255.0, -3.0, 1e4, 6.0e5],
                       np.float32)]
    for wid in (0, 1, 2):
        angles.append(np.unique(workloads.workload_freqs(wid)))
    rng = np.random.Generator(np.random.PCG64(5))
    angles.append(rng.uniform(-1e3, 1e3, 400).astype(np.float32))
    flat = np.unique(np.concatenate(angles))
    cos, sin = o.rope_cossin(flat.reshape(1, 1, 1, -1))
    _check_table_vs_mpmath(flat, cos.ravel(), sin.ravel())
    # signed zero
    c0, s0 = o.rope_cossin(np.array([-0.0, 0.0], np.float32).reshape(1, 1, 1, 2))
    assert c0.ravel().tolist() == [0x3F80, 0x3F80] and s0.ravel().tolist() == [0x8000, 0x0000]


def check_cossin_row_order(o):
    """Row b*S + s: the page permutes (S, B, 1, R) to (B, S, 1, R) and
    flattens [ERNIE-fuse §1]; numpy's transpose/reshape does the same move,
    on distinct per-batch angles and on a non-contiguous (strided) freqs."""
    S, B, R = 6, 3, 8
    fr = workloads.freqs_3axis((1, 2, 3), (2, 4, 2), B, batch_offsets=[0, 5, 11])
    cos, sin = o.rope_cossin(fr)
    cos_each, sin_each = o.rope_cossin(fr.reshape(1, 1, 1, -1))
    want_c = cos_each.reshape(S, B, 1, R).transpose(1, 0, 2, 3).reshape(B * S, R)
    want_s = sin_each.reshape(S, B, 1, R).transpose(1, 0, 2, 3).reshape(B * S, R)
    assert np.array_equal(cos, want_c) and np.array_equal(sin, want_s)
    wide = np.zeros((S, B, 1, R + 5), np.float32)
    wide[..., :R] = fr
    cos2, sin2 = o.rope_cossin(wide[..., :R])
    assert np.array_equal(cos2, want_c) and np.array_equal(sin2, want_s)


# ---------------------------------------------------------------------------
# Rotary angles of a 3-axis token grid
# ---------------------------------------------------------------------------

GRID_CASES = [  # B, grid, dims, theta, t_offset
    (1, (1, 64, 64), (32, 48, 48), 1e4, None),
    (2, (2, 8, 16), (24, 36, 36), 1e4, [0, 7]),
    (3, (3, 5, 7), (2, 4, 10), 256.0, [4, 0, 2]),
]


def check_angles_grid_vs_numpy_recipe(o):
    """The angles equal, bit for bit, the numpy form of the same reading
    (workloads.freqs_3axis: meshgrid positions, axis-wise outer products in
    float64, concatenation, cat(f, f), one cast to float32)."""
    for B, grid, dims, theta, off in GRID_CASES:
        got = o.rope_angles_grid(B, grid, dims, theta, off)
        want = workloads.freqs_3axis(grid, dims, B, theta=theta, batch_offsets=off)
        assert got.shape == want.shape
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), (grid, dims)


def check_angles_grid_closed_forms(o):
    """Closed forms of the reading: the first half-angle of each axis has
    frequency theta^0 = 1, so it equals that axis's position exactly; the
    second half of every row repeats the first; every angle is the exact
    product pos * theta^(-2i/d) (mpmath, 60 digits) rounded to float32,
    within one float32 step."""
    B, grid, dims, theta, off = 2, (3, 4, 5), (4, 6, 8), 1e4, [0, 9]
    a = o.rope_angles_grid(B, grid, dims, theta, off)[:, :, 0, :]
    S, R, half = 60, 18, 9
    s = np.arange(S)
    t, h, w = s // 20, (s // 5) % 4, s % 5
    for b in range(B):
        assert np.array_equal(a[:, b, 0], (t + off[b]).astype(np.float32))
        assert np.array_equal(a[:, b, 2], h.astype(np.float32))
        assert np.array_equal(a[:, b, 5], w.astype(np.float32))
    assert np.array_equal(a[..., :half], a[..., half:])
    mpmath.mp.dps = 60
    cols = [(0, i, 4) for i in range(2)] + [(1, i, 6) for i in range(3)] + \
           [(2, i, 8) for i in range(4)]
    for (k, i, d), j in zip(cols, range(half)):
        for si in (1, 23, 59):
            for b in range(B):
                pos = [t[si] + off[b], h[si], w[si]][k]
                exact = mpmath.mpf(int(pos)) * mpmath.power(mpmath.mpf(theta), mpmath.mpf(-2 * i) / d)
                got = float(a[si, b, j])
                ulp = float(np.spacing(np.float32(abs(got)))) if got else 2.0 ** -149
                assert abs(mpmath.mpf(got) - exact) <= ulp, (k, i, pos)


# ---------------------------------------------------------------------------
# GELU and the multiply
# ---------------------------------------------------------------------------

def check_gelu_closed_forms(o):
    """Textbook Phi values (tests/golden/gelu_closed_forms.txt)."""
    for x_bits, g_bits in _read_hex_table("gelu_closed_forms.txt"):
        got = o.gelu_bf16(x_bits)
        assert got == g_bits, f"GELU({bits_to_float(x_bits)}) = {hex(got)}, want {hex(g_bits)}"


def mp_gelu(x):
    x = mpmath.mpf(x)
    return x * mpmath.erfc(-x / mpmath.sqrt(2)) / 2


def check_gelu_exhaustive_mpmath(o, table=None):
    """All 65536 bf16 inputs: finite ones round to the nearest bf16 of
    mpmath's x*Phi(x) at 256 bits; NaN -> NaN, +inf -> +inf, -inf -> NaN."""
    if table is None:
        table = o.gelu_table()
    for g in range(65536):
        r = int(table[g])
        if (g & 0x7F80) == 0x7F80:
            if g & 0x7F:
                assert (r & 0x7F80) == 0x7F80 and (r & 0x7F), f"NaN input {hex(g)} -> {hex(r)}"
            elif g == 0x7F80:
                assert r == 0x7F80
            else:
                assert (r & 0x7F80) == 0x7F80 and (r & 0x7F), "GELU(-inf) must be NaN"
            continue
        x = bits_to_float(g)
        if x == 0.0:
            assert r == g, "GELU(+-0) = +-0"
            continue
        assert is_nearest_bf16(mp_gelu(x), r), f"GELU({x!r}) -> {hex(r)}"


def check_gelu_exact_odd_part(o):
    """Exact policy: GELU(x) - GELU(-x) = x (Phi(x) + Phi(-x) = 1), and
    GELU(x) = x * Phi(x) at textbook points."""
    rng = np.random.Generator(np.random.PCG64(41))
    for x in rng.uniform(-9, 9, 300):
        d = o.gelu_exact(x) - o.gelu_exact(-x)
        assert abs(d - x) <= 1e-14 * max(1.0, abs(x)), x
    for x, phi in ((1.0, 0.8413447460685429), (-1.0, 0.15865525393145707),
                   (2.0, 0.9772498680518208), (0.5, 0.6914624612740131)):
        assert abs(o.gelu_exact(x) - x * phi) <= 1e-15


def check_gelu_and_mul_vs_eager(o):
    """Against PyTorch's CPU bf16 `up * F.gelu(gate)` [ERNIE-fuse §3], bit for
    bit, on gates in [-3, 2^60] with |gate| >= 2^-60.  This fixes which half
    is the gate.  Outside that range float32 GELU itself drifts from the exact
    value (the 1 + erf form cancels for gate < -3, subnormals flush, 2x
    overflows near 2^127), so it is no pin there."""
    rows, hidden = 64, 96
    gate = workloads.normal_bf16((rows, hidden), 61, sigma=2.0)
    gv = workloads.bf16_bits_to_f32(gate)
    gate[gv < -3.0] = 0xC040  # -3
    gate[np.abs(gv) < 2.0 ** -60] = 0x3F80
    up = workloads.normal_bf16((rows, hidden), 62)
    inp = np.concatenate([gate, up], axis=1)
    got = o.gelu_and_mul(inp)
    want = _bits(_torch_bf16(up) * torch.nn.functional.gelu(_torch_bf16(gate)))
    bad = np.count_nonzero(got != want)
    assert bad == 0, f"{bad} elements differ from eager"


def check_mul_rounding_vs_torch(o):
    """The second rounding: out = rne(up * G) equals PyTorch's bf16 multiply of
    up by the oracle's own bf16 GELU values (edge-case up values included)."""
    rows, hidden = 32, 64
    gate = workloads.special_bf16((rows, hidden), 71)
    up = workloads.special_bf16((rows, hidden), 72)
    inp = np.concatenate([gate, up], axis=1)
    got = o.gelu_and_mul(inp)
    g_tab = o.gelu_table()[gate]
    want = _bits(_torch_bf16(up) * _torch_bf16(g_tab))
    assert _same_bits_or_both_nan(got, want).all()


# ---------------------------------------------------------------------------
# The gate_up projection and GEGLU on it
# ---------------------------------------------------------------------------

def _finite_bits(a):
    a = np.asarray(a, np.uint16).copy()
    a[(a & 0x7F80) == 0x7F80] = 0x3F80            # no Inf/NaN operands
    return a


def check_gemm_vs_exact_rationals(o):
    """Every output is the round-to-nearest-even bf16 of the exact sum of
    products, computed with Python fractions (exact for binary floats) and
    judged by distances to the neighbouring bf16 values."""
    from fractions import Fraction
    mpmath.mp.prec = 4000
    for M, K, N, seed, gen in ((3, 1, 4, 11, "normal"), (4, 37, 5, 12, "normal"),
                               (3, 64, 3, 13, "special"), (2, 130, 4, 14, "special")):
        g = workloads.special_bf16 if gen == "special" else workloads.normal_bf16
        x = _finite_bits(g((M, K), 7000 + seed))
        w = _finite_bits(g((N, K), 7100 + seed))
        got = o.gemm_bf16(x, w)
        xv = [[Fraction(bits_to_float(b)) for b in row] for row in x]
        wv = [[Fraction(bits_to_float(b)) for b in row] for row in w]
        for m in range(M):
            for n in range(N):
                exact = sum((a * b for a, b in zip(xv[m], wv[n])), Fraction(0))
                v = mpmath.mpf(exact.numerator) / mpmath.mpf(exact.denominator)
                if abs(v) >= mpmath.mpf(bits_to_float(0x7F7F)) * (1 + mpmath.mpf(2) ** -8):
                    assert (int(got[m, n]) & 0x7FFF) == 0x7F80, "overflow must give inf"
                    continue
                assert is_nearest_bf16(v, int(got[m, n])), (M, K, N, m, n, hex(int(got[m, n])))
    mpmath.mp.prec = 53


def check_gemm_cancellation_ties_and_sticky(o):
    """Sums that a short accumulator gets wrong: cancellation of huge terms,
    an exact tie (to even), and a tie broken by a term 2^-60 below it."""
    def bf(vals):
        return workloads.f32_to_bf16_bits(np.array(vals, np.float32))
    cases = [
        ([2.0 ** 60, 1.0, -2.0 ** 60], 0x3F80),              # exactly 1
        ([2.0 ** 100, 2.0 ** -100, -2.0 ** 100], int(bf([2.0 ** -100])[0])),
        ([1.0, 2.0 ** -8], 0x3F80),                           # tie -> even (1.0)
        ([1.0 + 2.0 ** -7, 2.0 ** -8], 0x3F82),               # tie -> even (0x3F82)
        ([1.0, 2.0 ** -8, 2.0 ** -60], 0x3F81),               # just above the tie
        ([1.0, 2.0 ** -8, -2.0 ** -60], 0x3F80),              # just below it
    ]
    for vals, want in cases:
        x = bf(vals).reshape(1, -1)
        w = bf([1.0] * len(vals)).reshape(1, -1)
        got = int(o.gemm_bf16(x, w)[0, 0])
        assert got == want, (vals, hex(got), hex(want))


def check_gemm_geglu_vs_eager(o):
    """GEGLU on the projection against PyTorch's CPU eager chain: a float32
    matmul of small integers (exact), the bf16 cast of the projection, then
    up * gelu(gate) in bf16, bit for bit where float GELU is exact
    (gates in [-3, 2^60])."""
    rng = np.random.Generator(np.random.PCG64(8101))
    M, K, H = 6, 24, 10
    xf = rng.integers(-3, 4, size=(M, K)).astype(np.float32) * 0.25
    wf = rng.integers(-3, 4, size=(2 * H, K)).astype(np.float32) * 0.125
    x = workloads.f32_to_bf16_bits(xf)
    w = workloads.f32_to_bf16_bits(wf)
    got = o.gemm_geglu(x, w)
    gate_up = (torch.from_numpy(xf) @ torch.from_numpy(wf).T).to(torch.bfloat16)
    gate, up = gate_up[:, :H], gate_up[:, H:]
    want = _bits(up * torch.nn.functional.gelu(gate))
    g = gate.float().numpy()
    ok = (g >= -3.0)
    assert ok.mean() > 0.9
    assert np.array_equal(got[ok], want[ok]), (got[ok], want[ok])


def _ordered(bits):
    b = np.asarray(bits, np.int64)
    return np.where(b & 0x8000, -(b & 0x7FFF), b)


ALL_CHECKS = [
    check_rounding_vs_torch,
    check_rope_worked_vectors,
    check_rope_vs_eager_chain,
    check_rope_zero_angle,
    check_rope_exact_invariants,
    check_rope_rows_form,
    check_cossin_row_order,
    check_cossin_vs_mpmath,
    check_angles_grid_vs_numpy_recipe,
    check_angles_grid_closed_forms,
    check_gelu_closed_forms,
    check_gelu_exact_odd_part,
    check_gelu_and_mul_vs_eager,
    check_mul_rounding_vs_torch,
    check_gelu_exhaustive_mpmath,
    check_gemm_vs_exact_rationals,
    check_gemm_cancellation_ties_and_sticky,
    check_gemm_geglu_vs_eager,
]
