"""Parity of the HIP path with the CPU oracle, through the C ABI (needs a GPU).

Bars, per step of the path:
  rotate-half RoPE and the tail passthrough: bit-exact, every element;
  cos/sin tables and GELU (transcendental stages): at most 1 bf16 ulp from
  the oracle with at least 99.99% of elements bit-identical (mismatch counts
  are printed; the kernels are designed to be correctly rounded, so the
  expected count is 0);
  GEGLU output: the oracle's bf16 product of up and the GPU's own GELU value
  must match bit for bit, and the end-to-end output meets the 1-ulp bar.

Inputs are the seeded workloads of workloads.py: the tiny workload whole, the
two mid-size RoPE workloads whole, the full-size GEGLU and fused-QKV
workloads on sampled rows (plus whole-tensor properties), and small
adversarial shapes spanning several workgroups with ragged ends.
"""
import os

import numpy as np
import pytest
import torch

import bf16_rope_geglu_amd as rgg
import oracle
import workloads as W
from _compare import assert_bitexact, assert_ulp_bar, ordered, say  # noqa: F401

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a HIP device")
    assert os.path.exists(rgg.LIBRARY), "librgg.so is not built"
    rgg.library()
    yield
    torch.cuda.synchronize()


@pytest.fixture(scope="module")
def orc():
    return oracle.get()


def dev(a):
    a = np.ascontiguousarray(a, dtype=np.uint16)
    return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()


def host(t):
    torch.cuda.synchronize()
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def with_guards(shape, fill=0x7FC1):
    """A bf16 tensor of `shape` inside a buffer whose 4 KiB guard bands hold
    a NaN pattern; returns (tensor, check) where check() verifies the bands."""
    n = int(np.prod(shape))
    g = 2048
    buf = torch.full((n + 2 * g,), fill, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    t = buf[g:g + n].view(shape)

    def check():
        b = host(buf)
        assert (b[:g] == fill).all() and (b[g + n:] == fill).all(), "write outside the output"
    return t, check


# ---------------------------------------------------------------------------
# Cos/sin tables
# ---------------------------------------------------------------------------

def gpu_cossin(freqs_np):
    f = torch.from_numpy(np.array(freqs_np, dtype=np.float32, order="C", copy=True)).cuda()
    c, s = rgg.rope_cossin_precompute(f)
    return host(c), host(s)


@pytest.mark.parametrize("wid", [0, 1, 2, 4])
def test_cossin_workload_tables(orc, wid):
    say(f"cos/sin table, workload {wid}")
    fr = W.workload_freqs(wid)
    gc, gs = gpu_cossin(fr)
    oc, os_ = orc.rope_cossin(fr)
    assert_ulp_bar(gc, oc, f"cos w{wid}")
    assert_ulp_bar(gs, os_, f"sin w{wid}")


def test_cossin_adversarial(orc):
    say("cos/sin adversarial angles, strided angles, per-batch angles")
    rng = np.random.Generator(np.random.PCG64(9))
    S, B, R = 37, 3, 24
    fr = np.empty((S, B, 1, R), np.float32)
    fr[:] = rng.uniform(-2e3, 2e3, fr.shape)
    fr.reshape(-1)[:40] = [0.0, -0.0, 1e-30, -1e-30, 1e-7, np.pi, -np.pi, np.pi / 2, 1e4, -1e4,
                           6e5, -6e5, 3e7, 1e-38, 2.0, 0.5, 100.0, 255.0, 63.0, 1.5707964,
                           3.1415927, 4.712389, 6.2831855, 0.7853982, 1e5, 123456.0, 7.0, 11.0,
                           0.1, 0.2, 0.3, 1.0, 2.5, 5.0, 10.0, 20.0, 50.0, 64.0, 128.0, 1000.0]
    gc, gs = gpu_cossin(fr)
    oc, os_ = orc.rope_cossin(fr)
    assert_ulp_bar(gc, oc, "cos adversarial")
    assert_ulp_bar(gs, os_, "sin adversarial")
    # strided (non-contiguous) angle view and distinct angles per batch row
    fr3 = W.freqs_3axis((2, 5, 7), (8, 12, 12), 3, batch_offsets=[0, 3, 9])
    wide = np.zeros(fr3.shape[:3] + (fr3.shape[3] + 8,), np.float32)
    wide[..., :fr3.shape[3]] = fr3
    wt = torch.from_numpy(wide).cuda()[..., :fr3.shape[3]]
    c, s = rgg.rope_cossin_precompute(wt)
    oc, os_ = orc.rope_cossin(fr3)
    assert_ulp_bar(host(c), oc, "cos strided")
    assert_ulp_bar(host(s), os_, "sin strided")


@pytest.mark.parametrize("S,B,R", [(97, 3, 32), (4099, 3, 256)], ids=["narrow", "wide"])
def test_cossin_mixed_paired_rows(orc, S, B, R):
    """Rows whose two halves repeat (cat(f, f)) next to rows whose halves
    differ, in the same waves: both branches of the paired table kernel, with
    4 columns per lane (small table) and with 8 (over 2^18 lanes of 4)."""
    say(f"cos/sin mixed paired / unpaired rows S={S} B={B} R={R}")
    fr = W.freqs_unpaired(S, B, R, 4040)
    rep = (np.arange(S) % 3) == 0
    fr[rep, :, :, R // 2:] = fr[rep, :, :, :R // 2]
    fr[5, 1, 0, R // 2] = -0.0
    fr[5, 1, 0, 0] = 0.0
    gc, gs = gpu_cossin(fr)
    oc, os_ = orc.rope_cossin(fr)
    assert_ulp_bar(gc, oc, "cos mixed rows")
    assert_ulp_bar(gs, os_, "sin mixed rows")


@pytest.mark.parametrize("S,B", [(8192, 2), (16385, 1)], ids=["at_threshold", "one_row_over"])
def test_cossin_lane_threshold(orc, S, B):
    """Tables of exactly 2^18 lanes of 4 columns (R = 128: 16384 rows) take
    the 4-column lanes, one row more the 8-column lanes; both match the
    oracle, with halves that repeat and halves that differ."""
    say(f"cos/sin at the lane threshold S={S} B={B}")
    R = 128
    fr = W.freqs_unpaired(S, B, R, 5150)
    rep = (np.arange(S) % 2) == 0
    fr[rep, :, :, R // 2:] = fr[rep, :, :, :R // 2]
    gc, gs = gpu_cossin(fr)
    oc, os_ = orc.rope_cossin(fr)
    assert_ulp_bar(gc, oc, "cos at threshold")
    assert_ulp_bar(gs, os_, "sin at threshold")


def test_cossin_empty_and_guards(orc):
    say("cos/sin empty shapes and guard bands")
    f = torch.zeros((0, 2, 1, 16), device="cuda")
    c, s = rgg.rope_cossin_precompute(f)
    assert c.shape == (0, 16)
    fr = W.freqs_1d(33, 2, 16)
    cg, ccheck = with_guards((66, 16))
    sg, scheck = with_guards((66, 16))
    rgg.rope_cossin_precompute(torch.from_numpy(fr).cuda(), cg, sg)
    ccheck()
    scheck()
    oc, os_ = orc.rope_cossin(fr)
    assert_ulp_bar(host(cg), oc, "cos guarded")
    assert_ulp_bar(host(sg), os_, "sin guarded")


# ---------------------------------------------------------------------------
# Cos/sin tables of a 3-axis token grid
# ---------------------------------------------------------------------------

GRID_TABLES = [  # B, grid, dims, theta, t_offset
    (1, (1, 64, 64), (32, 48, 48), 1e4, None),       # rope_qk
    (2, (1, 64, 64), (24, 36, 36), 1e4, None),       # partial
    (4, (2, 64, 64), (32, 48, 48), 1e4, None),       # dit_layer
    (3, (3, 7, 11), (16, 8, 8), 1e4, [0, 5, 1000]),  # ragged grid, per-batch shifts
    (2, (5, 1, 9), (0, 16, 16), 256.0, [7, -3]),     # an axis with no columns
    (1, (1, 2, 3), (2, 6, 8), 1e6, None),            # one 8-column group per row
    (2, (2, 3, 5), (256, 256, 128), 1e4, [3, 0]),    # R = 640: frequencies built on the device
    (2, (3, 67, 41), (32, 48, 48), 1e4, [0, 2]),     # ragged, just over 2^18 lanes of 4 columns
    (1, (4, 64, 64), (32, 48, 48), 1e4, None),       # exactly 2^18 lanes of 4 columns
    (5, (1, 29, 113), (32, 48, 48), 1e4, [0, 1, 2, 3, 4]),  # 16385 rows: one row over
]


@pytest.mark.parametrize("case", GRID_TABLES, ids=lambda c: "B{}g{}x{}x{}d{}-{}-{}".format(
    c[0], *c[1], *c[2]))
def test_cossin_from_grid(orc, case):
    B, grid, dims, theta, off = case
    say(f"grid tables {case}")
    T, Hg, Wg = grid
    S, R = T * Hg * Wg, sum(dims)
    offd = None if off is None else torch.tensor(off, dtype=torch.int32, device="cuda")
    gc_t, gs_t = with_guards((B * S, R)), with_guards((B * S, R))
    rgg.rope_cossin_from_grid(B, grid, dims, theta, offd, cos_out=gc_t[0], sin_out=gs_t[0])
    gc_t[1]()
    gs_t[1]()
    gc, gs = host(gc_t[0]), host(gs_t[0])
    angles = orc.rope_angles_grid(B, grid, dims, theta, off)
    oc, os_ = orc.rope_cossin(angles)
    assert_ulp_bar(gc, oc, "grid cos")
    assert_ulp_bar(gs, os_, "grid sin")
    # Same fp32 angles => the same bits as the precompute fed the oracle's angles.
    pc, ps = gpu_cossin(angles)
    assert_bitexact(gc, pc, "grid cos vs precompute of the oracle's angles")
    assert_bitexact(gs, ps, "grid sin vs precompute of the oracle's angles")


def test_cossin_from_grid_empty():
    say("grid tables, empty shapes")
    c, s_ = rgg.rope_cossin_from_grid(0, (1, 4, 4), (4, 6, 6))
    assert c.shape == (0, 16) and s_.shape == (0, 16)
    c, s_ = rgg.rope_cossin_from_grid(2, (1, 0, 4), (4, 6, 6))
    assert c.shape == (0, 16)
    torch.cuda.synchronize()


# ---------------------------------------------------------------------------
# Rotate-half RoPE
# ---------------------------------------------------------------------------

def oracle_rope(orc, x, cos, sin):
    return orc.rope_rotate_half(x, cos, sin)


def test_rope_tiny_workload(orc):
    say("rope tiny workload")
    r = W.WORKLOADS[0]["rope"]
    fr = W.workload_freqs(0)
    cos_d, sin_d = rgg.rope_cossin_precompute(torch.from_numpy(fr).cuda())
    cos, sin = host(cos_d), host(sin_d)
    x = W.normal_bf16((r["B"], r["S"], r["H"], r["D"]), W.seed_for(0, "x"))
    out = rgg.rope_rotate_half_bf16(dev(x), cos_d, sin_d)
    assert_bitexact(host(out), oracle_rope(orc, x, cos, sin), "rope tiny")
    # end to end against the oracle's own tables
    oc, os_ = orc.rope_cossin(fr)
    assert_ulp_bar(host(out), oracle_rope(orc, x, oc, os_), "rope tiny end-to-end")


@pytest.mark.parametrize("wid", [1, 2])
def test_rope_workload_whole(orc, wid):
    r = W.WORKLOADS[wid]["rope"]
    B, S, H, D, R = r["B"], r["S"], r["H"], r["D"], r["R"]
    say(f"rope workload {wid}: ({B},{S},{H},{D}) R={R} views={r['views']}")
    fr = W.workload_freqs(wid)
    cos_d, sin_d = rgg.rope_cossin_precompute(torch.from_numpy(fr).cuda())
    cos, sin = host(cos_d), host(sin_d)
    names = ["q", "k"][:r["views"]]
    xs = [W.normal_bf16((B, S, H, D), W.seed_for(wid, n)) for n in names]
    outs = rgg.rope_rotate_half_bf16([dev(x) for x in xs], cos_d, sin_d)
    for n, x, o in zip(names, xs, outs):
        got = host(o)
        assert_bitexact(got, oracle_rope(orc, x, cos, sin), f"rope w{wid} {n}")
        if R < D:
            assert np.array_equal(got[..., R:], x[..., R:]), "tail must pass through"


ADVERSARIAL = [  # B, S, H, D, R, views, data, tables
    (3, 37, 5, 48, 32, 1, "special", "unpaired"),
    (2, 129, 3, 64, 64, 2, "normal", "unpaired"),
    (1, 300, 2, 32, 16, 3, "special", "special"),
    (2, 17, 7, 128, 96, 4, "special", "unpaired"),
    (1, 5, 1, 16, 0, 1, "normal", "none"),
    (1, 1, 1, 16, 16, 1, "special", "special"),
    (5, 3, 33, 24, 16, 2, "normal", "unpaired"),
    (1, 23, 24, 128, 96, 2, "special", "unpaired"),
]


@pytest.mark.parametrize("case", ADVERSARIAL, ids=lambda c: "B{}S{}H{}D{}R{}v{}".format(*c[:6]))
def test_rope_adversarial(orc, case):
    B, S, H, D, R, nv, kind, tkind = case
    say(f"rope adversarial {case}")
    seed = 7000 + B * 100 + S + H + D + R + nv
    if tkind == "unpaired":
        cos, sin = orc.rope_cossin(W.freqs_unpaired(S, B, R, seed))
    elif tkind == "special":
        cos = W.special_bf16((B * S, R), seed + 1)
        sin = W.special_bf16((B * S, R), seed + 2)
    else:
        cos = np.zeros((B * S, 0), np.uint16)
        sin = np.zeros((B * S, 0), np.uint16)
    gen = W.special_bf16 if kind == "special" else W.normal_bf16
    xs = [gen((B, S, H, D), seed + 10 + v) for v in range(nv)]
    guarded = [with_guards((B, S, H, D)) for _ in range(nv)]
    xd = [dev(x) for x in xs]
    rgg.rope_rotate_half_bf16(xd, dev(cos) if R else torch.empty((B * S, 0), dtype=torch.bfloat16,
                                                                  device="cuda"),
                              dev(sin) if R else torch.empty((B * S, 0), dtype=torch.bfloat16,
                                                             device="cuda"),
                              out=[g[0] for g in guarded])
    for v in range(nv):
        guarded[v][1]()
        assert np.array_equal(host(xd[v]), xs[v]), "input modified"
        assert_bitexact(host(guarded[v][0]), oracle_rope(orc, xs[v], cos, sin), f"view {v}")


def _rope_fuzz_case(k):
    """A seeded random RoPE configuration; k % 4 steers it towards one launch
    path: 0 one vector per lane (wide rows, R/2 splitting lines, aligned),
    1 two-vector items on whole lines, 2 several tokens per workgroup,
    3 arbitrary 8-element strides."""
    rng = np.random.Generator(np.random.PCG64(7700 + k))
    kind = k % 4
    if kind == 0:
        D = int(rng.choice([128, 256, 512]))
        H = int(rng.integers(2112 // D + 1, 4096 // D + 1))
        R = int(rng.choice([r for r in range(16, D + 1, 16) if r % 64]))
        align = 64
    elif kind == 1:
        D = int(rng.choice([64, 128, 256]))
        H = int(rng.integers(2048 // D + 1, 40))
        R = int(rng.choice([r for r in range(64, D + 1, 64)]))
        align = 64
    elif kind == 2:
        D = int(rng.choice([16, 32, 48, 64, 128]))
        H = int(rng.integers(1, 9))
        R = int(rng.choice(range(0, D + 1, 16)))
        align = 8
    else:
        D = int(rng.choice([8 * i for i in range(1, 33)]))
        H = int(rng.integers(1, 24))
        R = int(rng.choice(range(0, D + 1, 16)))
        align = 8
    B, S = int(rng.integers(1, 4)), int(rng.integers(1, 40))
    nv = int(rng.integers(1, 5))
    views = []
    for v in range(nv):
        def strides():
            sh = D + align * int(rng.integers(0, 3))
            ss = H * sh + align * int(rng.integers(0, 3))
            sb = S * ss + align * int(rng.integers(0, 3))
            return sb, ss, sh, align * int(rng.integers(0, 4))
        xs = strides()
        in_place = kind != 0 and rng.random() < 0.25
        views.append((xs, None if in_place else strides()))
    return B, S, H, D, R, views, int(rng.integers(0, 1 << 30))


def _strided(buf, off, st, shape):
    return torch.as_strided(buf, shape, (st[0], st[1], st[2], 1), off)


@pytest.mark.parametrize("k", range(48))
def test_rope_random_layouts(orc, k):
    """Seeded random shapes, strides, view counts and in-place views over
    every launch path, element by element against the oracle, with the
    padding between rows left untouched."""
    B, S, H, D, R, views, seed = _rope_fuzz_case(k)
    say(f"rope fuzz {k}: B{B} S{S} H{H} D{D} R{R} views {views}")
    cos, sin = orc.rope_cossin(W.freqs_unpaired(S, B, R, seed)) if R else (
        np.zeros((B * S, 0), np.uint16), np.zeros((B * S, 0), np.uint16))
    sentinel = 0x7FC1
    xs, outs, bufs = [], [], []
    for v, (xst, ost) in enumerate(views):
        n_x = (B - 1) * xst[0] + (S - 1) * xst[1] + (H - 1) * xst[2] + D + xst[3]
        host_x = W.special_bf16((n_x,), seed + 1 + v)
        xbuf = dev(host_x)
        xv = _strided(xbuf, xst[3], xst, (B, S, H, D))
        if ost is None:
            ov, obuf = xv, None
        else:
            n_o = (B - 1) * ost[0] + (S - 1) * ost[1] + (H - 1) * ost[2] + D + ost[3]
            obuf = torch.full((n_o,), sentinel, dtype=torch.int16, device="cuda").view(torch.bfloat16)
            ov = _strided(obuf, ost[3], ost, (B, S, H, D))
        xs.append(xv)
        outs.append(ov)
        bufs.append((host_x, xbuf, obuf))
    rgg.rope_rotate_half_bf16(xs, dev(cos) if R else torch.empty((B * S, 0), dtype=torch.bfloat16,
                                                                  device="cuda"),
                              dev(sin) if R else torch.empty((B * S, 0), dtype=torch.bfloat16,
                                                             device="cuda"), out=outs)
    for v, ((xst, ost), (host_x, xbuf, obuf)) in enumerate(zip(views, bufs)):
        x_in = np.lib.stride_tricks.as_strided(host_x[xst[3]:], (B, S, H, D),
                                               tuple(2 * t for t in (xst[0], xst[1], xst[2], 1)))
        want = orc.rope_rotate_half(np.ascontiguousarray(x_in), cos, sin)
        if ost is None:                     # in place: the tail is left as it was
            want[..., R:] = x_in[..., R:]
            after = host(xbuf)
            got = np.lib.stride_tricks.as_strided(after[xst[3]:], (B, S, H, D),
                                                  tuple(2 * t for t in (xst[0], xst[1], xst[2], 1)))
            touched = np.zeros(after.shape, bool)
            np.lib.stride_tricks.as_strided(touched[xst[3]:], (B, S, H, D), tuple(
                t for t in (xst[0], xst[1], xst[2], 1)))[...] = True
            assert np.array_equal(after[~touched], host_x[~touched]), "wrote outside the view"
        else:
            after = host(obuf)
            got = np.lib.stride_tricks.as_strided(after[ost[3]:], (B, S, H, D),
                                                  tuple(2 * t for t in (ost[0], ost[1], ost[2], 1)))
            touched = np.zeros(after.shape, bool)
            np.lib.stride_tricks.as_strided(touched[ost[3]:], (B, S, H, D), tuple(
                t for t in (ost[0], ost[1], ost[2], 1)))[...] = True
            assert (after[~touched] == sentinel).all(), "wrote outside the output view"
            assert np.array_equal(host(xbuf), host_x), "input modified"
        assert_bitexact(np.ascontiguousarray(got), want, f"fuzz {k} view {v}")


def make_qkv(B, S, H, D, seed):
    qkv = W.normal_bf16((B, S, 3 * H * D), seed)
    return qkv


def qkv_views(t, H, D):
    B, S, _ = t.shape
    q = t[..., :H * D].view(B, S, H, D)
    k = t[..., H * D:2 * H * D].view(B, S, H, D)
    return q, k


def test_rope_fused_qkv_views_small(orc):
    """q/k as strided views of a fused QKV buffer, out of place and in place."""
    B, S, H, D, R = 2, 45, 4, 64, 64
    say(f"rope fused qkv small ({B},{S},{H},{D})")
    qkv = make_qkv(B, S, H, D, 8101)
    cos, sin = orc.rope_cossin(W.freqs_unpaired(S, B, R, 8102))
    t = dev(qkv)
    q, k = qkv_views(t, H, D)
    assert q.stride() == (S * 3 * H * D, 3 * H * D, D, 1)
    oq, ok = rgg.rope_rotate_half_bf16([q, k], dev(cos), dev(sin))
    hq = qkv[..., :H * D].reshape(B, S, H, D)
    hk = qkv[..., H * D:2 * H * D].reshape(B, S, H, D)
    assert_bitexact(host(oq), oracle_rope(orc, hq, cos, sin), "q from qkv")
    assert_bitexact(host(ok), oracle_rope(orc, hk, cos, sin), "k from qkv")
    # in place inside the fused buffer; v must be untouched
    rgg.rope_rotate_half_bf16([q, k], dev(cos), dev(sin), out=[q, k])
    after = host(t)
    assert np.array_equal(after[..., :H * D].reshape(B, S, H, D), host(oq))
    assert np.array_equal(after[..., H * D:2 * H * D].reshape(B, S, H, D), host(ok))
    assert np.array_equal(after[..., 2 * H * D:], qkv[..., 2 * H * D:]), "v modified"


def test_rope_partial_in_place_keeps_tail(orc):
    B, S, H, D, R = 2, 19, 3, 128, 96
    say("rope partial in place")
    x = W.special_bf16((B, S, H, D), 8201)
    cos, sin = orc.rope_cossin(W.freqs_unpaired(S, B, R, 8202))
    t = dev(x)
    rgg.rope_rotate_half_bf16(t, dev(cos), dev(sin), out=t)
    assert_bitexact(host(t), oracle_rope(orc, x, cos, sin), "in place with tail")


def test_rope_zero_rotary_width_one_token(orc):
    """R = 0 with one token per workgroup: the row copy only, with no cos/sin
    row to fetch (regression: an early fetch of the row must not run)."""
    say("rope R = 0, one token per workgroup")
    B, S, H, D = 1, 3, 20, 240
    x = W.special_bf16((B, S, H, D), 8700)
    empty = torch.empty((B * S, 0), dtype=torch.bfloat16, device="cuda")
    out = rgg.rope_rotate_half_bf16(dev(x), empty, empty)
    assert_bitexact(host(out), x, "R = 0 copy")


def test_rope_empty_shapes():
    say("rope empty shapes")
    c = torch.zeros((0, 16), dtype=torch.bfloat16, device="cuda")
    x = torch.zeros((0, 4, 2, 16), dtype=torch.bfloat16, device="cuda")
    assert rgg.rope_rotate_half_bf16(x, c, c).shape == x.shape
    x = torch.zeros((2, 0, 2, 16), dtype=torch.bfloat16, device="cuda")
    assert rgg.rope_rotate_half_bf16(x, c, c).shape == x.shape
    x = torch.zeros((1, 3, 0, 16), dtype=torch.bfloat16, device="cuda")
    c3 = torch.zeros((3, 16), dtype=torch.bfloat16, device="cuda")
    assert rgg.rope_rotate_half_bf16(x, c3, c3).shape == x.shape


def test_rope_on_side_stream(orc):
    say("rope on a non-default stream")
    B, S, H, D, R = 1, 64, 4, 32, 32
    x = W.normal_bf16((B, S, H, D), 8301)
    cos, sin = orc.rope_cossin(W.freqs_unpaired(S, B, R, 8302))
    xd, cd, sd = dev(x), dev(cos), dev(sin)
    torch.cuda.synchronize()
    st = torch.cuda.Stream()
    with torch.cuda.stream(st):
        out = rgg.rope_rotate_half_bf16(xd, cd, sd)
    st.synchronize()
    assert_bitexact(host(out), oracle_rope(orc, x, cos, sin), "side stream")


def oracle_rope_threaded(orc, x, cos, sin):
    """The oracle's rotate-half over a (B, S, H, D) array, split by token
    ranges over the host's cores (ctypes releases the interpreter lock, so
    the C oracle runs on every core at once)."""
    from concurrent.futures import ThreadPoolExecutor

    B, S, H, D = x.shape
    T = B * S
    xt = x.reshape(1, T, H, D)
    out = np.empty_like(xt)
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    n = max(1, min(n, 64))
    cuts = [T * i // n for i in range(n + 1)]

    def part(i):
        a, b = cuts[i], cuts[i + 1]
        if b > a:
            out[:, a:b] = orc.rope_rotate_half(xt[:, a:b], cos[a:b], sin[a:b])

    with ThreadPoolExecutor(max_workers=n) as pool:
        list(pool.map(part, range(n)))
    return out.reshape(B, S, H, D)


def test_rope_dit_layer_full_size(orc):
    """Full-size fused-QKV workload in the launch configuration the benchmark
    times: q and k strided views of (4, 8192, 3*32*128), contiguous outputs,
    one launch.  The whole cos/sin table and every element of both outputs
    (2 x 4*8192*32*128) are compared with the oracle."""
    r = W.WORKLOADS[4]["rope"]
    B, S, H, D, R = r["B"], r["S"], r["H"], r["D"], r["R"]
    say(f"rope full size ({B},{S},{H},{D}) from fused qkv")
    qkv = W.device_normal_bf16((B, S, 3 * H * D), W.seed_for(4, "qkv"))
    q, k = qkv_views(qkv, H, D)
    fr = W.workload_freqs(4)
    cos_d, sin_d = rgg.rope_cossin_precompute(torch.from_numpy(fr).cuda())
    oq, ok = rgg.rope_rotate_half_bf16([q, k], cos_d, sin_d)
    cos, sin = host(cos_d), host(sin_d)
    oc, os_ = orc.rope_cossin(fr)
    assert_ulp_bar(cos, oc, "cos full size")
    assert_ulp_bar(sin, os_, "sin full size")
    for name, xin, xout in (("q", q, oq), ("k", k, ok)):
        want = oracle_rope_threaded(orc, host(xin), cos, sin)
        assert_bitexact(host(xout), want, f"{name} full size, every token")
        del want
    del qkv, oq, ok


# ---------------------------------------------------------------------------
# GEGLU
# ---------------------------------------------------------------------------

def test_gelu_all_65536_inputs(orc):
    """Every bf16 gate with up = 1 (rne(1 * G) = G): the GPU's GELU table
    against the oracle's, all 65536 inputs (NaN only as NaN)."""
    say("gelu exhaustive")
    gate = np.arange(65536, dtype=np.uint32).astype(np.uint16).reshape(512, 128)
    up = np.full_like(gate, 0x3F80)
    out = host(rgg.gelu_and_mul_bf16(dev(np.concatenate([gate, up], 1))))
    want = orc.gelu_table().reshape(512, 128)
    nan_w = ((want & 0x7F80) == 0x7F80) & ((want & 0x7F) != 0)
    nan_g = ((out & 0x7F80) == 0x7F80) & ((out & 0x7F) != 0)
    assert np.array_equal(nan_w, nan_g), "NaN positions differ"
    assert_ulp_bar(out[~nan_w], want[~nan_w], "gelu all inputs")
    # scaled up: out = rne(up * G) with the same G
    up2 = W.special_bf16(gate.shape, 99)
    out2 = host(rgg.gelu_and_mul_bf16(dev(np.concatenate([gate, up2], 1))))
    want2 = orc.gelu_and_mul(np.concatenate([gate, up2], 1))
    fin = ~(nan_w | (((out2 & 0x7F80) == 0x7F80) & ((out2 & 0x7F) != 0)))
    assert_ulp_bar(out2[fin], want2[fin], "gelu all inputs, special up")


def geglu_inputs(rows, hidden, wid, gate_sigma):
    gate = W.normal_bf16((rows, hidden), W.seed_for(wid, "gate"), gate_sigma)
    up = W.normal_bf16((rows, hidden), W.seed_for(wid, "up"))
    return np.concatenate([gate, up], axis=1)


def check_geglu_given_gelu(orc, inp, got, what):
    """out == rne(up * G(gate)) bit for bit, with G the oracle's GELU table
    (the exact GELU rounded once).  The exhaustive test ties the GPU's table
    to the oracle's on all 65536 gates, so any difference here is in the
    multiply or the data movement, which must be exact."""
    want = orc.gelu_and_mul(inp)
    nan = (((want & 0x7F80) == 0x7F80) & ((want & 0x7F) != 0) &
           ((got & 0x7F80) == 0x7F80) & ((got & 0x7F) != 0))
    assert_bitexact(np.where(nan, 0, got), np.where(nan, 0, want), what)


def test_geglu_tiny_workload(orc):
    g = W.WORKLOADS[0]["geglu"]
    say("geglu tiny workload")
    inp = geglu_inputs(g["rows"], g["hidden"], 0, g["gate_sigma"])
    out_t, check = with_guards((g["rows"], g["hidden"]))
    xd = dev(inp)
    rgg.gelu_and_mul_bf16(xd, out_t)
    check()
    assert np.array_equal(host(xd), inp), "input modified"
    check_geglu_given_gelu(orc, inp, host(out_t), "geglu tiny")


GEGLU_EDGE = [  # rows, hidden, in row stride, out row stride, data
    (1, 8, 16, 8, "special"),
    (3, 24, 64, 40, "special"),
    (257, 40, 80, 40, "normal"),
    (1031, 96, 200, 104, "special"),
    (4099, 8, 16, 8, "normal"),
]


@pytest.mark.parametrize("case", GEGLU_EDGE, ids=lambda c: "r{}h{}is{}os{}".format(*c[:4]))
def test_geglu_edge_shapes(orc, case):
    rows, hidden, is_, os_, kind = case
    say(f"geglu edge {case}")
    gen = W.special_bf16 if kind == "special" else W.normal_bf16
    full = gen((rows, is_), 9000 + rows + hidden)
    inp = full[:, :2 * hidden]
    buf = torch.full((rows, os_), 0x7FC1, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    out = buf[:, :hidden]
    xd = dev(full)[:, :2 * hidden]
    rgg.gelu_and_mul_bf16(xd, out)
    b = host(buf)
    assert (b[:, hidden:] == 0x7FC1).all(), "wrote into the row padding"
    got = b[:, :hidden]
    want = orc.gelu_and_mul(inp)
    nan = ((want & 0x7F80) == 0x7F80) & ((want & 0x7F) != 0)
    assert ((got[nan] & 0x7F80) == 0x7F80).all() and ((got[nan] & 0x7F) != 0).all()
    assert_ulp_bar(got[~nan], want[~nan], f"geglu {case}")


@pytest.mark.parametrize("k", range(24))
def test_geglu_random_layouts(orc, k):
    """Seeded random rows, widths, row strides and in-place calls against the
    oracle, with the row padding left untouched."""
    rng = np.random.Generator(np.random.PCG64(8800 + k))
    rows = int(rng.integers(1, 700))
    hidden = 8 * int(rng.integers(1, 129))
    is_ = 2 * hidden + 8 * int(rng.integers(0, 5))
    in_place = rng.random() < 0.3
    os_ = is_ if in_place else hidden + 8 * int(rng.integers(0, 5))
    say(f"geglu fuzz {k}: rows {rows} hidden {hidden} strides {is_}/{os_} in place {in_place}")
    gen = W.special_bf16 if k % 2 else (lambda shape, seed: W.normal_bf16(shape, seed, 3.0))
    full = gen((rows, is_), 8900 + k)
    buf = dev(full)
    inp = buf[:, :2 * hidden]
    if in_place:
        out_buf, out = buf, buf[:, :hidden]
    else:
        out_buf = torch.full((rows, os_), 0x7FC1, dtype=torch.int16,
                             device="cuda").view(torch.bfloat16)
        out = out_buf[:, :hidden]
    rgg.gelu_and_mul_bf16(inp, out)
    after = host(out_buf)
    want = orc.gelu_and_mul(np.ascontiguousarray(full[:, :2 * hidden]))
    got = after[:, :hidden]
    if in_place:
        assert np.array_equal(after[:, hidden:], full[:, hidden:]), "wrote past the gate half"
    else:
        assert (after[:, hidden:] == 0x7FC1).all(), "wrote into the row padding"
        assert np.array_equal(host(buf), full), "input modified"
    nan = ((want & 0x7F80) == 0x7F80) & ((want & 0x7F) != 0)
    assert ((got[nan] & 0x7F80) == 0x7F80).all() and ((got[nan] & 0x7F) != 0).all()
    assert_ulp_bar(got[~nan], want[~nan], f"geglu fuzz {k}")


def test_geglu_in_place_and_empty(orc):
    say("geglu in place / empty")
    inp = geglu_inputs(300, 64, 11, 3.0)
    t = dev(inp)
    rgg.gelu_and_mul_bf16(t, t[:, :64])
    after = host(t)
    assert np.array_equal(after[:, 64:], inp[:, 64:]), "up half modified"
    check_geglu_given_gelu(orc, inp, after[:, :64], "geglu in place")
    e = rgg.gelu_and_mul_bf16(torch.empty((0, 32), dtype=torch.bfloat16, device="cuda"))
    assert e.shape == (0, 16)


@pytest.mark.parametrize("wid", [3, 4])
def test_geglu_full_size(orc, wid):
    """Full-size GEGLU workloads: sampled rows against the oracle directly,
    and every element against rne(up * T[gate]), T the oracle's table of
    all 65536 GELU values, evaluated by torch on the device."""
    g = W.WORKLOADS[wid]["geglu"]
    rows, hidden = g["rows"], g["hidden"]
    say(f"geglu full size workload {wid}: {rows} x {hidden}")
    gate = W.device_normal_bf16((rows, hidden), W.seed_for(wid, "gate"), g["gate_sigma"])
    up = W.device_normal_bf16((rows, hidden), W.seed_for(wid, "up"))
    inp = torch.cat([gate, up], dim=1)
    del gate, up
    out = rgg.gelu_and_mul_bf16(inp)
    rng = np.random.Generator(np.random.PCG64(wid))
    rsel = np.unique(np.concatenate([[0, rows - 1], rng.integers(0, rows, 48)]))
    rs = torch.from_numpy(rsel).cuda()
    hin = host(inp[rs])
    assert_ulp_bar(host(out[rs]), orc.gelu_and_mul(hin), f"geglu w{wid} sampled rows")
    table = torch.from_numpy(orc.gelu_table().view(np.int16)).cuda()
    gi = inp[:, :hidden].view(torch.int16).to(torch.int32) & 0xFFFF
    G = table[gi].view(torch.bfloat16)
    want = (inp[:, hidden:].float() * G.float()).to(torch.bfloat16)
    del G, gi
    diff = (out.view(torch.int16) != want.view(torch.int16))
    nan = torch.isnan(want) & torch.isnan(out)
    bad = int((diff & ~nan).sum())
    say(f"geglu w{wid} whole tensor vs up*T[gate]: {bad} of {out.numel()} differ")
    assert bad == 0


# ---------------------------------------------------------------------------
# The gate_up projection, alone and with GEGLU in its epilogue
#
# Bars: on exact-sum inputs (small integers times 2^-4: every partial sum is
# exact in fp32, whatever the order) the projection and the fused GEGLU are
# bit-exact with the oracle.  On Gaussian inputs every projection output must
# be a bf16 rounding of a value within the fp32 accumulation bound
# 2 (K + 16) 2^-24 sum_k |x_k w_k| + K 2^-149 of the exact sum, and at least 99% of
# outputs must equal the oracle's correctly rounded sum.  The fused form must
# equal GEGLU of the plain projection bit for bit (one accumulation order).
# ---------------------------------------------------------------------------

def bf16_rne_f64(v):
    """Round float64 values to bf16 bits, ties to even (normal range)."""
    v = np.asarray(v, np.float64)
    m, e = np.frexp(v)
    r = np.rint(m * 256.0) * np.ldexp(1.0, e - 8)     # 8 significant bits
    return (r.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


def check_projection_bound(x, w, got, orc_out, what):
    """got (M, N) bf16 bits of x (M, K) @ w (N, K)^T: each a rounding of a
    value within the fp32 accumulation bound of the exact sum; >= 99% equal to
    the oracle's correctly rounded sum."""
    xf = W.bf16_bits_to_f32(x).astype(np.float64)
    wf = W.bf16_bits_to_f32(w).astype(np.float64)
    exact = xf @ wf.T
    mag = np.abs(xf) @ np.abs(wf).T
    K = x.shape[1]
    E = 2.0 * (K + 16) * 2.0 ** -24 * mag + 2.0 ** -40 * mag + K * 2.0 ** -149
    lo, hi = ordered(bf16_rne_any(exact - E)), ordered(bf16_rne_any(exact + E))
    g = ordered(got)
    outside = np.count_nonzero((g < lo) | (g > hi))
    same = np.count_nonzero(got == orc_out)
    d = np.abs(g - ordered(orc_out))
    say(f"{what}: {got.size} outputs, {got.size - same} differ from the oracle "
        f"(max {int(d.max(initial=0))} ulp), {outside} outside the accumulation bound")
    assert outside == 0, f"{what}: {outside} outputs outside the fp32 accumulation bound"
    assert same >= 0.99 * got.size, f"{what}: only {same} of {got.size} equal the oracle"


def padded(a, cols, fill=0x7FC1):
    """a (rows, c) bf16 bits inside a (rows, cols) device buffer; returns
    (buffer, view of a)."""
    rows, c = a.shape
    full = np.full((rows, cols), fill, np.uint16)
    full[:, :c] = a
    buf = dev(full)
    return buf, buf[:, :c]


GEMM_EXACT = [  # M, K, hidden, x row pad, out row pad
    (1, 64, 64, 0, 0),
    (127, 64, 64, 8, 0),
    (128, 128, 128, 0, 16),
    (129, 192, 64, 24, 8),
    (300, 256, 192, 0, 0),
    (1000, 128, 320, 8, 24),
    (2053, 512, 128, 0, 0),
]


@pytest.mark.parametrize("case", GEMM_EXACT, ids=lambda c: "M{}K{}H{}".format(*c[:3]))
def test_gemm_exact_sums_bitexact(orc, case):
    """Exact-sum inputs: the plain projection and the fused GEGLU equal the
    oracle bit for bit, ragged M included; row padding is left untouched."""
    M, K, H, xpad, opad = case
    say(f"gemm exact sums {case}")
    x = W.small_int_bf16((M, K), 9100 + M)
    w = W.small_int_bf16((2 * H, K), 9200 + K + H)
    xb, xd = padded(x, K + xpad)
    _, wd = padded(w, K)
    pbuf = torch.full((M, 2 * H + opad), 0x7FC1, dtype=torch.int16,
                      device="cuda").view(torch.bfloat16)
    rgg.gemm_bf16_nt(xd, wd, out=pbuf[:, :2 * H])
    fbuf = torch.full((M, H + opad), 0x7FC1, dtype=torch.int16,
                      device="cuda").view(torch.bfloat16)
    rgg.gemm_geglu_bf16(xd, wd, out=fbuf[:, :H])
    pb, fb = host(pbuf), host(fbuf)
    assert (pb[:, 2 * H:] == 0x7FC1).all() and (fb[:, H:] == 0x7FC1).all(), "wrote into padding"
    assert np.array_equal(host(xb)[:, :K], x), "x modified"
    assert_bitexact(pb[:, :2 * H], orc.gemm_bf16(x, w), f"projection {case}")
    assert_bitexact(fb[:, :H], orc.gemm_geglu(x, w), f"fused geglu {case}")


@pytest.mark.parametrize("case", [(200, 256, 128, 1.0), (515, 1024, 192, 1.0),
                                  (64, 4096, 64, 3.0)],
                         ids=["M200K256", "M515K1024", "M64K4096"])
def test_gemm_gaussian_within_accumulation_bound(orc, case):
    """Gaussian x and 1/sqrt(K)-scaled weights: the projection within the
    accumulation bound of the exact sum, the fused form equal to GEGLU of it."""
    M, K, H, gsig = case
    say(f"gemm gaussian {case}")
    x = W.normal_bf16((M, K), 9300 + K)
    w = W.normal_bf16((2 * H, K), 9400 + K, gsig / np.sqrt(K))
    xd, wd = dev(x), dev(w)
    plain = rgg.gemm_bf16_nt(xd, wd)
    fused = host(rgg.gemm_geglu_bf16(xd, wd))
    again = host(rgg.gelu_and_mul_bf16(plain))
    p = host(plain)
    check_projection_bound(x, w, p, orc.gemm_bf16(x, w), f"projection {case}")
    assert_bitexact(fused, again, f"fused == gelu_and_mul(projection) {case}")
    assert_ulp_bar(fused, orc.gelu_and_mul(p), f"fused vs oracle GEGLU of the projection {case}")


def bf16_rne_any(v):
    """Round float64 values to bf16 bits, ties to even, subnormals included
    (|v| below 2^-126 is rounded to a multiple of 2^-133)."""
    v = np.asarray(v, np.float64)
    sub = np.abs(v) < 2.0 ** -126
    q = np.rint(v / 2.0 ** -133) * 2.0 ** -133
    r = np.where(sub, q, 0.0)
    nrm = bf16_rne_f64(np.where(sub, 1.0, v))
    bits = np.where(sub, (r.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16), nrm)
    return bits.astype(np.uint16)


@pytest.mark.parametrize("case", [("fp32-subnormal products", -65, -70),
                                  ("bf16-subnormal x", -131, 0)],
                         ids=["tiny_products", "subnormal_x"])
def test_gemm_tiny_and_subnormal_operands(orc, case):
    """Operands whose products and partial sums fall in the fp32 subnormal
    range (and bf16-subnormal inputs): every projection output within the
    accumulation bound plus the absolute term K * 2^-149 of the header's
    contract (gradual underflow: each product and each addition off by at most
    half the fp32 subnormal step), against the exact sums of the oracle's
    inputs; the count equal to the oracle is reported."""
    what, ex, ew = case
    M, K, H = 96, 256, 64
    say(f"gemm {what}")
    rng = np.random.Generator(np.random.PCG64(9500 + K))
    xi = rng.integers(-7, 8, (M, K)).astype(np.float64)
    wi = rng.integers(-7, 8, (2 * H, K)).astype(np.float64)
    x = bf16_rne_any(xi * 2.0 ** ex)
    w = bf16_rne_any(wi * 2.0 ** ew)
    xf = W.bf16_bits_to_f32(x).astype(np.float64)
    wf = W.bf16_bits_to_f32(w).astype(np.float64)
    assert np.array_equal(xf, xi * 2.0 ** ex) or ex < -126, "inputs exact"
    got = host(rgg.gemm_bf16_nt(dev(x), dev(w)))
    exact = xf @ wf.T
    mag = np.abs(xf) @ np.abs(wf).T
    E = 2.0 * (K + 16) * 2.0 ** -24 * mag + K * 2.0 ** -149
    lo, hi = ordered(bf16_rne_any(exact - E)), ordered(bf16_rne_any(exact + E))
    g = ordered(got)
    outside = np.count_nonzero((g < lo) | (g > hi))
    want = orc.gemm_bf16(x, w)
    same = np.count_nonzero(got == want)
    say(f"{what}: {got.size} outputs, {got.size - same} differ from the oracle, "
        f"{outside} outside the bound, {np.count_nonzero(want == 0)} oracle zeros, "
        f"{np.count_nonzero((want & 0x7F80) == 0)} oracle subnormal or zero")
    assert outside == 0, f"{what}: {outside} outputs outside the bound"


def test_gemm_zero_k_and_empty(orc):
    """K = 0: every projection output is +0 and GEGLU of it is +0; M = 0 and
    hidden = 0 are no-ops."""
    say("gemm K=0 / empty")
    x = torch.empty((5, 0), dtype=torch.bfloat16, device="cuda")
    w = torch.empty((128, 0), dtype=torch.bfloat16, device="cuda")
    p = rgg.gemm_bf16_nt(x, w, out=torch.full((5, 128), 3.0, dtype=torch.bfloat16, device="cuda"))
    f = rgg.gemm_geglu_bf16(x, w, out=torch.full((5, 64), 3.0, dtype=torch.bfloat16, device="cuda"))
    assert (host(p) == 0).all() and (host(f) == 0).all()
    e = rgg.gemm_geglu_bf16(torch.empty((0, 64), dtype=torch.bfloat16, device="cuda"),
                            dev(W.normal_bf16((128, 64), 9501)))
    assert e.shape == (0, 64)
    h0 = rgg.gemm_bf16_nt(dev(W.normal_bf16((3, 64), 9502)),
                          torch.empty((0, 64), dtype=torch.bfloat16, device="cuda"))
    assert h0.shape == (3, 0)


def test_gemm_long_k_and_widest_strides(orc):
    """Exact-sum inputs with K = 16384 (partial sums stay exact in fp32), and
    x and W rows at the largest row stride the projection takes (2^22 - 8
    elements: 256 rows of x span 2 GiB), bit-exact with the oracle."""
    say("gemm K = 16384")
    x = W.small_int_bf16((200, 16384), 9801)
    w = W.small_int_bf16((128, 16384), 9802)
    assert_bitexact(host(rgg.gemm_geglu_bf16(dev(x), dev(w))), orc.gemm_geglu(x, w), "K 16384 fused")
    assert_bitexact(host(rgg.gemm_bf16_nt(dev(x), dev(w))), orc.gemm_bf16(x, w), "K 16384 plain")
    stride = (1 << 22) - 8
    say(f"gemm row stride {stride} (x 256 rows, W 256 rows)")
    M, K, H = 256, 64, 128
    xs = W.small_int_bf16((M, K), 9803)
    ws = W.small_int_bf16((2 * H, K), 9804)
    bx = torch.empty((M, stride), dtype=torch.bfloat16, device="cuda")
    bw = torch.empty((2 * H, stride), dtype=torch.bfloat16, device="cuda")
    bx[:, :K].copy_(dev(xs))
    bw[:, :K].copy_(dev(ws))
    got_f = host(rgg.gemm_geglu_bf16(bx[:, :K], bw[:, :K]))
    got_p = host(rgg.gemm_bf16_nt(bx[:, :K], bw[:, :K]))
    del bx, bw
    torch.cuda.empty_cache()
    assert_bitexact(got_f, orc.gemm_geglu(xs, ws), "widest strides fused")
    assert_bitexact(got_p, orc.gemm_bf16(xs, ws), "widest strides plain")


def test_gemm_side_stream_and_first_calls_from_threads(orc):
    """In a fresh process, four host threads make their first projection
    calls at once (the per-device kernel attribute and the GELU table are
    set up once), each on its own stream; every result matches the oracle."""
    import subprocess
    import sys
    import tempfile
    code = r"""
import sys, threading
sys.path.insert(0, %r)
import numpy as np
import torch
import bf16_rope_geglu_amd as rgg
import workloads as W
N = 4
xs = [W.small_int_bf16((300 + 50 * k, 128), 9700 + k) for k in range(N)]
ws = [W.small_int_bf16((256, 128), 9710 + k) for k in range(N)]
dx = [torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda() for a in xs]
dw = [torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda() for a in ws]
outs = [None] * N
streams = [torch.cuda.Stream() for _ in range(N)]
torch.cuda.synchronize()
go = threading.Barrier(N)
def work(k):
    with torch.cuda.stream(streams[k]):
        go.wait()
        outs[k] = rgg.gemm_geglu_bf16(dx[k], dw[k]) if k %% 2 == 0 else rgg.gemm_bf16_nt(dx[k], dw[k])
threads = [threading.Thread(target=work, args=(k,)) for k in range(N)]
for t in threads: t.start()
for t in threads: t.join()
torch.cuda.synchronize()
for k in range(N):
    np.save(sys.argv[1] + "/x%%d.npy" %% k, xs[k])
    np.save(sys.argv[1] + "/w%%d.npy" %% k, ws[k])
    np.save(sys.argv[1] + "/out%%d.npy" %% k, outs[k].view(torch.int16).cpu().numpy().view(np.uint16))
print("ok", flush=True)
""" % os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    say("gemm first calls from 4 threads (fresh process)")
    with tempfile.TemporaryDirectory() as d:
        r = subprocess.run([sys.executable, "-c", code, d], capture_output=True, text=True,
                           timeout=110)
        assert r.returncode == 0 and "ok" in r.stdout, r.stderr[-2000:]
        for k in range(4):
            x, w = np.load(f"{d}/x{k}.npy"), np.load(f"{d}/w{k}.npy")
            got = np.load(f"{d}/out{k}.npy")
            want = orc.gemm_geglu(x, w) if k % 2 == 0 else orc.gemm_bf16(x, w)
            assert_bitexact(got, want, f"thread {k}")


def test_gemm_full_size(orc):
    """The dit-layer projection at its full size, 32768 x 4096 times
    (2 x 8192) x 4096: exact-sum inputs bit-exact with the oracle on sampled
    rows; Gaussian inputs within the accumulation bound on sampled rows; the
    fused output equal to GEGLU of the projection over the whole tensor."""
    pr = W.WORKLOADS[4]["proj"]
    M, K, H = pr["rows"], pr["dim"], pr["hidden"]
    rng = np.random.Generator(np.random.PCG64(9600))
    rsel = np.unique(np.concatenate([[0, 127, 128, M - 1], rng.integers(0, M, 4)]))
    rs = torch.from_numpy(rsel).cuda()
    say(f"gemm full size exact sums: {M} x {K} x {2 * H}, rows {rsel.tolist()}")
    x = W.device_small_int_bf16((M, K), W.seed_for(4, "x"))
    w = W.device_small_int_bf16((2 * H, K), W.seed_for(4, "weight"))
    fused = rgg.gemm_geglu_bf16(x, w)
    hx, hw = host(x[rs]), host(w)
    assert_bitexact(host(fused[rs]), orc.gemm_geglu(hx, hw), "full size fused, exact sums")
    plain = rgg.gemm_bf16_nt(x, w)
    assert_bitexact(host(plain[rs]), orc.gemm_bf16(hx, hw), "full size projection, exact sums")
    del plain, fused, x, w
    say("gemm full size gaussian")
    x = W.device_normal_bf16((M, K), W.seed_for(4, "x"))
    w = W.device_normal_bf16((2 * H, K), W.seed_for(4, "weight"), 1.0 / np.sqrt(K))
    plain = rgg.gemm_bf16_nt(x, w)
    fused = rgg.gemm_geglu_bf16(x, w)
    again = rgg.gelu_and_mul_bf16(plain)
    bad = int((fused.view(torch.int16) != again.view(torch.int16)).sum())
    say(f"full size fused vs gelu_and_mul(projection): {bad} of {fused.numel()} differ")
    assert bad == 0
    hx, hw = host(x[rs]), host(w)
    check_projection_bound(hx, hw, host(plain[rs]), orc.gemm_bf16(hx, hw),
                           "full size projection, gaussian")


@pytest.mark.parametrize("K", [64, 192, 320])
def test_gemm_several_tiles_per_workgroup(orc, K):
    """More output tiles than workgroups (17 x 16 = 272, ragged last row
    block), so workgroups walk several tiles in turn, with K of 1, 3 and 5
    slices of 64 (an odd count ends a tile in the other LDS stage):
    exact-sum inputs bit-exact with the oracle, fused and plain, on rows
    sampled from every row block."""
    M, H = 17 * 256 - 3, 16 * 128
    rng = np.random.Generator(np.random.PCG64(9700 + K))
    rsel = np.unique(np.concatenate([np.arange(0, M, 256), np.arange(255, M, 256),
                                     rng.integers(0, M, 8), [M - 1]]))
    rs = torch.from_numpy(rsel).cuda()
    say(f"gemm several tiles per workgroup: {M} x {K} x {2 * H}, {len(rsel)} rows")
    x = W.device_small_int_bf16((M, K), 9700 + K)
    w = W.device_small_int_bf16((2 * H, K), 9800 + K)
    fused = rgg.gemm_geglu_bf16(x, w)
    plain = rgg.gemm_bf16_nt(x, w)
    hx, hw = host(x[rs]), host(w)
    assert_bitexact(host(fused[rs]), orc.gemm_geglu(hx, hw), f"several tiles fused K={K}")
    assert_bitexact(host(plain[rs]), orc.gemm_bf16(hx, hw), f"several tiles projection K={K}")


# ---------------------------------------------------------------------------
# layouts, limits, graphs
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("shape", [(2, 40, 6, 64, 64), (2, 37, 8, 64, 32), (1, 50, 16, 128, 128),
                                   (2, 19, 4, 128, 96)],
                         ids=["H6D64", "H8D64R32", "H16D128", "H4D128R96"])
def test_rope_into_attention_layout(orc, shape):
    """Outputs written straight into a (B, H, S, D) buffer (the layout an
    attention kernel reads) through output strides, q and k in one launch:
    a token whose vectors do not fill whole waves (H6D64), and tokens that
    do (the streaming-store path, rotary parts with and without a tail, the
    last workgroup partly past the end)."""
    B, S, H, D, R = shape
    say(f"rope into (B,H,S,D) outputs {shape}")
    q = W.normal_bf16((B, S, H, D), 8401)
    k = W.normal_bf16((B, S, H, D), 8402)
    cos, sin = orc.rope_cossin(W.freqs_unpaired(S, B, R, 8403))
    oq = torch.empty((B, H, S, D), dtype=torch.bfloat16, device="cuda")
    ok = torch.empty((B, H, S, D), dtype=torch.bfloat16, device="cuda")
    rgg.rope_rotate_half_bf16([dev(q), dev(k)], dev(cos), dev(sin),
                              out=[oq.permute(0, 2, 1, 3), ok.permute(0, 2, 1, 3)])
    assert_bitexact(host(oq).transpose(0, 2, 1, 3), oracle_rope(orc, q, cos, sin), "q -> BHSD")
    assert_bitexact(host(ok).transpose(0, 2, 1, 3), oracle_rope(orc, k, cos, sin), "k -> BHSD")


@pytest.mark.parametrize("shape", [(1, 3, 2, 2048, 1024), (1, 5, 1, 8192, 4096),
                                   (2, 7, 3, 512, 512), (1, 2, 4, 1024, 16),
                                   (2, 9, 20, 128, 112), (1, 4, 3, 1024, 1008),
                                   (1, 3, 1, 8192, 8192)],
                         ids=["D2048R1024", "D8192R4096", "D512R512", "D1024R16",
                              "H20D128R112", "D1024R1008", "D8192R8192"])
def test_rope_wide_heads(orc, shape):
    """Head widths up to the 8192-column limit, with and without tails."""
    B, S, H, D, R = shape
    say(f"rope wide heads {shape}")
    x = W.special_bf16((B, S, H, D), 8500 + D)
    cos, sin = orc.rope_cossin(W.freqs_unpaired(S, B, R, 8501 + D))
    out = rgg.rope_rotate_half_bf16(dev(x), dev(cos), dev(sin))
    assert_bitexact(host(out), oracle_rope(orc, x, cos, sin), f"wide {shape}")


@pytest.mark.parametrize("R", [16, 64], ids=["lane_path", "slot_path"])
def test_rope_launch_split_over_many_workgroups(orc, R):
    """4 views x 262147 one-token workgroups is more than one launch takes
    (2^20 workgroups), so the call is split; tokens on both sides of the split
    and at the ends are checked.  Inputs are stride-0 views of one row per
    view, so only the outputs take memory (4 x 1.1 GB)."""
    B, S, H, D, nv = 1, 262147, 1, 2112, 4
    say(f"rope split launch: S={S} H={H} D={D} R={R} views={nv}")
    rows = [W.special_bf16((1, 1, H, D), 8600 + R + v) for v in range(nv)]
    cos = W.normal_bf16((B * S, R), 8610 + R)
    sin = W.normal_bf16((B * S, R), 8620 + R)
    xs = [dev(r).expand(B, S, H, D) for r in rows]
    outs = [torch.empty((B, S, H, D), dtype=torch.bfloat16, device="cuda") for _ in range(nv)]
    rgg.rope_rotate_half_bf16(xs, dev(cos), dev(sin), out=outs)
    split = (1 << 20) // nv
    rng = np.random.Generator(np.random.PCG64(8630))
    tokens = sorted({0, 1, split - 1, split, split + 1, S - 1} |
                    set(rng.integers(0, S, 16).tolist()))
    for v in range(nv):
        got = np.stack([host(outs[v][0, t]) for t in tokens])
        want = np.stack([orc.rope_rotate_half(rows[v], cos[t:t + 1], sin[t:t + 1])[0, 0]
                         for t in tokens])
        assert_bitexact(got, want, f"view {v}, tokens {tokens[:6]}...")


def test_geglu_wide_rows(orc):
    say("geglu wide rows")
    inp = W.special_bf16((3, 2 * 65536), 8601)
    out = host(rgg.gelu_and_mul_bf16(dev(inp)))
    want = orc.gelu_and_mul(inp)
    nan = ((want & 0x7F80) == 0x7F80) & ((want & 0x7F) != 0)
    assert_ulp_bar(out[~nan], want[~nan], "geglu 3 x 65536")


def test_graph_capture_replays(orc):
    """The entry points captured in one HIP graph (tables, RoPE, GEGLU and the
    projection with GEGLU fused) and replayed several times, with eager work
    and synchronisation between replays; every replay matches the eager
    result."""
    say("graph capture of the whole path")
    rgg.prepare_device(0)
    B, S, H, D, R = 1, 64, 4, 64, 64
    fr = torch.from_numpy(W.freqs_1d(S, B, R)).cuda()
    x = dev(W.normal_bf16((B, S, H, D), 8701))
    inp = dev(W.normal_bf16((96, 2 * 128), 8702, 2.0))
    cos = torch.empty((B * S, R), dtype=torch.bfloat16, device="cuda")
    sin = torch.empty_like(cos)
    xo = torch.empty_like(x)
    go = torch.empty((96, 128), dtype=torch.bfloat16, device="cuda")
    xg = dev(W.normal_bf16((300, 128), 8703))
    wg = dev(W.normal_bf16((256, 128), 8704, 1.0 / np.sqrt(128)))
    pg = torch.empty((300, 128), dtype=torch.bfloat16, device="cuda")

    def path():
        rgg.rope_cossin_precompute(fr, cos, sin)
        rgg.rope_rotate_half_bf16(x, cos, sin, out=xo)
        rgg.gelu_and_mul_bf16(inp, go)
        rgg.gemm_geglu_bf16(xg, wg, pg)

    outs = (cos, sin, xo, go, pg)
    path()
    want = [host(t).copy() for t in outs]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        path()
    for rep in range(4):
        for t in outs:
            t.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = [host(t) for t in outs]
        for g, w, name in zip(got, want, ("cos", "sin", "rope", "geglu", "projection geglu")):
            assert np.array_equal(g, w), f"replay {rep}: {name} differs from eager"
        _ = (x.float() * 2).sum().item()  # eager work between replays


def test_first_gelu_call_while_capturing_is_refused():
    """In a fresh process, a first GEGLU call made under graph capture returns
    RGG_ERR_CAPTURING instead of building its table; rgg_prepare_device then
    makes capture work."""
    import subprocess
    import sys
    code = r"""
import sys
sys.path.insert(0, %r)
import torch
import bf16_rope_geglu_amd as rgg
inp = torch.zeros((8, 16), dtype=torch.bfloat16, device="cuda")
out = torch.empty((8, 8), dtype=torch.bfloat16, device="cuda")
torch.cuda.synchronize()
g = torch.cuda.CUDAGraph()
status = None
with torch.cuda.graph(g):
    try:
        rgg.gelu_and_mul_bf16(inp, out)
    except rgg.RggError as e:
        status = e.status
print("status", status, flush=True)
rgg.prepare_device(0)
g2 = torch.cuda.CUDAGraph()
with torch.cuda.graph(g2):
    rgg.gelu_and_mul_bf16(inp, out)
g2.replay()
torch.cuda.synchronize()
print("ok", flush=True)
""" % os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=240)
    say(r.stdout.strip())
    assert r.returncode == 0, r.stderr[-2000:]
    assert "status 7" in r.stdout and "ok" in r.stdout


def test_first_gelu_calls_from_several_threads(orc):
    """In a fresh process, four host threads make their first GEGLU call at
    once, each on its own stream: the one-time table build is serialized and
    waited for, so every thread's result is right."""
    import subprocess
    import sys
    code = r"""
import sys, threading
sys.path.insert(0, %r)
import numpy as np
import torch
import bf16_rope_geglu_amd as rgg
import workloads as W
N = 4
inps = [W.normal_bf16((512, 2 * 1024), 9100 + k, 2.0) for k in range(N)]
dev = [torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda() for a in inps]
outs = [None] * N
streams = [torch.cuda.Stream() for _ in range(N)]
torch.cuda.synchronize()
go = threading.Barrier(N)
def work(k):
    with torch.cuda.stream(streams[k]):
        go.wait()
        outs[k] = rgg.gelu_and_mul_bf16(dev[k])
threads = [threading.Thread(target=work, args=(k,)) for k in range(N)]
for t in threads: t.start()
for t in threads: t.join()
torch.cuda.synchronize()
for k in range(N):
    np.save(sys.argv[1] + "/out%%d.npy" %% k, outs[k].view(torch.int16).cpu().numpy().view(np.uint16))
print("ok", flush=True)
""" % os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    import tempfile
    with tempfile.TemporaryDirectory() as d:
        r = subprocess.run([sys.executable, "-c", code, d], capture_output=True, text=True,
                           timeout=240)
        say(r.stdout.strip(), r.stderr.strip()[-500:])
        assert r.returncode == 0 and "ok" in r.stdout
        for k in range(4):
            inp = W.normal_bf16((512, 2 * 1024), 9100 + k, 2.0)
            got = np.load(os.path.join(d, f"out{k}.npy"))
            assert_ulp_bar(got, orc.gelu_and_mul(inp), f"thread {k}")


def test_selfcheck_passes():
    """The library's own bit-exactness gate passes on this device, on the
    default stream and on a side stream, twice in a row."""
    say("selfcheck")
    assert rgg.selfcheck() == 0
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        assert rgg.selfcheck() == 0
    torch.cuda.synchronize()


def test_selfcheck_refused_while_capturing():
    say("selfcheck under capture")
    rgg.prepare_device(0)
    ws = torch.empty(rgg.SELFCHECK_WORKSPACE_BYTES, dtype=torch.uint8, device="cuda")
    g = torch.cuda.CUDAGraph()
    status = None
    with torch.cuda.graph(g):
        status = rgg.library().rgg_selfcheck(
            ws.data_ptr(), ws.numel(), torch.cuda.current_stream().cuda_stream, None)
    assert status == 7
    torch.cuda.synchronize()


# ---------------------------------------------------------------------------
# The C ABI from plain C: tests/host/capi_client.c, no Python in between
# ---------------------------------------------------------------------------

CLIENT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "host", "_bin", "capi_client")


def test_plain_c_client(orc, tmp_path):
    import subprocess

    assert os.path.exists(CLIENT), "tests/host/_bin/capi_client is not built"
    S, B, H, D, R, rows, hidden = 300, 2, 3, 64, 48, 77, 136
    M, K, Hp = 333, 192, 192
    say(f"C client: rope ({B},{S},{H},{D}) R={R}, geglu ({rows},{hidden}), "
        f"projection ({M},{K}) x (2*{Hp},{K})")
    freqs = W.freqs_unpaired(S, B, R, 71)
    x = W.normal_bf16((B, S, H, D), 72)
    inp = np.concatenate([W.normal_bf16((rows, hidden), 73, 2.0),
                          W.normal_bf16((rows, hidden), 74)], axis=1)
    px = W.small_int_bf16((M, K), 75)
    pw = W.small_int_bf16((2 * Hp, K), 76)
    src, dst = tmp_path / "in.bin", tmp_path / "out.bin"
    with open(src, "wb") as f:
        f.write(np.array([S, B, H, D, R, rows, hidden, M, K, Hp], np.int64).tobytes())
        f.write(np.ascontiguousarray(freqs, np.float32).tobytes())
        f.write(np.ascontiguousarray(x, np.uint16).tobytes())
        f.write(np.ascontiguousarray(inp, np.uint16).tobytes())
        f.write(np.ascontiguousarray(px, np.uint16).tobytes())
        f.write(np.ascontiguousarray(pw, np.uint16).tobytes())
    proc = subprocess.run([CLIENT, str(src), str(dst)], capture_output=True, text=True,
                          timeout=60)
    say(proc.stdout.strip(), proc.stderr.strip())
    assert proc.returncode == 0, f"capi_client exit status {proc.returncode}"
    got = np.fromfile(dst, np.uint16)
    n_t, n_x = B * S * R, x.size
    n_o = rows * hidden
    assert got.size == 2 * n_t + n_x + n_o + M * Hp + M * 2 * Hp
    cos, sin = got[:n_t].reshape(B * S, R), got[n_t:2 * n_t].reshape(B * S, R)
    rope = got[2 * n_t:2 * n_t + n_x].reshape(x.shape)
    geglu = got[2 * n_t + n_x:2 * n_t + n_x + n_o].reshape(rows, hidden)
    fused = got[2 * n_t + n_x + n_o:2 * n_t + n_x + n_o + M * Hp].reshape(M, Hp)
    proj = got[2 * n_t + n_x + n_o + M * Hp:].reshape(M, 2 * Hp)
    oc, os_ = orc.rope_cossin(freqs)
    assert_ulp_bar(cos, oc, "C client cos")
    assert_ulp_bar(sin, os_, "C client sin")
    assert_bitexact(rope, oracle_rope(orc, x, cos, sin), "C client rope")
    assert_ulp_bar(geglu, orc.gelu_and_mul(inp), "C client geglu")
    assert_bitexact(fused, orc.gemm_geglu(px, pw), "C client projection + GEGLU")
    assert_bitexact(proj, orc.gemm_bf16(px, pw), "C client projection")
