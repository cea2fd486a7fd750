"""The C ABI on the host, without a GPU.

Covers: the library loads and exports every function include/rgg.h declares,
status strings, every argument check that returns before anything is
enqueued (made with fake device addresses, which are never dereferenced),
the overlap analysis against brute force (host-only C++ under ASan/UBSan),
and the Python binding's own argument checks.  No call here reaches a launch.
"""
import ctypes
import os
import re
import sys
import subprocess

import pytest
import torch

import bf16_rope_geglu_amd as rgg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rgg.h")

OK, NULL, SHAPE, UNSUPPORTED, ALIGN, ALIAS, HIP, CAPTURING, SELFCHECK = range(9)
A = 0x7F0000000000  # a 16-byte aligned fake device address


def declared_functions():
    with open(HEADER) as f:
        text = f.read()
    return re.findall(r"RGG_API\s+[\w\s\*]+?\b(\w+)\s*\(", text)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(rgg.LIBRARY):
        import bf16_rope_geglu_amd.build as b
        b.build()
    return rgg.library()


def test_exports_every_declared_function(lib):
    names = declared_functions()
    assert set(names) == {"rope_cossin_precompute", "rope_cossin_from_grid",
                          "rope_rotate_half_bf16", "gelu_and_mul_bf16", "gemm_bf16_nt",
                          "gemm_geglu_bf16", "rgg_prepare_device", "rgg_selfcheck", "rgg_selfcheck_noalloc",
                          "rgg_status_string"}
    for n in names:
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", rgg.LIBRARY], capture_output=True,
                         text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    assert set(names) <= exported


def test_status_strings(lib):
    for code in range(9):
        s = lib.rgg_status_string(code)
        assert s and s.decode() != "unknown status"
    assert lib.rgg_status_string(99).decode() == "unknown status"


def cossin(lib, freqs=A, S=4, B=2, R=8, ss=16, sb=8, cos=A + 4096, sin=A + 8192):
    return lib.rope_cossin_precompute(freqs, S, B, R, ss, sb, cos, sin, None)


def test_cossin_checks(lib):
    assert cossin(lib, freqs=None) == NULL
    assert cossin(lib, cos=None) == NULL
    assert cossin(lib, S=-1) == SHAPE
    assert cossin(lib, ss=-4) == SHAPE
    assert cossin(lib, R=12) == UNSUPPORTED
    assert cossin(lib, freqs=A + 4) == ALIGN
    assert cossin(lib, cos=A + 4096 + 2) == ALIGN
    assert cossin(lib, ss=18) == ALIGN
    assert cossin(lib, sin=A + 4096 + 16) == ALIAS   # tables overlap
    assert cossin(lib, cos=A + 16) == ALIAS          # table over the angles
    assert cossin(lib, S=0) == OK
    assert cossin(lib, B=0, freqs=None) == OK
    assert cossin(lib, R=0) == OK


def grid(lib, B=2, T=1, Hg=4, Wg=4, d=(4, 6, 6), theta=1e4, off=None, cos=A, sin=A + 8192):
    return lib.rope_cossin_from_grid(B, T, Hg, Wg, *d, theta, off, cos, sin, None)


def test_grid_checks(lib):
    assert grid(lib, cos=None) == NULL
    assert grid(lib, B=-1) == SHAPE
    assert grid(lib, d=(4, 5, 7)) == SHAPE           # odd axis width
    assert grid(lib, d=(-2, 6, 12)) == SHAPE
    assert grid(lib, theta=0.0) == SHAPE
    assert grid(lib, theta=float("inf")) == SHAPE
    assert grid(lib, theta=float("nan")) == SHAPE
    assert grid(lib, d=(4, 6, 2)) == UNSUPPORTED     # R = 12
    assert grid(lib, d=(4096, 4096, 16)) == UNSUPPORTED  # R > 8192
    assert grid(lib, cos=A + 2) == ALIGN
    assert grid(lib, off=A + 1 + (1 << 20)) == ALIGN
    assert grid(lib, sin=A + 16) == ALIAS            # tables overlap
    assert grid(lib, off=A + 64) == ALIAS            # offsets inside a table
    assert grid(lib, T=0) == OK
    assert grid(lib, B=0, cos=None) == OK
    assert grid(lib, d=(0, 0, 0)) == OK


def view(x=A, out=A + (1 << 24), xs=(8192, 1024, 128), os_=(8192, 1024, 128)):
    return rgg.RopeView(x, out, *xs, *os_)


def rope(lib, views, n=None, B=2, S=8, H=8, D=128, R=128, cos=A + (1 << 26),
         sin=A + (1 << 26) + (1 << 20)):
    arr = (rgg.RopeView * max(1, len(views)))(*views)
    n = len(views) if n is None else n
    return lib.rope_rotate_half_bf16(arr if views else None, n, B, S, H, D, R, cos, sin, None)


def test_rope_checks(lib):
    v = view()
    assert rope(lib, [v], n=0) == SHAPE
    assert rope(lib, [v], n=5) == SHAPE
    assert rope(lib, [v], R=3) == SHAPE
    assert rope(lib, [v], R=144) == SHAPE             # R > D
    assert rope(lib, [v], B=-1) == SHAPE
    assert rope(lib, [view(xs=(8192, -1024, 128))]) == SHAPE
    assert rope(lib, [v], D=12, R=0) == UNSUPPORTED
    assert rope(lib, [v], R=24, D=32) == UNSUPPORTED  # half not a whole vector
    assert rope(lib, [], n=1) == NULL
    assert rope(lib, [view(x=None)]) == NULL
    assert rope(lib, [v], cos=None) == NULL
    assert rope(lib, [view(x=A + 8)]) == ALIGN
    assert rope(lib, [view(xs=(8192, 1024, 132))]) == ALIGN
    assert rope(lib, [v], sin=A + (1 << 26) + 2) == ALIGN
    # output rows overlapping each other
    assert rope(lib, [view(os_=(8192, 1024, 64))]) == UNSUPPORTED
    # partial overlap of out and x, and of out and the tables
    assert rope(lib, [view(out=A + 256)]) == ALIAS
    assert rope(lib, [view(out=A + (1 << 26))]) == ALIAS
    # two views writing the same place; one view's out over another's x
    assert rope(lib, [view(), view(x=A + (1 << 22))]) == ALIAS
    assert rope(lib, [view(), view(x=A + (1 << 22), out=A)]) == ALIAS
    # empty is a no-op
    assert rope(lib, [v], B=0) == OK
    assert rope(lib, [v], S=0, cos=None, sin=None) == OK


def gelu(lib, inp=A, rows=16, hidden=64, is_=128, out=A + (1 << 20), os_=64):
    return lib.gelu_and_mul_bf16(inp, rows, hidden, is_, out, os_, None)


def test_gelu_checks(lib):
    assert gelu(lib, rows=-1) == SHAPE
    assert gelu(lib, is_=-8) == SHAPE
    assert gelu(lib, hidden=12) == UNSUPPORTED
    assert gelu(lib, os_=56) == UNSUPPORTED
    assert gelu(lib, inp=None) == NULL
    assert gelu(lib, out=None) == NULL
    assert gelu(lib, inp=A + 2) == ALIGN
    assert gelu(lib, is_=132) == ALIGN
    assert gelu(lib, out=A + 64) == ALIAS             # inside the input, not the in-place form
    assert gelu(lib, out=A, os_=64) == ALIAS          # in place needs the input's row stride
    assert gelu(lib, rows=0) == OK
    assert gelu(lib, hidden=0, inp=None) == OK


def gemm(lib, x=A, M=256, K=128, xs=128, w=A + (1 << 24), N=256, ws=128, out=A + (1 << 25),
         os_=256, geglu=False):
    f = lib.gemm_geglu_bf16 if geglu else lib.gemm_bf16_nt
    return f(x, M, K, xs, w, N, ws, out, os_, None)


@pytest.mark.parametrize("geglu", [False, True])
def test_gemm_checks(lib, geglu):
    N = 128 if geglu else 256          # hidden for the fused form, 2*hidden for the plain one
    g = lambda **kw: gemm(lib, N=kw.pop("N", N), os_=kw.pop("os_", N), geglu=geglu, **kw)
    assert g(M=-1) == SHAPE
    assert g(K=-64) == SHAPE
    assert g(N=-128) == SHAPE
    assert g(xs=-128) == SHAPE
    assert g(K=96, xs=96, ws=96) == UNSUPPORTED        # K not a multiple of 64
    assert g(N=N + 32, os_=N + 32) == UNSUPPORTED      # hidden not a multiple of 64
    assert g(xs=64) == UNSUPPORTED                     # x rows shorter than K
    assert g(ws=64) == UNSUPPORTED                     # W rows shorter than K
    assert g(os_=N - 8) == UNSUPPORTED                 # output rows shorter than the output
    assert g(x=None) == NULL
    assert g(w=None) == NULL
    assert g(out=None) == NULL
    assert g(x=A + 8) == ALIGN
    assert g(w=A + (1 << 24) + 2) == ALIGN
    assert g(xs=136 + 4) == ALIGN
    assert g(os_=N + 4) == ALIGN
    assert g(out=A + 4096) == ALIAS                    # inside x
    assert g(out=A + (1 << 24) + 4096) == ALIAS        # inside W
    assert g(M=0) == OK
    assert g(N=0, os_=0, w=None) == OK
    assert g(M=1 << 31) == UNSUPPORTED                 # M >= 2^31
    h = 1 << 15                                        # 2^8 column blocks of 128
    assert g(M=1 << 24, N=h * (1 if geglu else 2),
             os_=h * (1 if geglu else 2)) == UNSUPPORTED   # 2^16 x 2^8 = 2^24 blocks
    assert g(K=1 << 31, xs=1 << 31, ws=1 << 31) == UNSUPPORTED   # K >= 2^31
    assert g(xs=1 << 22) == UNSUPPORTED                # x row stride >= 2^22
    assert g(ws=1 << 22) == UNSUPPORTED                # W row stride >= 2^22


def test_gemm_plain_needs_whole_gate_up_pairs(lib):
    assert gemm(lib, N=192, os_=192) == UNSUPPORTED    # N = 2*96: hidden not a multiple of 64
    assert gemm(lib, N=-1) == SHAPE


def test_prepare_device_bad_index(lib):
    assert lib.rgg_prepare_device(-1) == SHAPE


def test_overlap_analysis_bruteforce(tmp_path):
    exe = os.path.join(tmp_path, "layout_check")
    subprocess.run(["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=all",
                    "-I", os.path.join(ROOT, "bf16_rope_geglu_amd", "csrc"),
                    os.path.join(ROOT, "tests", "host", "layout_check.cpp"), "-o", exe],
                   check=True)
    r = subprocess.run([exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.startswith("ok")


def test_fastdiv_matches_division(tmp_path):
    exe = os.path.join(tmp_path, "fastdiv_check")
    subprocess.run(["g++", "-std=c++17", "-O2", "-D__HIP_PLATFORM_AMD__",
                    "-I", os.path.join(ROOT, "bf16_rope_geglu_amd", "csrc"),
                    "-I", "/opt/rocm/include",
                    os.path.join(ROOT, "tests", "host", "fastdiv_check.cpp"), "-o", exe],
                   check=True)
    r = subprocess.run([exe], capture_output=True, text=True)
    assert r.returncode == 0 and "ok" in r.stdout, r.stdout + r.stderr


def test_binding_rejects_host_tensors():
    x = torch.zeros(1, 4, 2, 16, dtype=torch.bfloat16)
    cs = torch.zeros(4, 16, dtype=torch.bfloat16)
    with pytest.raises(TypeError):
        rgg.rope_rotate_half_bf16(x, cs, cs)
    with pytest.raises(TypeError):
        rgg.gelu_and_mul_bf16(torch.zeros(4, 16, dtype=torch.bfloat16))
    with pytest.raises(TypeError):
        rgg.rope_cossin_precompute(torch.zeros(4, 1, 1, 16))
    tab = torch.zeros(2 * 16, 16, dtype=torch.bfloat16)
    with pytest.raises(TypeError):
        rgg.rope_cossin_from_grid(2, (1, 4, 4), (4, 6, 6), cos_out=tab, sin_out=tab.clone())
    xp = torch.zeros(8, 64, dtype=torch.bfloat16)
    wp = torch.zeros(128, 64, dtype=torch.bfloat16)
    with pytest.raises(TypeError):
        rgg.gemm_geglu_bf16(xp, wp)
    with pytest.raises(TypeError):
        rgg.gemm_bf16_nt(xp, wp)


def test_binding_projection_shape_checks():
    """Shape errors are raised before anything reaches the library (or a
    device): weight not (N, K) with the input's K, an odd gate/up row count."""
    xp = torch.zeros(8, 64, dtype=torch.bfloat16)
    with pytest.raises((ValueError, TypeError)):
        rgg.gemm_geglu_bf16(xp, torch.zeros(128, 32, dtype=torch.bfloat16))
    with pytest.raises(ValueError):
        rgg.gemm_geglu_bf16(xp, torch.zeros(129, 64, dtype=torch.bfloat16))
    with pytest.raises(ValueError):
        rgg.gemm_bf16_nt(xp, torch.zeros(128, 64, 1, dtype=torch.bfloat16))


def test_binding_error_carries_status(lib):
    err = rgg.RggError("f", ALIAS, lib.rgg_status_string(ALIAS).decode())
    assert err.status == ALIAS and "overlaps" in str(err)


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_c_client_compiles_as_c11(tmp_path):
    """include/rgg.h is usable from plain C: the client builds with gcc -Werror."""
    import bf16_rope_geglu_amd.build as libbuild

    exe = libbuild.build_capi_client(out=os.path.join(tmp_path, "capi_client"))
    assert os.path.exists(exe)


def test_stream_reference_loads_and_checks_arguments():
    """The streaming reference bench.py times beside the kernels: exported,
    and bad arguments are refused before anything reaches a device."""
    import bench

    ref = bench.stream_ref_library()

    def call(a=A, b=None, out=A + 4096, n=16, block=256, vpl=1, grid=0, policy=3, lds=0):
        return ref.rgg_stream_ref(a, b, out, n, block, vpl, grid, policy, lds, None)

    assert call(n=0) == 2
    assert call(n=1 << 27) == 2                  # beyond the 32-bit byte offsets of the stores
    assert call(block=96) == 2
    assert call(block=2048) == 2
    assert call(a=A + 8) == 2
    assert call(a=None, b=A) == 2
    assert call(out=None) == 2
    assert call(vpl=3) == 2
    assert call(grid=-1) == 2
    assert call(policy=8) == 2
    assert call(lds=65537) == 2


def test_selfcheck_argument_checks(lib):
    """Refused before any device work: no workspace, too small, misaligned."""
    import ctypes
    failed = ctypes.c_uint32(5)
    assert lib.rgg_selfcheck(None, 1 << 20, None, ctypes.byref(failed)) == NULL
    assert failed.value == 0
    assert lib.rgg_selfcheck(A, (1 << 20) - 1, None, None) == SHAPE
    assert lib.rgg_selfcheck(A + 128, 1 << 20, None, None) == ALIGN


def _c_array(text, name):
    body = re.search(name + r"\[[^=]*=\s*\{(.*?)\};", text, re.S).group(1)
    body = re.sub(r"//[^\n]*", "", body)
    return [int(v, 16) for v in re.findall(r"0x([0-9A-Fa-f]+)", body)]


def test_selfcheck_expected_values_agree_with_oracle_and_mpmath():
    """The self-check's expected bits (hand-derived in selfcheck.cpp) agree
    with the pinned oracle and with 50-digit cos/sin, so a typo there is
    caught without a GPU."""
    import mpmath
    import numpy as np

    import oracle
    o = oracle.get()
    with open(os.path.join(ROOT, "bf16_rope_geglu_amd", "csrc", "selfcheck.cpp")) as f:
        text = f.read()
    angles = np.array(_c_array(text, "kAngles"), np.uint32).view(np.float32)
    cos, sin = _c_array(text, "kCos"), _c_array(text, "kSin")
    oc, os_ = o.rope_cossin(angles.reshape(1, 1, 1, 8))
    assert oc.ravel().tolist() == cos and os_.ravel().tolist() == sin
    mpmath.mp.dps = 50
    for a, c, s_ in zip(angles, cos, sin):
        for fn, bits in ((mpmath.cos, c), (mpmath.sin, s_)):
            v = float(np.array([bits << 16], np.uint32).view(np.float32)[0])
            exact = fn(mpmath.mpf(float(a)))
            if v != 0:
                step = 2.0 ** (int(np.floor(np.log2(abs(v)))) - 7)
                assert abs(exact - v) <= step / 2
    rope = np.array(_c_array(text, "kRope"), np.uint16).reshape(8, 8)
    x = np.concatenate([rope[:, 0], rope[:, 1]]).reshape(1, 1, 1, 16)
    cs = np.concatenate([rope[:, 2], rope[:, 4]]).reshape(1, 16)
    sn = np.concatenate([rope[:, 3], rope[:, 5]]).reshape(1, 16)
    out = o.rope_rotate_half(x, cs, sn).ravel()
    assert out[:8].tolist() == rope[:, 6].tolist() and out[8:].tolist() == rope[:, 7].tolist()
    gel = np.array(_c_array(text, "kGelu"), np.uint16).reshape(8, 2)
    for g, want in gel:
        assert o.gelu_bf16(int(g)) == want
    # bit 6: one-hot x and W built as selfcheck.cpp describes; the oracle's
    # projection copies W's column, and its fused GEGLU gives G or 2 G
    M, K, H = 40, 64, 64
    x = np.zeros((M, K), np.uint16)
    x[np.arange(M), np.arange(M)] = 0x3F80
    w = np.zeros((2 * H, K), np.uint16)
    for j in range(H):
        for m in range(M):
            w[j, m] = gel[(m + j) % 8, 0]
            w[H + j, m] = 0x4000 if (m + j) % 2 else 0x3F80
    assert np.array_equal(o.gemm_bf16(x, w), w[:, :M].T)
    fused = o.gemm_geglu(x, w)
    for m in range(M):
        for j in range(H):
            G = float(np.array([int(gel[(m + j) % 8, 1]) << 16], np.uint32).view(np.float32)[0])
            want = np.array([G * (2.0 if (m + j) % 2 else 1.0)], np.float32).view(np.uint32)[0] >> 16
            assert fused[m, j] == want


def test_cpu_baseline_leg_runs_on_a_small_sample():
    """bench.py's cpu_baseline leg: the oracle on one thread and on all cores."""
    import bench

    out = bench.run_cpu_baseline(4, tokens=64, geglu_rows=16)
    assert out["kind"] == "oracle" and out["cores"] == 1 and out["value"] > 0
    assert out["all_cores"]["cores"] >= 1 and out["all_cores"]["value"] > 0


def test_step_bytes_are_the_three_kernels():
    """One dit_layer step moves 33.55 MB (tables) + 1090.52 MB (q and k RoPE)
    + 1610.61 MB (GEGLU) algorithmically, and nothing else counts."""
    import bench

    assert bench.step_algo_bytes(4) == 33554432 + 1090519040 + 1610612736 == 2734686208


def test_size_limits_are_refused_before_any_launch(lib):
    """Every documented size limit returns RGG_ERR_UNSUPPORTED (the checks run
    before anything touches a device)."""
    v = view()
    assert rope(lib, [v], B=1 << 16, S=1 << 15) == UNSUPPORTED          # B*S = 2^31
    assert rope(lib, [v], D=8200, R=128) == UNSUPPORTED                   # D > 8192
    assert rope(lib, [v], H=4096, D=8192, R=128) == UNSUPPORTED           # H*D = 2^25
    assert gelu(lib, rows=1 << 28, hidden=64, is_=128, os_=64) == UNSUPPORTED  # rows*hidden/8
    assert cossin(lib, S=1 << 16, B=1 << 15) == UNSUPPORTED              # S*B = 2^31
    assert cossin(lib, S=1 << 14, B=1 << 14, R=32) == UNSUPPORTED        # S*B*R/4 = 2^31
    assert grid(lib, B=1, T=1 << 11, Hg=1 << 10, Wg=1 << 10) == UNSUPPORTED  # S = 2^31
    assert grid(lib, B=1 << 12, T=1, Hg=1 << 10, Wg=1 << 9, d=(16, 8, 8)) == UNSUPPORTED


def test_projection_bytes_and_trace_names():
    """The projection's algorithmic bytes (x and W once, output once) and the
    trace summary's names for its two template instances."""
    sys.path.insert(0, ROOT)
    import bench
    b = bench.projection_algo_bytes()
    x, w = 2 * 32768 * 4096, 2 * 16384 * 4096
    assert b == {"projection_geglu": x + w + 2 * 32768 * 8192,
                 "projection_plain": x + w + 2 * 32768 * 16384}
    assert bench._short_kernel(
        "void rgg::(anonymous namespace)::gemm_gate_up_kernel<true>(rgg::GemmParams)") \
        == "gemm_gate_up_kernel<true>"
    assert bench._short_kernel(
        "void rgg::(anonymous namespace)::gemm_gate_up_kernel<false>(rgg::GemmParams)") \
        == "gemm_gate_up_kernel<false>"
    assert bench._short_kernel(
        "void rgg::(anonymous namespace)::rope_rotate_half_kernel<true, false>(rgg::RopeParams)") \
        == "rope_rotate_half_kernel"


def test_counter_summary_medians(tmp_path):
    """bench.py --counter-summary: per dispatch, a counter's hardware
    instances are summed; across dispatches the median is kept; passes in
    separate folders merge; the platform GEMM gets its own column."""
    sys.path.insert(0, ROOT)
    import bench
    head = "Dispatch_Id,Kernel_Name,Counter_Name,Counter_Value\n"
    plain = "void rgg::(anonymous namespace)::gemm_gate_up_kernel<false>(rgg::GemmParams)"
    blas = "Custom_Cijk_Alik_Bljk_BBS_MT256x256x64_gfx950"
    rows1 = [(1, plain, "GRBM_GUI_ACTIVE", 10), (1, plain, "GRBM_GUI_ACTIVE", 5),
             (2, plain, "GRBM_GUI_ACTIVE", 30), (3, plain, "GRBM_GUI_ACTIVE", 20),
             (4, blas, "GRBM_GUI_ACTIVE", 7), (5, "other_kernel", "GRBM_GUI_ACTIVE", 99)]
    rows2 = [(1, plain, "MfmaUtil", 60.0), (2, plain, "MfmaUtil", 70.0), (3, plain, "MfmaUtil", 80.0)]
    for name, rows in (("p1", rows1), ("p2", rows2)):
        d = tmp_path / name
        d.mkdir()
        (d / "x_counter_collection.csv").write_text(
            head + "".join(f'{a},"{b}",{c},{v}\n' for a, b, c, v in rows))
    out = tmp_path / "summary.md"
    bench.counter_summary(str(tmp_path), str(out), "cmd")
    text = out.read_text()
    table = {ln.split("|")[1].strip(): [c.strip() for c in ln.strip().strip("|").split("|")[1:]]
             for ln in text.splitlines() if ln.startswith("| ") and not ln.startswith("| counter")}
    header = [c.strip() for c in text.splitlines()[4].strip().strip("|").split("|")[1:]]
    assert header == ["gemm_gate_up_kernel<false>", "hipBLASLt GEMM (torch.matmul)"]
    assert table["GRBM_GUI_ACTIVE"] == ["20", "7"]      # dispatch 1 sums to 15; median of 15, 30, 20
    assert table["MfmaUtil"] == ["70", ""]


def test_source_digest_tracks_step_code_not_comments(tmp_path, monkeypatch):
    """bench.py keys the committed counter traffic to a digest of the step
    kernels' code: comments and the projection kernel do not move it, any
    other code change in kernels.hip or launch.h does."""
    import bench
    src = open(bench.KERNELS_SRC).read()
    lh = open(bench.LAUNCH_H).read()
    k, h = tmp_path / "kernels.hip", tmp_path / "launch.h"
    k.write_text(src)
    h.write_text(lh)
    monkeypatch.setattr(bench, "KERNELS_SRC", str(k))
    monkeypatch.setattr(bench, "LAUNCH_H", str(h))
    d0 = bench.source_digest()
    h.write_text(lh + "\n// a comment\n/* another */\n")
    assert bench.source_digest() == d0
    h.write_text(lh.replace("kTableNarrowLanes = 1u << 18", "kTableNarrowLanes = 1u << 17"))
    assert bench.source_digest() != d0
    h.write_text(lh)
    k.write_text(src.replace("kGemmStaggerRow = 4", "kGemmStaggerRow = 3"))
    assert bench.source_digest() == d0
    k.write_text(src.replace("constexpr uint32_t kTieGuard = 4;", "constexpr uint32_t kTieGuard = 5;"))
    assert bench.source_digest() != d0
