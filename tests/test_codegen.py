"""Guards on the generated gfx950 code of the hot kernels (no GPU needed).

The projection kernel writes M0 itself (it holds the LDS address of the
direct global-to-LDS loads) in inline assembly. M0 is a reserved register:
the compiler does not save it across an asm statement, so the asm is only
safe while no compiler-generated instruction in that kernel reads or
writes M0. This test compiles kernels.hip to gfx950 assembly with the
library's flags and fails if that ever changes (a compiler upgrade, an edit
of the kernel), and also if a hot kernel starts spilling to scratch memory.
"""
import os
import re
import subprocess

import pytest

from bf16_rope_geglu_amd import build

HOT = {
    "gemm_gate_up_kernel<true>": "_ZN3rgg12_GLOBAL__N_119gemm_gate_up_kernelILb1EEEvNS_10GemmParamsE",
    "gemm_gate_up_kernel<false>": "_ZN3rgg12_GLOBAL__N_119gemm_gate_up_kernelILb0EEEvNS_10GemmParamsE",
}


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    out = os.path.join(tmp_path_factory.mktemp("codegen"), "kernels.s")
    flags = [f for f in build.FLAGS if f not in ("-shared", "-fPIC")]
    subprocess.run([build.HIPCC, *flags, "--cuda-device-only", "-S",
                    os.path.join(build.CSRC, "kernels.hip"), "-o", out],
                   check=True, capture_output=True, text=True)
    with open(out) as f:
        return f.read()


def _body(asm, symbol):
    start = asm.index(f"\n{symbol}:")
    end = asm.index(f".Lfunc_end", start)
    return asm[start:end]


def _m0_problems(body):
    """What breaks the M0 rule in one kernel's assembly: M0-setting asm
    blocks that are not 's_mov_b32 m0' followed by the direct load, and
    compiler-generated lines that name M0."""
    blocks = re.findall(r";;#ASMSTART\n(.*?);;#ASMEND", body, flags=re.S)
    loads = [b for b in blocks if re.search(r"\bm0\b", b)]
    bad = [] if loads else ["no M0-setting inline asm"]
    for b in loads:
        lines = [ln.strip() for ln in b.splitlines() if ln.strip()]
        if not (lines[0].startswith("s_mov_b32 m0,") and
                lines[-1].startswith("global_load_lds_dwordx4")):
            bad.append(lines)
    outside = re.sub(r";;#ASMSTART\n.*?;;#ASMEND", "", body, flags=re.S)
    bad += [ln for ln in outside.splitlines() if re.search(r"\bm0\b", ln.split(";")[0])]
    return bad


def test_m0_check_catches_compiler_use():
    ok = ("k:\n\t;;#ASMSTART\n\ts_mov_b32 m0, s4\n\ts_nop 0\n\tglobal_load_lds_dwordx4 v2, s[6:7]\n"
          "\t;;#ASMEND\n\tv_mfma_f32_32x32x16_bf16 a[0:15], v[0:3], v[4:7], a[0:15]\n")
    assert _m0_problems(ok) == []
    assert _m0_problems(ok + "\ts_mov_b32 m0, -1\n") == ["\ts_mov_b32 m0, -1"]
    assert _m0_problems(ok + "\tds_read_b32 v1, v0 ; uses m0 in a comment\n") == []


def test_gemm_m0_only_in_its_own_asm(asm):
    for name, sym in HOT.items():
        assert _m0_problems(_body(asm, sym)) == [], name


def test_hot_kernels_do_not_spill(asm):
    sizes = dict(re.findall(r"\.name:\s+(\S+)\n(?:.*\n)*?\s+\.private_segment_fixed_size:\s+(\d+)", asm))
    hot = [s for s in sizes if any(k in s for k in ("gemm_gate_up_kernel", "rope_lean_kernel",
                                                   "gelu_and_mul_kernel", "rope_xlane_kernel"))]
    assert len(hot) >= 6, sorted(sizes)
    spilled = {s: sizes[s] for s in hot if sizes[s] != "0"}
    assert not spilled, spilled
