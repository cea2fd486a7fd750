"""rgg_selfcheck_noalloc against rgg_selfcheck, through the C ABI.

The allocation-free self-check stages its inputs in a device array the
library holds for each GPU, instead of a caller workspace.  Its results (the
status and the mask of failed checks) must equal those of rgg_selfcheck with
a caller workspace, restricted to the selected checks: on two calls in a row,
the second selecting fewer checks (a smaller staged input) after the first
has left its contents in the array.  The checks themselves compare the
library's outputs with hand-derived expected bits (rgg_selfcheck).
"""
import ctypes

import pytest
import torch

import bf16_rope_geglu_amd as rgg

pytestmark = pytest.mark.gpu

ALL = 0x7F


def _lib():
    lib = rgg.library()
    lib.rgg_selfcheck_noalloc.restype = ctypes.c_int
    lib.rgg_selfcheck_noalloc.argtypes = [ctypes.c_uint32, ctypes.c_void_p,
                                          ctypes.POINTER(ctypes.c_uint32)]
    return lib


def _with_workspace(lib):
    ws = torch.empty(1 << 20, dtype=torch.uint8, device="cuda")
    failed = ctypes.c_uint32(0xFFFFFFFF)
    st = lib.rgg_selfcheck(ws.data_ptr(), ws.numel(), torch.cuda.current_stream().cuda_stream,
                           ctypes.byref(failed))
    torch.cuda.synchronize()
    return st, failed.value


def _noalloc(lib, checks):
    failed = ctypes.c_uint32(0xFFFFFFFF)
    st = lib.rgg_selfcheck_noalloc(checks, torch.cuda.current_stream().cuda_stream,
                                   ctypes.byref(failed))
    torch.cuda.synchronize()
    return st, failed.value


def test_noalloc_selfcheck_matches_workspace_form():
    lib = _lib()
    st_ref, mask_ref = _with_workspace(lib)
    print(f"rgg_selfcheck: status {st_ref}, failed mask {mask_ref:#x}", flush=True)
    for checks in (ALL, 0x03):   # every check, then the two smallest (tables, worked vectors)
        st, mask = _noalloc(lib, checks)
        print(f"rgg_selfcheck_noalloc({checks:#x}): status {st}, failed mask {mask:#x}", flush=True)
        want_mask = mask_ref & checks
        assert mask == want_mask, f"checks {checks:#x}: mask {mask:#x}, workspace form {want_mask:#x}"
        assert st == (8 if want_mask else 0), f"checks {checks:#x}: status {st}"
    assert st_ref == 0 and mask_ref == 0, "the device self-check itself fails"


def test_noalloc_selfcheck_rejects_bad_masks():
    lib = _lib()
    stream = torch.cuda.current_stream().cuda_stream
    failed = ctypes.c_uint32(0)
    assert lib.rgg_selfcheck_noalloc(0, stream, ctypes.byref(failed)) == 2
    assert lib.rgg_selfcheck_noalloc(0x80, stream, ctypes.byref(failed)) == 2
