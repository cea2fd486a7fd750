"""Python binding of the C ABI in include/rgg.h (librgg.so, built for gfx950).

Argument marshalling only: every step of the path runs in the library's HIP
kernels.  torch supplies device memory and the current stream; the library
never sees a torch type.  There is no fallback: if librgg.so is missing or a
call returns a nonzero status, these functions raise.

Method: "[sglang] ERNIE-Image의 RoPE와 GELU-mul 융합 및 RoPE cos/sin 호이스팅을
통한 성능 최적화" (blog.secrett2633.cloud, sglang PR 34306 analysis):
  rope_cossin_precompute  -- §1, cos/sin hoisted once per forward
  rope_cossin_from_grid   -- §1, the same tables straight from 3-axis grid
                             positions (a reading of the angle producer)
  rope_rotate_half_bf16   -- §2, bit-exact rotate-half RoPE, tail passthrough
  gelu_and_mul_bf16       -- §3, GEGLU with bf16 activation rounding
  gemm_bf16_nt,           -- §3, the gate_up projection before GEGLU, alone
  gemm_geglu_bf16            or with GEGLU in its epilogue (on the matrix cores)
The page's own Python names are kept as aliases at the bottom.
"""
import ctypes
import math
import os

import torch  # must come first: the HIP runtime torch has loaded is the one librgg binds to

_HERE = os.path.dirname(os.path.abspath(__file__))
LIBRARY = os.path.join(_HERE, "lib", "librgg.so")

__all__ = [
    "rope_cossin_precompute", "rope_cossin_from_grid", "rope_rotate_half_bf16",
    "gelu_and_mul_bf16", "gemm_bf16_nt", "gemm_geglu_bf16", "prepare_device", "selfcheck", "RggError", "library",
    "precompute_rope_cos_sin", "fused_rope_rotate_half_bitexact",
    "gelu_and_mul_with_activation_rounding",
]


class RggError(RuntimeError):
    """A nonzero rgg_status from the library."""

    def __init__(self, func, status, text):
        super().__init__(f"{func}: {text} (status {status})")
        self.status = status


class RopeView(ctypes.Structure):
    """rgg_rope_view."""
    _fields_ = [("x", ctypes.c_void_p), ("out", ctypes.c_void_p),
                ("x_stride_b", ctypes.c_int64), ("x_stride_s", ctypes.c_int64),
                ("x_stride_h", ctypes.c_int64), ("out_stride_b", ctypes.c_int64),
                ("out_stride_s", ctypes.c_int64), ("out_stride_h", ctypes.c_int64)]


_lib = None
_P = ctypes.c_void_p
_I = ctypes.c_int64


def library():
    """The loaded librgg.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIBRARY):
            raise RuntimeError(f"{LIBRARY} is missing: build it with "
                               "`python -m bf16_rope_geglu_amd.build`")
        lib = ctypes.CDLL(LIBRARY)
        lib.rope_cossin_precompute.argtypes = [_P, _I, _I, _I, _I, _I, _P, _P, _P]
        lib.rope_cossin_from_grid.argtypes = [_I, _I, _I, _I, ctypes.c_int32, ctypes.c_int32,
                                              ctypes.c_int32, ctypes.c_double, _P, _P, _P, _P]
        lib.rope_rotate_half_bf16.argtypes = [ctypes.POINTER(RopeView), ctypes.c_int, _I, _I, _I,
                                              _I, _I, _P, _P, _P]
        lib.gelu_and_mul_bf16.argtypes = [_P, _I, _I, _I, _P, _I, _P]
        lib.gemm_bf16_nt.argtypes = [_P, _I, _I, _I, _P, _I, _I, _P, _I, _P]
        lib.gemm_geglu_bf16.argtypes = [_P, _I, _I, _I, _P, _I, _I, _P, _I, _P]
        lib.rgg_prepare_device.argtypes = [ctypes.c_int]
        lib.rgg_selfcheck.argtypes = [_P, _I, _P, ctypes.POINTER(ctypes.c_uint32)]
        lib.rgg_status_string.argtypes = [ctypes.c_int]
        lib.rgg_status_string.restype = ctypes.c_char_p
        for f in (lib.rope_cossin_precompute, lib.rope_cossin_from_grid,
                  lib.rope_rotate_half_bf16, lib.gelu_and_mul_bf16, lib.gemm_bf16_nt,
                  lib.gemm_geglu_bf16, lib.rgg_prepare_device,
                  lib.rgg_selfcheck):
            f.restype = ctypes.c_int
        _lib = lib
    return _lib


def _check(func, status):
    if status != 0:
        raise RggError(func, status, library().rgg_status_string(status).decode())


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need(t, dtype, name):
    if not isinstance(t, torch.Tensor) or t.dtype != dtype or t.device.type != "cuda":
        raise TypeError(f"{name} must be a {dtype} tensor on a HIP device")


def _one_device(dev, **tensors):
    """Every tensor of one call must live on the device the call runs on."""
    for name, t in tensors.items():
        if t is not None and t.device != dev:
            raise ValueError(f"{name} is on {t.device}, the call runs on {dev}")


def rope_cossin_precompute(freqs, cos_out=None, sin_out=None):
    """(S, B, 1, R) fp32 angles -> (cos, sin), each bf16 (B*S, R), row b*S + s.

    `freqs` may be any strided view with unit stride along R.  Output tensors
    are allocated when not given (they must be contiguous (B*S, R) bf16)."""
    _need(freqs, torch.float32, "freqs")
    if freqs.dim() != 4 or freqs.shape[2] != 1:
        raise ValueError("freqs must have shape (S, B, 1, R)")
    S, B, _, R = freqs.shape
    dev = freqs.device
    if cos_out is None:
        cos_out = torch.empty((B * S, R), dtype=torch.bfloat16, device=dev)
    if sin_out is None:
        sin_out = torch.empty((B * S, R), dtype=torch.bfloat16, device=dev)
    for name, t in (("cos_out", cos_out), ("sin_out", sin_out)):
        _need(t, torch.bfloat16, name)
        if tuple(t.shape) != (B * S, R) or not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous ({B * S}, {R})")
    if R > 0 and freqs.numel() > 0 and freqs.stride(3) != 1:
        raise ValueError("freqs needs unit stride along its last dimension")
    _one_device(dev, cos_out=cos_out, sin_out=sin_out)
    with torch.cuda.device(dev):
        _check("rope_cossin_precompute", library().rope_cossin_precompute(
            freqs.data_ptr(), S, B, R, freqs.stride(0), freqs.stride(1),
            cos_out.data_ptr(), sin_out.data_ptr(), _stream(dev)))
    return cos_out, sin_out


def rope_cossin_from_grid(B, grid, dims, theta=10000.0, t_offset=None, cos_out=None,
                          sin_out=None, device=None):
    """cos/sin tables, each bf16 (B*S, R), of a (T, Hg, Wg) token grid's 3-axis
    rotary angles: axis k owns dims[k] columns (half-angles pos_k *
    theta^(-2i/dims[k])), R = sum(dims), rows b*S + s with s = (t*Hg + h)*Wg + w.
    `t_offset`, if given, is an int32 tensor of B shifts of t on the device."""
    T, Hg, Wg = (int(v) for v in grid)
    d0, d1, d2 = (int(v) for v in dims)
    S, R = T * Hg * Wg, d0 + d1 + d2
    for name, t in (("cos_out", cos_out), ("sin_out", sin_out)):
        if t is not None:
            _need(t, torch.bfloat16, name)
    if t_offset is not None:
        _need(t_offset, torch.int32, "t_offset")
    if device is not None:
        dev = torch.device(device)
    elif cos_out is not None:
        dev = cos_out.device
    elif t_offset is not None:
        dev = t_offset.device
    else:
        dev = torch.device("cuda", torch.cuda.current_device())
    if cos_out is None:
        cos_out = torch.empty((B * S, R), dtype=torch.bfloat16, device=dev)
    if sin_out is None:
        sin_out = torch.empty((B * S, R), dtype=torch.bfloat16, device=dev)
    for name, t in (("cos_out", cos_out), ("sin_out", sin_out)):
        _need(t, torch.bfloat16, name)
        if tuple(t.shape) != (B * S, R) or not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous ({B * S}, {R})")
    _one_device(dev, cos_out=cos_out, sin_out=sin_out, t_offset=t_offset)
    off = None
    if t_offset is not None:
        if tuple(t_offset.shape) != (B,) or not t_offset.is_contiguous():
            raise ValueError(f"t_offset must be a contiguous ({B},) int32 tensor")
        off = t_offset.data_ptr()
    with torch.cuda.device(cos_out.device):
        _check("rope_cossin_from_grid", library().rope_cossin_from_grid(
            B, T, Hg, Wg, d0, d1, d2, float(theta), off, cos_out.data_ptr(), sin_out.data_ptr(),
            _stream(cos_out.device)))
    return cos_out, sin_out


def rope_rotate_half_bf16(x, cos, sin, out=None):
    """Rotate-half RoPE over the leading R = cos.shape[-1] columns.

    `x` is one (B, S, H, D) bf16 tensor or a list of up to four sharing one
    shape (e.g. q and k, possibly strided views of a fused QKV output); each
    needs unit stride along D.  cos/sin are contiguous (B*S, R) bf16.  `out`
    (same structure) may be given, including out is x for in place; else
    contiguous outputs are allocated.  Returns out in x's structure."""
    single = isinstance(x, torch.Tensor)
    xs = [x] if single else list(x)
    if out is None:
        outs = [torch.empty(t.shape, dtype=torch.bfloat16, device=t.device) for t in xs]
    else:
        outs = [out] if isinstance(out, torch.Tensor) else list(out)
    if not 1 <= len(xs) <= 4 or len(outs) != len(xs):
        raise ValueError("one to four x tensors, and as many outputs")
    _need(cos, torch.bfloat16, "cos")
    _need(sin, torch.bfloat16, "sin")
    shape = tuple(xs[0].shape)
    if len(shape) != 4:
        raise ValueError("x must be (B, S, H, D)")
    B, S, H, D = shape
    R = cos.shape[-1]
    if cos.dim() != 2 or tuple(cos.shape) != (B * S, R) or tuple(sin.shape) != (B * S, R) \
            or not cos.is_contiguous() or not sin.is_contiguous():
        raise ValueError(f"cos and sin must be contiguous ({B * S}, R)")
    views = (RopeView * len(xs))()
    for v, (xv, ov) in enumerate(zip(xs, outs)):
        _need(xv, torch.bfloat16, "x")
        _need(ov, torch.bfloat16, "out")
        if tuple(xv.shape) != shape or tuple(ov.shape) != shape:
            raise ValueError("all x and out tensors must share one (B, S, H, D) shape")
        if xv.numel() and (xv.stride(3) != 1 or ov.stride(3) != 1):
            raise ValueError("x and out need unit stride along D")
        views[v] = RopeView(xv.data_ptr(), ov.data_ptr(), xv.stride(0), xv.stride(1),
                            xv.stride(2), ov.stride(0), ov.stride(1), ov.stride(2))
    dev = xs[0].device
    _one_device(dev, cos=cos, sin=sin, **{f"x[{v}]": t for v, t in enumerate(xs)},
                **{f"out[{v}]": t for v, t in enumerate(outs)})
    with torch.cuda.device(dev):
        _check("rope_rotate_half_bf16", library().rope_rotate_half_bf16(
            views, len(xs), B, S, H, D, R, cos.data_ptr(), sin.data_ptr(), _stream(dev)))
    return outs[0] if single else outs


def gelu_and_mul_bf16(input, out=None):
    """GEGLU: input (..., 2*hidden) bf16, gate = first half, up = second half;
    returns rne_bf16(up * rne_bf16(gelu(gate))) of shape (..., hidden).

    The leading dimensions must collapse to rows with one row stride.  `out`
    may be given (shape (..., hidden)), including the in-place form
    out = input[..., :hidden] (same row stride)."""
    _need(input, torch.bfloat16, "input")
    if input.dim() < 1 or input.shape[-1] % 2:
        raise ValueError("input's last dimension must be even (gate | up)")
    hidden = input.shape[-1] // 2
    lead = tuple(input.shape[:-1])
    if out is None:
        out = torch.empty(lead + (hidden,), dtype=torch.bfloat16, device=input.device)
    _need(out, torch.bfloat16, "out")
    if tuple(out.shape) != lead + (hidden,):
        raise ValueError("out must have shape (..., hidden)")
    inp2 = input.reshape(-1, 2 * hidden) if input.numel() else input.new_empty(0, 2 * hidden)
    out2 = out.view(-1, hidden) if out.numel() else out.new_empty(0, hidden)
    if inp2.numel() and (inp2.data_ptr() != input.data_ptr() or inp2.stride(1) != 1):
        raise ValueError("input's leading dimensions must collapse into rows without a copy")
    if out2.numel() and out2.stride(1) != 1:
        raise ValueError("out needs unit stride along its last dimension")
    rows = inp2.shape[0]
    dev = input.device
    _one_device(dev, out=out)
    with torch.cuda.device(dev):
        _check("gelu_and_mul_bf16", library().gelu_and_mul_bf16(
            inp2.data_ptr(), rows, hidden, inp2.stride(0) if rows else 2 * hidden,
            out2.data_ptr(), out2.stride(0) if rows else hidden, _stream(dev)))
    return out


def _projection(name, x, weight, out_cols, out):
    """Shared marshalling of gemm_bf16_nt / gemm_geglu_bf16: x (..., K) rows,
    weight (N, K); returns out (..., out_cols).  The size argument of the C
    call is out_cols for both (N for the plain product, hidden for GEGLU)."""
    _need(x, torch.bfloat16, "x")
    _need(weight, torch.bfloat16, "weight")
    if x.dim() < 1 or weight.dim() != 2 or weight.shape[1] != x.shape[-1]:
        raise ValueError("x must be (..., K) and weight (N, K)")
    K = x.shape[-1]
    lead = tuple(x.shape[:-1])
    if out is None:
        out = torch.empty(lead + (out_cols,), dtype=torch.bfloat16, device=x.device)
    _need(out, torch.bfloat16, "out")
    if tuple(out.shape) != lead + (out_cols,):
        raise ValueError(f"out must have shape (..., {out_cols})")
    M = math.prod(lead)
    xp, xs = 0, K
    if M and K:
        x2 = x.reshape(M, K)
        if x2.data_ptr() != x.data_ptr() or x2.stride(1) != 1:
            raise ValueError("x's leading dimensions must collapse into rows without a copy")
        xp, xs = x2.data_ptr(), (x2.stride(0) if M > 1 else K)
    if weight.numel() and weight.stride(1) != 1:
        raise ValueError("weight needs unit stride along K")
    op, os_ = 0, out_cols
    if M and out_cols:
        out2 = out.view(M, out_cols)
        if out2.stride(1) != 1:
            raise ValueError("out needs unit stride along its last dimension")
        op, os_ = out2.data_ptr(), (out2.stride(0) if M > 1 else out_cols)
    dev = x.device
    _one_device(dev, weight=weight, out=out)
    with torch.cuda.device(dev):
        _check(name, getattr(library(), name)(
            xp, M, K, xs, weight.data_ptr() if weight.numel() else 0, out_cols,
            weight.stride(0) if weight.shape[0] > 1 and K else K, op, os_, _stream(dev)))
    return out


def gemm_bf16_nt(x, weight, out=None):
    """The gate_up projection: x (..., K) bf16 times weight (N, K) bf16
    transposed (a linear layer without bias), fp32 accumulation, each output
    rounded once to bf16; returns (..., N).  K a multiple of 64, N of 128."""
    if not isinstance(weight, torch.Tensor) or weight.dim() != 2:
        raise ValueError("weight must be (N, K)")
    return _projection("gemm_bf16_nt", x, weight, weight.shape[0], out)


def gemm_geglu_bf16(x, weight, out=None):
    """GEGLU fused into the gate_up projection: weight (2*hidden, K) holds the
    gate rows then the up rows; returns rne_bf16(up * rne_bf16(gelu(gate))) of
    shape (..., hidden), bit for bit gelu_and_mul_bf16(gemm_bf16_nt(x, weight))
    without the (..., 2*hidden) projection in memory."""
    if not isinstance(weight, torch.Tensor) or weight.dim() != 2 or weight.shape[0] % 2:
        raise ValueError("weight must be (2*hidden, K)")
    return _projection("gemm_geglu_bf16", x, weight, weight.shape[0] // 2, out)


def prepare_device(device=None):
    """Build the constant GELU table on `device` now (before graph capture)."""
    idx = torch.cuda.current_device() if device is None else torch.device(device).index
    _check("rgg_prepare_device", library().rgg_prepare_device(idx))


SELFCHECK_WORKSPACE_BYTES = 1 << 20
_SELFCHECK_FAILED = 8


def selfcheck(device=None):
    """Run the device self-check on `device` (default: current) on the current
    stream; returns the mask of failed checks (0 when every result has its
    expected bits).  Raises RggError for any other error."""
    dev = torch.device("cuda", torch.cuda.current_device() if device is None
                       else torch.device(device).index)
    ws = torch.empty(SELFCHECK_WORKSPACE_BYTES, dtype=torch.uint8, device=dev)
    failed = ctypes.c_uint32(0)
    with torch.cuda.device(dev):
        status = library().rgg_selfcheck(ws.data_ptr(), ws.numel(), _stream(dev),
                                         ctypes.byref(failed))
    if status not in (0, _SELFCHECK_FAILED):
        _check("rgg_selfcheck", status)
    return failed.value


# The page's own names ---------------------------------------------------------

def precompute_rope_cos_sin(freqs):
    """Alias of rope_cossin_precompute for (S, B, 1, R) fp32 angles."""
    return rope_cossin_precompute(freqs)


def fused_rope_rotate_half_bitexact(x, cos, sin):
    """Alias of rope_rotate_half_bf16 for one (B, S, H, D) tensor, out of place."""
    return rope_rotate_half_bf16(x, cos, sin)


def gelu_and_mul_with_activation_rounding(input, out=None):
    """Alias of gelu_and_mul_bf16."""
    return gelu_and_mul_bf16(input, out)
