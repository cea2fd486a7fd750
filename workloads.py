"""Seeded synthetic workloads for the fused RoPE + GEGLU path.

This module only draws inputs and describes shapes; it holds none of the
method's arithmetic.  Both sides of every parity check (the CPU oracle and the
HIP library) receive the same bits from here.

Shapes follow the DiT activations of the ERNIE-Image fusion page (sglang PR
34306 analysis): x (B, S, H, D) q/k projections, rotary angles (S, B, 1, R),
and a concatenated gate/up FFN projection (tokens, 2*hidden).  The page gives
no resolution, so the five workloads below are synthetic stand-ins:

  tiny      x (1,256,4,64), R=64, 1-D positions 0..255; GEGLU 256 x 256
  rope_qk   q and k (1,4096,32,128), R=128, 3-axis grid (1,64,64), axis dims 32/48/48
  partial   x (2,4096,24,128), R=96 (32-column tail), 3-axis grid (1,64,64), dims 24/36/36
  geglu     gate/up 8192 x 12288, gate sigma 3, up sigma 1
  dit_layer fused qkv (4,8192,3*32*128); q/k strided views, R=128, grid (2,64,64),
            dims 32/48/48; GEGLU 32768 x 8192; the gate_up projection that feeds
            it: x (32768, 4096) (model width H*D), weight (2*8192, 4096)

Angles: for a 3-axis grid (T, Hg, Wg) token s = (t*Hg + h)*Wg + w, axis k of
dimension d_k contributes d_k/2 half-angles pos_k * theta^(-2i/d_k); the R/2
half-angles are concatenated over the axes and then repeated, freqs =
cat(f, f), the layout a rotate-half RoPE pairs column j with j + R/2 in.
Angles are computed in float64 and rounded once to float32.

Random tensors: numpy PCG64 seeded with 1000*workload + tensor id (x/q 1,
k 2, gate 3, up 4, qkv 5, extra 6, weight 7), float32 N(0, sigma^2), converted
to bf16 by torch's round-to-nearest-even cast; projection weights have sigma
1/sqrt(K), so gates come out near N(0, 1).  Exact-sum inputs for the
projection are small integers times a power of two (`small_int_bf16`): every
partial sum of their products is a float32 integer multiple of that power, so
any summation order gives the exact sum.  For full-size GPU runs the same
recipe is drawn on the device by torch's generator (`device_normal_bf16`).
"""
import numpy as np

THETA = 1.0e4

WORKLOADS = {
    0: dict(name="tiny",
            rope=dict(B=1, S=256, H=4, D=64, R=64, views=1, layout="separate",
                      freqs=dict(kind="1d")),
            geglu=dict(rows=256, hidden=256, gate_sigma=1.0)),
    1: dict(name="rope_qk",
            rope=dict(B=1, S=4096, H=32, D=128, R=128, views=2, layout="separate",
                      freqs=dict(kind="3axis", grid=(1, 64, 64), dims=(32, 48, 48)))),
    2: dict(name="partial",
            rope=dict(B=2, S=4096, H=24, D=128, R=96, views=1, layout="separate",
                      freqs=dict(kind="3axis", grid=(1, 64, 64), dims=(24, 36, 36)))),
    3: dict(name="geglu",
            geglu=dict(rows=8192, hidden=12288, gate_sigma=3.0)),
    4: dict(name="dit_layer",
            rope=dict(B=4, S=8192, H=32, D=128, R=128, views=2, layout="qkv",
                      freqs=dict(kind="3axis", grid=(2, 64, 64), dims=(32, 48, 48))),
            geglu=dict(rows=32768, hidden=8192, gate_sigma=1.0),
            proj=dict(rows=32768, dim=4096, hidden=8192)),
}

TENSOR_ID = dict(x=1, q=1, k=2, gate=3, up=4, qkv=5, extra=6, weight=7)


def seed_for(workload, tensor):
    return 1000 * int(workload) + TENSOR_ID[tensor]


# ---------------------------------------------------------------------------
# bf16 bit patterns
# ---------------------------------------------------------------------------

def f32_to_bf16_bits(a):
    """torch's float32 -> bfloat16 cast (round to nearest even), as uint16 bits."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def bf16_bits_to_f32(b):
    """Exact widening of bf16 bit patterns to float32."""
    b = np.asarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def normal_bf16(shape, seed, sigma=1.0):
    """N(0, sigma^2) drawn in float32 by PCG64(seed), cast to bf16 bits."""
    rng = np.random.Generator(np.random.PCG64(seed))
    a = rng.standard_normal(size=shape, dtype=np.float32)
    if sigma != 1.0:
        a = a * np.float32(sigma)
    return f32_to_bf16_bits(a)


def special_bf16(shape, seed):
    """Finite bf16 bit patterns rich in edge cases.

    Mix: N(0,1) values, signed zeros, subnormals, the smallest normals,
    powers of two, values near the largest finite, and values whose products
    with short-mantissa cos/sin entries land on exact rounding ties.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    n = int(np.prod(shape))
    kind = rng.integers(0, 8, size=n)
    normal = normal_bf16((n,), seed + 7919)
    sign = (rng.integers(0, 2, size=n).astype(np.uint16) << 15)
    mant = rng.integers(0, 128, size=n).astype(np.uint16)
    out = normal.copy()
    out[kind == 1] = sign[kind == 1]                                     # +-0
    sub = mant.copy()
    sub[sub == 0] = 1
    out[kind == 2] = sign[kind == 2] | sub[kind == 2]                    # subnormals
    out[kind == 3] = sign[kind == 3] | (0x0080 + mant[kind == 3])        # smallest normals
    exp = rng.integers(1, 255, size=n).astype(np.uint16)
    out[kind == 4] = sign[kind == 4] | (exp[kind == 4] << 7)             # powers of two
    out[kind == 5] = sign[kind == 5] | (0x7F00 + mant[kind == 5])        # near max finite
    short = (rng.integers(120, 134, size=n).astype(np.uint16) << 7) | \
        (rng.integers(0, 8, size=n).astype(np.uint16) << 4)
    out[kind == 6] = sign[kind == 6] | short[kind == 6]                  # few mantissa bits
    near_one = (0x3F00 + rng.integers(0, 256, size=n)).astype(np.uint16) & 0x7FFF
    out[kind == 7] = sign[kind == 7] | near_one[kind == 7]               # around 1.0
    return out.reshape(shape)


def device_normal_bf16(shape, seed, sigma=1.0, device="cuda"):
    """Full-size draw on the device: torch generator seeded with `seed`, float32
    N(0, sigma^2) cast to bf16 (torch tensor)."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    t = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if sigma != 1.0:
        t.mul_(sigma)
    return t.to(torch.bfloat16)


def small_int_bf16(shape, seed, bound=7, exp=-4):
    """Integers uniform in [-bound, bound] times 2^exp, as bf16 bits (exact)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    a = rng.integers(-bound, bound + 1, size=shape).astype(np.float32) * np.float32(2.0 ** exp)
    return f32_to_bf16_bits(a)


def device_small_int_bf16(shape, seed, bound=7, exp=-4, device="cuda"):
    """small_int_bf16's recipe drawn on the device by torch's generator."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    t = torch.randint(-bound, bound + 1, shape, generator=g, device=device, dtype=torch.int32)
    return (t.to(torch.float32) * (2.0 ** exp)).to(torch.bfloat16)


# ---------------------------------------------------------------------------
# rotary angles (S, B, 1, R) float32
# ---------------------------------------------------------------------------

def freqs_1d(S, B, R, theta=THETA):
    """pos * theta^(-2i/R) for pos = 0..S-1, i < R/2, laid out as cat(f, f)."""
    half = R // 2
    i = np.arange(half, dtype=np.float64)
    omega = theta ** (-2.0 * i / R)
    f = np.arange(S, dtype=np.float64)[:, None] * omega[None, :]
    full = np.concatenate([f, f], axis=1).astype(np.float32)           # (S, R)
    return np.ascontiguousarray(np.broadcast_to(full[:, None, None, :], (S, B, 1, R)))


def grid_positions(grid):
    """(t, h, w) of token s = (t*Hg + h)*Wg + w for a (T, Hg, Wg) grid."""
    T, Hg, Wg = grid
    t, h, w = np.meshgrid(np.arange(T), np.arange(Hg), np.arange(Wg), indexing="ij")
    return np.stack([t.ravel(), h.ravel(), w.ravel()], axis=1).astype(np.float64)


def freqs_3axis(grid, dims, B, theta=THETA, batch_offsets=None):
    """3-axis angles, cat(f, f) layout, replicated over B.

    `batch_offsets`, if given, is a length-B array added to the t position of
    batch row b, so that different batch rows get different angles.
    """
    pos = grid_positions(grid)                                         # (S, 3)
    S = pos.shape[0]
    R = sum(dims)
    out = np.empty((S, B, 1, R), np.float32)
    for b in range(B):
        p = pos.copy()
        if batch_offsets is not None:
            p[:, 0] += float(batch_offsets[b])
        parts = []
        for k, d in enumerate(dims):
            i = np.arange(d // 2, dtype=np.float64)
            omega = theta ** (-2.0 * i / d)
            parts.append(p[:, k:k + 1] * omega[None, :])
        f = np.concatenate(parts, axis=1)
        out[:, b, 0, :] = np.concatenate([f, f], axis=1).astype(np.float32)
    return out


def freqs_unpaired(S, B, R, seed):
    """Angles whose two halves differ (cos[j] != cos[j + R/2]); distinct per b."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return rng.uniform(-300.0, 300.0, size=(S, B, 1, R)).astype(np.float32)


def workload_freqs(wid):
    r = WORKLOADS[wid]["rope"]
    fk = r["freqs"]
    if fk["kind"] == "1d":
        return freqs_1d(r["S"], r["B"], r["R"])
    return freqs_3axis(fk["grid"], fk["dims"], r["B"])


def algo_bytes(wid):
    """Algorithmic bytes per stage: every input read once, every output written once."""
    w = WORKLOADS[wid]
    out = {}
    if "rope" in w:
        r = w["rope"]
        T = r["B"] * r["S"]
        out["precompute"] = T * r["R"] * 4 + 2 * T * r["R"] * 2
        out["precompute_grid"] = 2 * T * r["R"] * 2
        x = r["views"] * T * r["H"] * r["D"] * 2
        out["rope"] = 2 * x + 2 * T * r["R"] * 2
    if "geglu" in w:
        g = w["geglu"]
        out["geglu"] = g["rows"] * g["hidden"] * 2 * 3
    return out
