"""Throughput of the fused RoPE + GEGLU path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload dit_layer]

One step = one pass of the whole path over one batch of synthetic input:
  1. rope_cossin_precompute  angles (S, B, 1, R) fp32 -> cos/sin (B*S, R) bf16
  2. rope_rotate_half_bf16   q and k, strided views of the fused QKV projection
                             output (B, S, 3*H*D), one launch -> contiguous q/k
  3. gelu_and_mul_bf16       (tokens, 2*hidden) -> (tokens, hidden)
on the dit_layer workload (B=4, S=8192, H=32, D=128, R=128; GEGLU 32768 x
8192), inputs drawn on the device before timing.  W untimed steps, then K
steps between two device synchronisations; value = algorithmic bytes of a
step / mean step time (GB/s, 1e9 bytes).  Every kernel is also bracketed by
HIP events on the stream it runs on, which gives each one's mean launch
duration and its algorithmic GB/s; `roofline` reports the dominant kernel.

`projection` times the gate_up projection of the same layer on the matrix
cores, x (32768, 4096) times W (2 x 8192, 4096): GEGLU fused into its
epilogue, the plain projection, the unfused pair, and the platform library
GEMM followed by gelu_and_mul_bf16 for comparison (TFLOP/s against the
2.5 PFLOP/s dense bf16 peak).  It is outside the step and its `value`.

`configs` holds every graded kernel on every workload that has it (RoPE on
rope_qk, partial and dit_layer; GEGLU on geglu and dit_layer), timed with
cold caches (a HIP graph of launches over rotating buffer sets touching at
least 2 GiB), each beside the fastest member of a family of plain streaming
kernels moving the same bytes (STREAM_FAMILY, timed the same way on the same
box) and its fraction of that ceiling (`vs_ceiling`).

`cpu_baseline` times the CPU oracle on a bounded sample of the same
workload (16384 tokens, 8192 GEGLU rows): `value` on one thread, and
`all_cores` with the sample split over every core the process may use;
`cpu` names the host CPU model.  `roofline.traffic` comes from the committed rocprofv3
counter summary for the dominant kernel, and is null if the code of the
step's kernels (comments and the projection kernel aside) has changed since
the counters were taken.

    python bench.py --pmc-summary DIR --pmc-out FILE
turns rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE outputs (DIR/fetch, DIR/write)
into that summary; --calibration-copy adds a plain device copy of known size
to each step so the same runs calibrate the counters.

    python bench.py --traffic-run rope_qk|partial
runs only the RoPE kernel on that workload (and the calibration copy), for
the same two counter passes; --pmc-set rope_qk|partial summarises them.

    python bench.py --projection [--calibration-copy]
times only the gate_up projection entry points (and adds the calibration
copy); --pmc-set projection summarises counters of such runs.

    python bench.py --counter-summary DIR --counter-out FILE
summarises any other rocprofv3 --pmc passes over `--projection` runs (one
subfolder per pass): the median per dispatch of each counter for the
projection kernels and the platform GEMM.

    python bench.py --sweep
prints a markdown table of every kernel on every workload with cold caches
(replayed from one HIP graph), each beside the streaming reference
(bf16_rope_geglu_amd/lib/libstreamref.so) moving the same bytes with the
same read:write ratio (write-only for the tables built from grid
positions): the practical ceiling for that traffic.

    python bench.py --stream-sweep [--stream-sweep-out FILE]
times the whole streaming family (workgroup size, vectors per lane, one pass
or persistent grids, load and store cache policies, residency caps) at each
graded size and writes the ranking as markdown.
"""
import argparse
import csv
import glob
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "fused RoPE + GEGLU effective HBM GB/s and % of MI355X peak (bf16)"
PEAK_HBM_GBPS = 8000.0
KERNELS_SRC = os.path.join(ROOT, "bf16_rope_geglu_amd", "csrc", "kernels.hip")
LAUNCH_H = os.path.join(ROOT, "bf16_rope_geglu_amd", "csrc", "launch.h")
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "gelu_and_mul_dit_layer_traffic.md")
KERNEL_SYMBOL = {
    "precompute": "rope_cossin_kernel",
    "rope": "rope_lean_kernel",
    "geglu": "gelu_and_mul_kernel",
}
COPY_BYTES = 1 << 30


def source_digest():
    """Hash of the code of the kernels the step runs: kernels.hip and
    launch.h (parameter blocks, launch thresholds), with comments and
    whitespace dropped, and without the projection kernel (its constants,
    kernel and launcher), which the step never launches.  The counters of
    the step's kernels stay current across those edits and go stale with any
    other change to the code of either file (helpers shared with the
    projection included)."""
    with open(KERNELS_SRC) as f:
        text = f.read()
    a = text.index("typedef __bf16 bf16x8")
    b = text.index("#undef RGG_FENCE")
    text = text[:a] + text[b:]
    c = text.index("hipError_t launch_gemm_gate_up(")
    d = text.index("\n}\n", c)
    text = text[:c] + text[d + 3:]
    with open(LAUNCH_H) as f:
        text += "\n" + f.read()
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    text = " ".join(text.split())
    return hashlib.sha256(text.encode()).hexdigest()[:16]


# ---------------------------------------------------------------------------
# GPU benchmark
# ---------------------------------------------------------------------------

def step_algo_bytes(wid):
    """Algorithmic bytes of one step: the three kernels the step launches."""
    import workloads as W

    algo = W.algo_bytes(wid)
    return algo["precompute"] + algo["rope"] + algo["geglu"]


def run_gpu(args):
    import torch

    import bf16_rope_geglu_amd as rgg
    import workloads as W

    wid = {w["name"]: k for k, w in W.WORKLOADS.items()}[args.workload]
    wl = W.WORKLOADS[wid]
    r, g = wl["rope"], wl["geglu"]
    B, S, H, D, R = r["B"], r["S"], r["H"], r["D"], r["R"]
    rows, hidden = g["rows"], g["hidden"]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    freqs = torch.from_numpy(W.workload_freqs(wid)).to(dev)
    qkv = W.device_normal_bf16((B, S, 3 * H * D), W.seed_for(wid, "qkv"), device=dev)
    q = qkv[..., :H * D].view(B, S, H, D)
    k = qkv[..., H * D:2 * H * D].view(B, S, H, D)
    cos = torch.empty((B * S, R), dtype=torch.bfloat16, device=dev)
    sin = torch.empty_like(cos)
    q_out = torch.empty((B, S, H, D), dtype=torch.bfloat16, device=dev)
    k_out = torch.empty_like(q_out)
    gate = W.device_normal_bf16((rows, hidden), W.seed_for(wid, "gate"), g["gate_sigma"], dev)
    up = W.device_normal_bf16((rows, hidden), W.seed_for(wid, "up"), device=dev)
    gate_up = torch.cat([gate, up], dim=1)
    del gate, up
    geglu_out = torch.empty((rows, hidden), dtype=torch.bfloat16, device=dev)
    if args.calibration_copy:
        copy_src = torch.ones(COPY_BYTES // 2, dtype=torch.bfloat16, device=dev)
        copy_dst = torch.empty_like(copy_src)
    rgg.prepare_device(0)
    torch.cuda.synchronize()

    algo = W.algo_bytes(wid)
    names = ["precompute", "rope", "geglu"]
    step_bytes = step_algo_bytes(wid)

    def step(events=None):
        if events:
            events[0].record()
        rgg.rope_cossin_precompute(freqs, cos, sin)
        if events:
            events[1].record()
        rgg.rope_rotate_half_bf16([q, k], cos, sin, out=[q_out, k_out])
        if events:
            events[2].record()
        rgg.gelu_and_mul_bf16(gate_up, geglu_out)
        if events:
            events[3].record()
        if args.calibration_copy:
            copy_dst.copy_(copy_src)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # whole-step throughput: K back-to-back steps, no per-kernel events
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record()
    for _ in range(args.steps):
        step()
    stop.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = start.elapsed_time(stop) / args.steps

    # per-kernel launch durations: HIP events on the launch stream around each kernel
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    for e in evs:
        step(e)
    torch.cuda.synchronize()
    per = {n: 0.0 for n in names}
    for e in evs:
        for i, n in enumerate(names):
            per[n] += e[i].elapsed_time(e[i + 1]) / args.steps
    kernels = {}
    for n in names:
        us = per[n] * 1e3
        gbps = algo[n] / (us * 1e-6) / 1e9
        kernels[n] = {"symbol": KERNEL_SYMBOL[n], "us": round(us, 2), "algo_bytes": algo[n],
                      "GBps": round(gbps, 1), "frac": round(gbps / PEAK_HBM_GBPS, 4)}
    dominant = max(names, key=lambda n: per[n])
    return {
        "wid": wid, "ms_per_step": ms_per_step, "wall_s": wall, "step_bytes": step_bytes,
        "kernels": kernels, "dominant": dominant, "shape": (B, S, H, D, R, rows, hidden),
    }


# ---------------------------------------------------------------------------
# the gate_up projection with GEGLU in its epilogue (matrix cores)
# ---------------------------------------------------------------------------

PEAK_BF16_TFLOPS = 2500.0


def run_projection(reps=10, warmup=2):
    """The dit_layer projection, x (32768, 4096) times W (2 x 8192, 4096):
    gemm_geglu_bf16 (fused), gemm_bf16_nt alone, gemm_bf16_nt followed by
    gelu_and_mul_bf16 (the unfused path), and torch.matmul (the platform's
    library GEMM) followed by gelu_and_mul_bf16, for comparison.  Every case
    runs `warmup` times first (so the first one timed does not pay for the
    clock ramp after an idle GPU); then two rounds time each case as the mean
    of `reps` launches between HIP events on the launch stream, and the
    faster round is reported.  TFLOP/s counts 2 M K (2 H) multiply-adds."""
    import torch

    import bf16_rope_geglu_amd as rgg
    import workloads as W

    pr = W.WORKLOADS[4]["proj"]
    M, K, H = pr["rows"], pr["dim"], pr["hidden"]
    dev = torch.device("cuda:0")
    x = W.device_normal_bf16((M, K), W.seed_for(4, "x"), device=dev)
    w = W.device_normal_bf16((2 * H, K), W.seed_for(4, "weight"), 1.0 / K ** 0.5, dev)
    out = torch.empty((M, H), dtype=torch.bfloat16, device=dev)
    proj = torch.empty((M, 2 * H), dtype=torch.bfloat16, device=dev)
    rgg.prepare_device(0)
    flops = 2.0 * M * K * 2 * H
    cases = [
        ("gemm_geglu_bf16", lambda: rgg.gemm_geglu_bf16(x, w, out)),
        ("gemm_bf16_nt", lambda: rgg.gemm_bf16_nt(x, w, proj)),
        ("gemm_bf16_nt + gelu_and_mul_bf16",
         lambda: (rgg.gemm_bf16_nt(x, w, proj), rgg.gelu_and_mul_bf16(proj, out))),
        ("torch.matmul + gelu_and_mul_bf16 (comparison)",
         lambda: (torch.matmul(x, w.t(), out=proj), rgg.gelu_and_mul_bf16(proj, out))),
    ]
    for _ in range(warmup):
        for _, fn in cases:
            fn()
    torch.cuda.synchronize()
    best = {}
    for _ in range(2):
        for name, fn in cases:
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record()
            for _ in range(reps):
                fn()
            b.record()
            torch.cuda.synchronize()
            us = a.elapsed_time(b) * 1e3 / reps
            best[name] = min(best.get(name, us), us)
    res = {}
    for name, _ in cases:
        us = best[name]
        tf = flops / (us * 1e-6) / 1e12
        res[name] = {"us": round(us, 1), "TFLOPs": round(tf, 1),
                     "frac": round(tf / PEAK_BF16_TFLOPS, 4)}
    del x, w, out, proj
    torch.cuda.empty_cache()
    return {"shape": {"M": M, "K": K, "hidden": H}, "flops": flops,
            "intermediate_bytes_avoided": 2 * M * 2 * H * 2, "peak_TFLOPs": PEAK_BF16_TFLOPS,
            "results": res}


# ---------------------------------------------------------------------------
# per-kernel sweep over every workload, cold caches
# ---------------------------------------------------------------------------

def stream_ref_library():
    """ctypes handle of bf16_rope_geglu_amd/lib/libstreamref.so (built by
    __graft_entry__.build()), the streaming references timed as ceilings."""
    import ctypes

    import torch  # noqa: F401  (loads the HIP runtime the library links)

    path = os.path.join(ROOT, "bf16_rope_geglu_amd", "lib", "libstreamref.so")
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: run __graft_entry__.build()")
    lib = ctypes.CDLL(path)
    lib.rgg_stream_ref.restype = ctypes.c_int
    lib.rgg_stream_ref.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                   ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                   ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    return lib


COLD_REPS = 40
COLD_TOUCH = 2 << 30

# Members of the streaming-reference family timed as the ceiling for a
# kernel's traffic: (workgroup size, 16-byte vectors per lane, grid (0: one
# pass, else that many persistent workgroups), cache policy (1: nontemporal
# loads; +2 nontemporal stores; +4 write-through stores), LDS bytes per
# workgroup (caps residency; 0: none)).  These are the fastest members at
# each workload size in a sweep of the whole family (block 256/512/1024,
# 1/2/4/8 vectors per lane, one pass or 256..2048 persistent workgroups,
# every policy, residency caps of 3..6 workgroups per compute unit,
# `profiles/stream_family_sweep.md`); the ceiling reported is the best of
# them on the box at hand.
STREAM_FAMILY = [(256, 1, 0, 7, 0), (256, 1, 0, 5, 0), (256, 1, 0, 3, 0), (256, 2, 0, 3, 0),
                 (512, 1, 0, 7, 0), (256, 1, 1024, 7, 0), (256, 1, 0, 7, 27136)]


def cold_us(fns, reps=COLD_REPS):
    """Per-launch time of `fns` (launchers over disjoint buffer sets) replayed
    round robin from one HIP graph of `reps` launches between two events:
    the sets together touch far more than the 256 MB Infinity Cache, so every
    launch streams from HBM, and host launch overhead does not pad short
    kernels.  The faster of three replays."""
    import torch

    for f in fns:
        f()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for r in range(reps):
            fns[r % len(fns)]()
    graph.replay()
    torch.cuda.synchronize()
    best = None
    for _ in range(3):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        graph.replay()
        b.record()
        torch.cuda.synchronize()
        us = a.elapsed_time(b) * 1e3 / reps
        best = us if best is None else min(best, us)
    del graph
    return best


def stream_ceiling(ref, nbytes, reads, dev, family=STREAM_FAMILY, touch=COLD_TOUCH):
    """The fastest member of the streaming-reference family moving `nbytes`
    with `reads` (0, 1 or 2) reads per write, same cold-cache rotation:
    (us per launch, member)."""
    import torch

    wbytes = nbytes // (1 + reads)
    nsets = max(2, -(-touch // nbytes))
    sets = [[torch.empty(wbytes, dtype=torch.uint8, device=dev) for _ in range(reads + 1)]
            for _ in range(nsets)]

    def launch(st, cfg):
        a = st[0].data_ptr() if reads >= 1 else None
        b = st[1].data_ptr() if reads == 2 else None
        status = ref.rgg_stream_ref(a, b, st[-1].data_ptr(), wbytes // 16, *cfg,
                                    torch.cuda.current_stream(dev).cuda_stream)
        if status:
            raise RuntimeError(f"rgg_stream_ref returned {status}")
    best = None
    for cfg in family:
        us = cold_us([(lambda st=st, cfg=cfg: launch(st, cfg)) for st in sets])
        if best is None or us < best[0]:
            best = (us, cfg)
    del sets
    return best


def run_stream_sweep(out=None):
    """The whole streaming-reference family at the graded traffic of each
    workload (RoPE 1 read : 1 write at 104 MB, 136 MB and 1.09 GB; GEGLU
    2 : 1 at 604 MB and 1.61 GB), cold caches as cold_us times them: workgroup
    size, vectors per lane, one pass or persistent grids, cache policy and
    residency caps.  Writes a markdown summary (the ten fastest members per
    size and the fastest of each grid form) to `out`."""
    import itertools

    import torch

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    ref = stream_ref_library()
    sizes = [("partial RoPE traffic", 103809024, 1), ("rope_qk RoPE traffic", 136314880, 1),
             ("dit_layer RoPE traffic", 1090519040, 1), ("geglu GEGLU traffic", 603979776, 2),
             ("dit_layer GEGLU traffic", 1610612736, 2)]
    caps = {3: 54528, 4: 40960, 5: 32768, 6: 27136}
    lines = ["# Streaming-reference family, cold caches", "",
             "Command: `python bench.py --stream-sweep --stream-sweep-out profiles/stream_family_sweep.md`",
             "", "Members: (workgroup size, 16-byte vectors per lane, grid: 0 one pass / n persistent "
             "workgroups, policy: 1 nontemporal loads, +2 nontemporal stores, +4 write-through (sc1) "
             "stores, LDS bytes per workgroup capping residency).  Time per launch from a HIP graph "
             "of 40 launches over buffer sets touching >= 2 GiB (cold_us in bench.py).", ""]
    for label, nbytes, reads in sizes:
        wbytes = nbytes // (1 + reads)
        nvec = wbytes // 16
        nsets = max(2, -(-COLD_TOUCH // nbytes))
        sets = [[torch.ones(wbytes, dtype=torch.uint8, device=dev) for _ in range(reads + 1)]
                for _ in range(nsets)]
        cfgs = []
        for vpl, block, pol in itertools.product((1, 2, 4, 8), (256, 512, 1024), (1, 2, 3, 5, 7)):
            for grid in (0, 256, 512, 1024, 2048):
                if grid and grid * block * vpl >= nvec:
                    continue
                cfgs.append((block, vpl, grid, pol, 0))
        for (block, vpl), pol, n in itertools.product(((256, 1), (256, 2)), (3, 7), caps):
            cfgs.append((block, vpl, 0, pol, caps[n]))
        res = []
        for cfg in cfgs:
            def launch(st, cfg=cfg):
                b = st[1].data_ptr() if reads == 2 else None
                status = ref.rgg_stream_ref(st[0].data_ptr(), b, st[-1].data_ptr(), nvec, *cfg,
                                            torch.cuda.current_stream(dev).cuda_stream)
                if status:
                    raise RuntimeError(f"rgg_stream_ref returned {status}")
            us = cold_us([(lambda st=st: launch(st)) for st in sets])
            res.append((us, cfg))
        del sets
        torch.cuda.empty_cache()
        res.sort()
        frac = lambda us: 100 * nbytes / (us * 1e-6) / 1e9 / PEAK_HBM_GBPS
        lines += [f"## {label}: {nbytes} bytes, {reads} read(s) per write, {len(res)} members", "",
                  "| rank | block | vectors/lane | grid | policy | LDS | us | % of 8 TB/s |",
                  "|---|---|---|---|---|---|---|---|"]
        for k, (us, c) in enumerate(res[:10]):
            lines.append(f"| {k + 1} | {c[0]} | {c[1]} | {c[2]} | {c[3]} | {c[4]} | {us:.2f} | {frac(us):.1f} |")
        lines += ["", "Fastest per grid form: " + "; ".join(
            f"grid {g}: {min(us for us, c in res if c[2] == g):.2f} us"
            for g in sorted({c[2] for _, c in res})), ""]
        print("\n".join(lines[-16:]), flush=True)
    text = "\n".join(lines) + "\n"
    if out:
        with open(out, "w") as f:
            f.write(text)
    return text


def rope_cold_sets(wid, dev, touch=COLD_TOUCH, layouts=False):
    """Buffer sets of a RoPE workload for cold timing: angles, tables, the
    input views and separate outputs (and, for the fused-QKV workload, the
    attention consumer's (B, H, S, D) outputs when `layouts`)."""
    import torch

    import bf16_rope_geglu_amd as rgg
    import workloads as W

    r = W.WORKLOADS[wid]["rope"]
    B, S, H, D = r["B"], r["S"], r["H"], r["D"]
    algo = W.algo_bytes(wid)
    nsets = max(2, -(-touch // (algo["rope"] + algo["precompute"])))
    fr = torch.from_numpy(W.workload_freqs(wid)).to(dev)
    sets = []
    for k in range(nsets):
        freqs = fr.clone()
        cos, sin = rgg.rope_cossin_precompute(freqs)
        if r["layout"] == "qkv":
            qkv = W.device_normal_bf16((B, S, 3 * H * D), 100 + k, device=dev)
            xs = [qkv[..., :H * D].view(B, S, H, D), qkv[..., H * D:2 * H * D].view(B, S, H, D)]
        else:
            xs = [W.device_normal_bf16((B, S, H, D), 100 + 4 * k + v, device=dev)
                  for v in range(r["views"])]
        outs = [torch.empty((B, S, H, D), dtype=torch.bfloat16, device=dev) for _ in xs]
        bhsd = ([torch.empty((B, H, S, D), dtype=torch.bfloat16, device=dev).permute(0, 2, 1, 3)
                 for _ in xs] if layouts and r["layout"] == "qkv" else None)
        sets.append({"freqs": freqs, "cos": cos, "sin": sin, "x": xs, "out": outs, "bhsd": bhsd})
    return sets


def geglu_cold_sets(rows, hidden, gate_sigma, dev, seed0=200, touch=COLD_TOUCH):
    import torch

    import workloads as W

    nsets = max(2, -(-touch // (rows * hidden * 6)))
    return [(W.device_normal_bf16((rows, 2 * hidden), seed0 + k, gate_sigma, dev),
             torch.empty((rows, hidden), dtype=torch.bfloat16, device=dev)) for k in range(nsets)]


def _entry(us, nbytes, ceiling=None):
    e = {"us": round(us, 2), "algo_bytes": nbytes,
         "GBps": round(nbytes / (us * 1e-6) / 1e9, 1),
         "frac": round(nbytes / (us * 1e-6) / 1e9 / PEAK_HBM_GBPS, 4)}
    if ceiling:
        cus, cfg = ceiling
        e["ceiling"] = {"us": round(cus, 2), "frac": round(nbytes / (cus * 1e-6) / 1e9 / PEAK_HBM_GBPS, 4),
                        "stream": {"block": cfg[0], "vectors_per_lane": cfg[1], "grid": cfg[2],
                                   "policy": cfg[3], "lds": cfg[4]}}
        e["vs_ceiling"] = round(cus / us, 4)
    return e


def run_configs(dev):
    """The graded kernels on every workload that carries them, cold caches,
    each beside the fastest streaming reference of the same traffic:
    rope_rotate_half_bf16 on rope_qk, partial and dit_layer (q and k views of
    the fused QKV output), gelu_and_mul_bf16 on geglu and dit_layer."""
    import torch

    import bf16_rope_geglu_amd as rgg
    import workloads as W

    ref = stream_ref_library()
    res = {}
    for wid, wl in sorted(W.WORKLOADS.items()):
        if wid == 0:
            continue
        algo = W.algo_bytes(wid)
        ent = {}
        if "rope" in wl:
            sets = rope_cold_sets(wid, dev)
            us = cold_us([(lambda st=st: rgg.rope_rotate_half_bf16(st["x"], st["cos"], st["sin"],
                                                                  out=st["out"])) for st in sets])
            del sets
            ent["rope_rotate_half_bf16"] = _entry(us, algo["rope"],
                                                  stream_ceiling(ref, algo["rope"], 1, dev))
        if "geglu" in wl:
            g = wl["geglu"]
            sets = geglu_cold_sets(g["rows"], g["hidden"], g["gate_sigma"], dev)
            us = cold_us([(lambda st=st: rgg.gelu_and_mul_bf16(st[0], st[1])) for st in sets])
            del sets
            ent["gelu_and_mul_bf16"] = _entry(us, algo["geglu"],
                                              stream_ceiling(ref, algo["geglu"], 2, dev))
        res[wl["name"]] = ent
        torch.cuda.empty_cache()
    return res


def run_sweep():
    """Per-launch time of each kernel on each workload, cold caches (see
    cold_us), each beside the fastest streaming reference of the same traffic
    (see stream_ceiling), then one rank's share of dit_layer and the
    projection."""
    import torch

    import bf16_rope_geglu_amd as rgg
    import workloads as W

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    rgg.prepare_device(0)
    rows_out = []
    ref = stream_ref_library()

    def add(label, name, nbytes, nsets, fns, reads):
        us = cold_us(fns)
        cus, _ = stream_ceiling(ref, nbytes, reads, dev)
        rows_out.append((label, name, nbytes, nsets, us, nbytes / (us * 1e-6) / 1e9, cus))

    for wid, wl in sorted(W.WORKLOADS.items()):
        if wid == 0:
            continue
        algo = W.algo_bytes(wid)
        if "rope" in wl:
            r = wl["rope"]
            B = r["B"]
            sets = rope_cold_sets(wid, dev, layouts=True)
            n = len(sets)
            add(wl["name"], "rope_cossin_precompute", algo["precompute"], n,
                [(lambda st=st: rgg.rope_cossin_precompute(st["freqs"], st["cos"], st["sin"]))
                 for st in sets], 1)
            fk = r["freqs"]
            if fk["kind"] == "3axis":
                add(wl["name"], "rope_cossin_from_grid", algo["precompute_grid"], n,
                    [(lambda st=st: rgg.rope_cossin_from_grid(
                        B, fk["grid"], fk["dims"], W.THETA, cos_out=st["cos"], sin_out=st["sin"]))
                     for st in sets], 0)
            add(wl["name"], "rope_rotate_half_bf16", algo["rope"], n,
                [(lambda st=st: rgg.rope_rotate_half_bf16(st["x"], st["cos"], st["sin"], out=st["out"]))
                 for st in sets], 1)
            if r["layout"] == "qkv":
                add(wl["name"], "rope_rotate_half_bf16, in place in qkv", algo["rope"], n,
                    [(lambda st=st: rgg.rope_rotate_half_bf16(st["x"], st["cos"], st["sin"], out=st["x"]))
                     for st in sets], 1)
                add(wl["name"], "rope_rotate_half_bf16, into (B, H, S, D)", algo["rope"], n,
                    [(lambda st=st: rgg.rope_rotate_half_bf16(st["x"], st["cos"], st["sin"],
                                                             out=st["bhsd"])) for st in sets], 1)
            del sets
        if "geglu" in wl:
            g = wl["geglu"]
            sets = geglu_cold_sets(g["rows"], g["hidden"], g["gate_sigma"], dev)
            add(wl["name"], "gelu_and_mul_bf16", algo["geglu"], len(sets),
                [(lambda st=st: rgg.gelu_and_mul_bf16(st[0], st[1])) for st in sets], 2)
            del sets
        torch.cuda.empty_cache()

    # One rank's share of dit_layer when the layer is split over 8 GPUs: the
    # path has no exchange of its own, so a rank runs the same kernels on a
    # slice, tokens (sequence parallel: qkv rows S/8, table rows of its own
    # tokens; GEGLU rows/8) or heads (q and k with H/8 heads after the
    # all-to-all, the whole table; GEGLU with hidden/8 columns).
    P = 8
    r = W.WORKLOADS[4]["rope"]
    g = W.WORKLOADS[4]["geglu"]
    B, S, H, D, R = r["B"], r["S"], r["H"], r["D"], r["R"]
    fr_all = torch.from_numpy(W.workload_freqs(4)).to(dev)
    for split, s_loc, h_loc in (("S/8 tokens", S // P, H), ("H/8 heads", S, H // P)):
        label = f"dit_layer, 1 of {P} ranks ({split})"
        T = B * s_loc
        pre_b = T * R * 4 + 2 * T * R * 2
        rope_b = 2 * (2 * T * h_loc * D * 2) + 2 * T * R * 2
        nsets = max(2, -(-COLD_TOUCH // (rope_b + pre_b)))
        sets = []
        for k in range(nsets):
            freqs = fr_all[:s_loc].clone()
            cos, sin = rgg.rope_cossin_precompute(freqs)
            if h_loc == H:
                qkv = W.device_normal_bf16((B, s_loc, 3 * H * D), 300 + k, device=dev)
                xs = [qkv[..., :H * D].view(B, s_loc, H, D),
                      qkv[..., H * D:2 * H * D].view(B, s_loc, H, D)]
            else:
                xs = [W.device_normal_bf16((B, s_loc, h_loc, D), 300 + 2 * k + v, device=dev)
                      for v in range(2)]
            outs = [torch.empty((B, s_loc, h_loc, D), dtype=torch.bfloat16, device=dev) for _ in xs]
            sets.append((freqs, cos, sin, xs, outs))
        if h_loc == H:
            add(label, "rope_cossin_precompute", pre_b, nsets,
                [(lambda st=st: rgg.rope_cossin_precompute(st[0], st[1], st[2])) for st in sets], 1)
        add(label, "rope_rotate_half_bf16", rope_b, nsets,
            [(lambda st=st: rgg.rope_rotate_half_bf16(st[3], st[1], st[2], out=st[4])) for st in sets], 1)
        del sets
    for split, rows, hid in (("S/8 tokens", g["rows"] // P, g["hidden"]),
                             ("hidden/8 columns", g["rows"], g["hidden"] // P)):
        sets = geglu_cold_sets(rows, hid, g["gate_sigma"], dev, seed0=400)
        add(f"dit_layer, 1 of {P} ranks ({split})", "gelu_and_mul_bf16", rows * hid * 6, len(sets),
            [(lambda st=st: rgg.gelu_and_mul_bf16(st[0], st[1])) for st in sets], 2)
        del sets
    del fr_all
    torch.cuda.empty_cache()

    proj = run_projection()
    print(f"Projection {proj['shape']} (matrix cores, {proj['flops']:.3e} flop per launch)")
    print("| entry point | us per launch | TFLOP/s | % of 2.5 PFLOP/s |")
    print("|---|---|---|---|")
    for n, r in proj["results"].items():
        print(f"| {n} | {r['us']:.1f} | {r['TFLOPs']:.1f} | {100 * r['frac']:.1f} |")
    print()
    print("| workload | entry point | algorithmic bytes | buffer sets | us per launch | GB/s "
          "| % of 8 TB/s | stream ceiling us (% of 8 TB/s) | kernel vs ceiling |")
    print("|---|---|---|---|---|---|---|---|---|")
    for w, n, b, k, us, gbps, sus in rows_out:
        sfrac = 100 * b / (sus * 1e-6) / 1e9 / PEAK_HBM_GBPS
        print(f"| {w} | {n} | {b} | {k} | {us:.1f} | {gbps:.0f} | {100 * gbps / PEAK_HBM_GBPS:.1f} "
              f"| {sus:.1f} ({sfrac:.1f}) | {100 * sus / us:.1f}% |")
    sys.stdout.flush()


# ---------------------------------------------------------------------------
# CPU baseline: the oracle on a bounded sample of the same workload
# ---------------------------------------------------------------------------

def run_cpu_baseline(wid, tokens=16384, geglu_rows=8192):
    """The oracle on a bounded sample of the workload: first on one thread
    (the reported value), then the same sample split over every core the
    process may use (ctypes releases the GIL, so threads run the C oracle in
    parallel on disjoint token and row ranges)."""
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np

    import oracle
    import workloads as W

    o = oracle.get()
    wl = W.WORKLOADS[wid]
    r, g = wl["rope"], wl["geglu"]
    H, D, R, hidden = r["H"], r["D"], r["R"], g["hidden"]
    # the first `tokens` table rows b*S + s, as angles of one batch row
    full = W.workload_freqs(wid)
    fr = np.ascontiguousarray(full.transpose(1, 0, 2, 3).reshape(-1, 1, 1, R)[:tokens])
    q = W.normal_bf16((1, tokens, H, D), W.seed_for(wid, "q"))
    k = W.normal_bf16((1, tokens, H, D), W.seed_for(wid, "k"))
    gate = W.normal_bf16((geglu_rows, hidden), W.seed_for(wid, "gate"), g["gate_sigma"])
    up = W.normal_bf16((geglu_rows, hidden), W.seed_for(wid, "up"))
    inp = np.concatenate([gate, up], axis=1)

    def part(t_lo, t_hi, g_lo, g_hi):
        cos, sin = o.rope_cossin(np.ascontiguousarray(fr[t_lo:t_hi]))
        o.rope_rotate_half(q[:, t_lo:t_hi], cos, sin)
        o.rope_rotate_half(k[:, t_lo:t_hi], cos, sin)
        o.gelu_and_mul(inp[g_lo:g_hi])

    t0 = time.perf_counter()
    part(0, tokens, 0, geglu_rows)
    dt = time.perf_counter() - t0
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    n = max(1, min(n, 64))
    cuts_t = [tokens * i // n for i in range(n + 1)]
    cuts_g = [geglu_rows * i // n for i in range(n + 1)]
    t0 = time.perf_counter()
    with ThreadPoolExecutor(max_workers=n) as pool:
        list(pool.map(lambda i: part(cuts_t[i], cuts_t[i + 1], cuts_g[i], cuts_g[i + 1]),
                      range(n)))
    dt_n = time.perf_counter() - t0
    nbytes = (tokens * R * 4 + 2 * tokens * R * 2) + (2 * 2 * tokens * H * D * 2 + 2 * tokens * R * 2) \
        + geglu_rows * hidden * 2 * 3
    return {
        "value": round(nbytes / dt / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
        "sample": (f"{tokens} of {r['B'] * r['S']} tokens (cos/sin, q and k RoPE) and "
                   f"{geglu_rows} of {g['rows']} GEGLU rows; {nbytes} algorithmic bytes in "
                   f"{dt:.2f} s on one thread"),
        "all_cores": {"value": round(nbytes / dt_n / 1e9, 4), "unit": "GB/s", "cores": n,
                      "seconds": round(dt_n, 2)},
        "cpu": _cpu_model(),
    }


def run_traffic(name, reps=6):
    """The RoPE launch of workload `name` (rope_qk or partial) over cold
    buffer sets, `reps` times, then a plain device copy of known size: the
    program that rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE passes profile for
    that workload's counter summary (--pmc-set NAME)."""
    import torch

    import bf16_rope_geglu_amd as rgg
    import workloads as W

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    wid = {w["name"]: k for k, w in W.WORKLOADS.items()}[name]
    sets = rope_cold_sets(wid, dev)
    for k in range(reps):
        st = sets[k % len(sets)]
        rgg.rope_rotate_half_bf16(st["x"], st["cos"], st["sin"], out=st["out"])
    src = torch.ones(COPY_BYTES // 2, dtype=torch.bfloat16, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(f"{name}: {reps} RoPE launches and 3 copies of {COPY_BYTES} bytes", flush=True)


def _cpu_model():
    """The host CPU's model name, as /proc/cpuinfo gives it (None if absent)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


# ---------------------------------------------------------------------------
# rocprofv3 counter summary (HBM traffic of the dominant kernel)
# ---------------------------------------------------------------------------

def _counter_rows(d):
    rows = []
    for path in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        with open(path) as f:
            rows.extend(csv.DictReader(f))
    return rows


def _per_dispatch(rows, counter, symbol):
    vals = {}
    for row in rows:
        name = row.get("Kernel_Name", "")
        if row.get("Counter_Name") != counter or symbol not in name:
            continue
        key = row.get("Dispatch_Id") or row.get("Correlation_Id") or str(len(vals))
        vals[key] = vals.get(key, 0.0) + float(row["Counter_Value"])
    return sorted(vals.values())


KNOWN_KERNELS = ("rope_cossin_kernel", "rope_cossin_grid_kernel", "rope_rotate_half_kernel",
                 "rope_rotate_half_lane_kernel", "rope_lean_kernel", "rope_xlane_kernel",
                 "gelu_and_mul_kernel", "build_gelu_table_kernel", "gemm_gate_up_kernel",
                 "stream_ref_kernel")


def _short_kernel(name):
    """The kernel's own name inside a demangled symbol such as
    `rgg::(anonymous namespace)::rope_rotate_half_kernel<true, true>(...)`;
    the projection kernel keeps its template argument (true: GEGLU epilogue)."""
    m = re.search(r"gemm_gate_up_kernel\s*<\s*(true|false)\s*>", name)
    if m:
        return f"gemm_gate_up_kernel<{m.group(1)}>"
    for v in KNOWN_KERNELS:
        if re.search(r"(?:^|::|\s)" + v + r"\s*[<(]", name):
            return v
    return None


def trace_summary(d, out, command):
    """Short markdown summary of a rocprofv3 --kernel-trace run: the --stats
    table if present, and the median dispatch duration of each run of
    consecutive dispatches of one kernel and grid (one workload of a sweep)."""
    lines = ["# rocprofv3 kernel trace", "", f"Command: `{command}`", ""]
    stats = []
    for path in glob.glob(os.path.join(d, "**", "*kernel_stats.csv"), recursive=True):
        with open(path) as f:
            stats.extend(csv.DictReader(f))
    if stats:
        lines += ["| kernel | calls | average us | min us | max us |", "|---|---|---|---|---|"]
        for row in stats:
            short = _short_kernel(row["Name"])
            if short:
                lines.append(f"| {short} | {row['Calls']} | {float(row['AverageNs']) / 1e3:.2f} | "
                             f"{float(row['MinNs']) / 1e3:.2f} | {float(row['MaxNs']) / 1e3:.2f} |")
        lines.append("")
    trace = []
    for path in glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True):
        with open(path) as f:
            trace.extend(csv.DictReader(f))
    trace = [r for r in trace if _short_kernel(r["Kernel_Name"])]
    trace.sort(key=lambda r: int(r["Start_Timestamp"]))
    groups = {}
    for r in trace:
        key = (_short_kernel(r["Kernel_Name"]), r["Grid_Size_X"], r["Workgroup_Size_X"])
        dur = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        groups.setdefault(key, []).append(dur)
    if groups:
        lines += ["Dispatch durations per kernel and launch shape, in order of first launch:", "",
                  "| kernel | grid threads | workgroup | dispatches | median us | min us |",
                  "|---|---|---|---|---|---|"]
        for (k, g, w), ds in groups.items():
            ds.sort()
            lines.append(f"| {k} | {g} | {w} | {len(ds)} | {ds[len(ds) // 2]:.2f} | {ds[0]:.2f} |")
        lines.append("")
    text = "\n".join(lines)
    if out:
        with open(out, "w") as f:
            f.write(text)
    print(text)


PROJ_SYMBOL = {
    "projection_geglu": "gemm_gate_up_kernel<true>",
    "projection_plain": "gemm_gate_up_kernel<false>",
}


def projection_algo_bytes():
    """x and W read once, the output written once (dit_layer projection)."""
    import workloads as W
    pr = W.WORKLOADS[4]["proj"]
    M, K, H = pr["rows"], pr["dim"], pr["hidden"]
    inputs = 2 * M * K + 2 * 2 * H * K
    return {"projection_geglu": inputs + 2 * M * H, "projection_plain": inputs + 2 * M * 2 * H}


def pmc_summary(d, out, command="", which="step"):
    fetch = _counter_rows(os.path.join(d, "fetch"))
    write = _counter_rows(os.path.join(d, "write"))
    copy_sym = "copyBuffer"   # the HIP runtime's device-to-device copy kernel
    res = {"source_digest": source_digest(), "copy_bytes": COPY_BYTES}
    cf = _per_dispatch(fetch, "FETCH_SIZE", copy_sym)
    cw = _per_dispatch(write, "WRITE_SIZE", copy_sym)
    big_f = [v for v in cf if v * 1024 > COPY_BYTES / 2]
    big_w = [v for v in cw if v * 1024 > COPY_BYTES / 2]
    f_scale = COPY_BYTES / (1024 * sorted(big_f)[len(big_f) // 2]) if big_f else None
    w_scale = COPY_BYTES / (1024 * sorted(big_w)[len(big_w) // 2]) if big_w else None
    res["fetch_scale"] = f_scale
    res["write_scale"] = w_scale
    if which == "projection":
        title, symbols, algo = ("the gate_up projection of the dit_layer workload", PROJ_SYMBOL,
                                projection_algo_bytes())
    elif which == "step":
        import workloads as W
        title, symbols, algo = "dit_layer workload", KERNEL_SYMBOL, W.algo_bytes(4)
    else:
        import workloads as W
        wid = {w["name"]: k for k, w in W.WORKLOADS.items()}[which]
        title, symbols, algo = (f"{which} workload", {"rope": KERNEL_SYMBOL["rope"]},
                                W.algo_bytes(wid))
    lines = [f"# HBM traffic per dispatch from rocprofv3 counters ({title})", "",
             f"Commands: `{command}`", ""]
    for n, sym in symbols.items():
        f = _per_dispatch(fetch, "FETCH_SIZE", sym)
        w = _per_dispatch(write, "WRITE_SIZE", sym)
        if not f or not w:
            continue
        fk, wk = f[len(f) // 2], w[len(w) // 2]
        fb = fk * 1024 * (f_scale or 1.0)
        wb = wk * 1024 * (w_scale or 1.0)
        res[n] = {"fetch_kib": fk, "write_kib": wk, "bytes": fb + wb, "dispatches": len(f)}
        lines.append(f"- {sym}: FETCH_SIZE {fk:.0f} KiB, WRITE_SIZE {wk:.0f} KiB per dispatch "
                     f"(median of {len(f)}); scaled total {(fb + wb) / 1e9:.4f} GB"
                     + (f" against {algo[n] / 1e9:.4f} GB algorithmic" if n in algo else ""))
    lines += ["", f"Copy calibration ({COPY_BYTES} bytes each way): fetch scale {f_scale}, "
              f"write scale {w_scale}", "", "```json", json.dumps(res, indent=1), "```", ""]
    with open(out, "w") as f:
        f.write("\n".join(lines))
    print("\n".join(lines))


def counter_summary(d, out, command=""):
    """Median per dispatch (summed over the counter's hardware instances) of
    every counter found under `d` (one subfolder per rocprofv3 --pmc pass),
    for the projection kernels and the platform GEMM that `--projection`
    times beside them."""
    vals = {}
    for path in sorted(glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)):
        per = {}
        with open(path) as f:
            for r in csv.DictReader(f):
                name = r["Kernel_Name"]
                short = _short_kernel(name)
                if short is None and "Cijk_" in name:
                    short = "hipBLASLt GEMM (torch.matmul)"
                if short is None:
                    continue
                key = (short, r["Counter_Name"], r["Dispatch_Id"])
                per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
        for (k, c, _), v in per.items():
            vals.setdefault((k, c), []).append(v)
    kernels = sorted({k for k, _ in vals})
    counters = sorted({c for _, c in vals})
    lines = ["# rocprofv3 counters per dispatch (the gate_up projection of the dit_layer workload)",
             "", f"Commands: `{command}`", "",
             "| counter | " + " | ".join(kernels) + " |",
             "|---|" + "---|" * len(kernels)]
    for c in counters:
        cells = []
        for k in kernels:
            v = sorted(vals.get((k, c), []))
            cells.append(f"{v[len(v) // 2]:.6g}" if v else "")
        lines.append(f"| {c} | " + " | ".join(cells) + " |")
    lines.append("")
    text = "\n".join(lines)
    if out:
        with open(out, "w") as f:
            f.write(text)
    print(text)


def traffic_for(kernel):
    """Counter bytes of `kernel` from the committed summary, if still current."""
    try:
        with open(TRAFFIC_SUMMARY) as f:
            text = f.read()
        blob = json.loads(text.split("```json", 1)[1].split("```", 1)[0])
    except (OSError, IndexError, ValueError):
        return None
    if blob.get("source_digest") != source_digest() or kernel not in blob:
        return None
    return blob[kernel]["bytes"]


# ---------------------------------------------------------------------------

def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="dit_layer", choices=["dit_layer"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the per-workload cold-cache kernel timings in the JSON line")
    ap.add_argument("--no-projection", action="store_true",
                    help="skip the gate_up projection timings in the JSON line")
    ap.add_argument("--calibration-copy", action="store_true")
    ap.add_argument("--pmc-summary", metavar="DIR")
    ap.add_argument("--pmc-out", metavar="FILE", default=TRAFFIC_SUMMARY)
    ap.add_argument("--pmc-set", choices=["step", "projection", "rope_qk", "partial"], default="step")
    ap.add_argument("--traffic-run", choices=["rope_qk", "partial"],
                    help="run one workload's RoPE launches and a calibration copy (for --pmc)")
    ap.add_argument("--projection", action="store_true",
                    help="time only the gate_up projection entry points (JSON)")
    ap.add_argument("--counter-summary", metavar="DIR")
    ap.add_argument("--counter-out", metavar="FILE")
    ap.add_argument("--trace-summary", metavar="DIR")
    ap.add_argument("--trace-out", metavar="FILE")
    ap.add_argument("--command", default="", help="command line recorded in summaries")
    ap.add_argument("--sweep", action="store_true",
                    help="time every kernel on every workload (cold caches) instead")
    ap.add_argument("--stream-sweep", action="store_true",
                    help="time the whole streaming-reference family at each workload's traffic")
    ap.add_argument("--stream-sweep-out", metavar="FILE")
    args = ap.parse_args()

    if args.pmc_summary:
        pmc_summary(args.pmc_summary, args.pmc_out, args.command, args.pmc_set)
        return 0
    if args.traffic_run:
        run_traffic(args.traffic_run)
        return 0
    if args.projection:
        import torch
        torch.cuda.set_device(0)
        res = run_projection()
        if args.calibration_copy:
            src = torch.ones(COPY_BYTES // 2, dtype=torch.bfloat16, device="cuda:0")
            dst = torch.empty_like(src)
            for _ in range(3):
                dst.copy_(src)
            torch.cuda.synchronize()
        print(json.dumps(res), flush=True)
        return 0
    if args.trace_summary:
        trace_summary(args.trace_summary, args.trace_out, args.command)
        return 0
    if args.counter_summary:
        counter_summary(args.counter_summary, args.counter_out, args.command)
        return 0
    if args.sweep:
        run_sweep()
        return 0
    if args.stream_sweep:
        run_stream_sweep(args.stream_sweep_out)
        return 0
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this path has no multi-GPU step (each rank would run "
              "the same per-token kernels on its own shard with no exchange); run with --gpus 1.",
              file=sys.stderr)
        return 2

    res = run_gpu(args)
    B, S, H, D, R, rows, hidden = res["shape"]
    dom = res["dominant"]
    kd = res["kernels"][dom]
    traffic = traffic_for(dom)
    value = res["step_bytes"] / (res["ms_per_step"] * 1e-3) / 1e9
    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(res["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) bf16 activations, 3-axis rotary angles)",
        "config": {"workload": f"{args.workload}: fused QKV (B={B}, S={S}, 3*{H}*{D}) with q/k "
                               f"strided views, rot_dim={R}; GEGLU {rows} x 2*{hidden}",
                   "step_bytes": res["step_bytes"], "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "hbm", "kernel": kd["symbol"], "achieved": kd["GBps"],
                     "peak": PEAK_HBM_GBPS, "unit": "GB/s", "frac": kd["frac"],
                     "traffic": traffic},
        "kernels": res["kernels"],
        "frac_of_peak": round(value / PEAK_HBM_GBPS, 4),
    }
    if not args.no_configs:
        import torch
        line["configs"] = run_configs(torch.device("cuda:0"))
    if not args.no_projection:
        line["projection"] = run_projection()
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = run_cpu_baseline(res["wid"])
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
