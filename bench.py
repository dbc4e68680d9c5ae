#!/usr/bin/env python3
"""Throughput of the NVFP4 block-scaled batched GEMV on one MI355X.

One step = one call of the GEMV (all of its kernels) on one batch of inputs.
With no arguments the GEMV is measured on each of its five workloads in turn
and one JSON line is printed per workload, the batched workload (l=8,
m=4096, k=7168, the largest operand that the metric's "batched GEMV" names)
last:

  tiny      l=1,  m=128,  k=256    integer-coded, alpha 1   (launch-bound)
  decode    l=1,  m=7168, k=16384  integer-coded, alpha 1
  shortk    l=4,  m=7168, k=2048   integer-coded, alpha 1
  gaussian  l=16, m=2048, k=4096   bf16 N(0,1) quantised per batch, alpha gA*gx
  batched   l=8,  m=4096, k=7168   integer-coded, alpha U[0.5, 2]

Every footprint fits in MI355X's 256 MB Infinity Cache, so the timed steps
rotate over device copies of the inputs (>= 1 GB together) and every step
reads its operands from HBM; a cache-resident ("warm") figure is reported
separately and labelled as such.

Timing: W warm-up steps, then a synchronisation, then exactly K steps between
two HIP events on the launch stream, then a synchronisation.  A GPU-side
delay kernel (about 0.8 ms) runs before the start event, so the stream is not
idle while the host enqueues the first steps and the clocks have left their
idle state.  The K steps are launched one by one from Python, and the same
K steps are also captured once into a HIP graph, replayed once untimed and
timed as one replay; both figures are reported.  With --launch graph (the
default) the replay is the headline figure, as in a decode loop captured in
a graph; --launch stream makes the one-by-one launches the headline.

Each JSON line:
  value        algorithmic bytes per step (A + sfA + x + sfx + c) / time, GB/s
  roofline     the same rate against the 8 TB/s HBM peak, the kernel's HBM
               traffic from rocprofv3 counters when they were taken on this
               kernel source, and the read rates of streaming-read probes
               measured in the same run, each the faster of stream launches
               and a graph replay (a flat 1 GiB read; the workload's own A and
               sfA read with the long-row GEMV's load pattern; a flat read of
               the same size)
  cpu_baseline the CPU oracle (plain C, fp64, OpenMP over rows) on the same
               workload on this host's cores, with the parity of the last
               timed call against it

Other paths (--path), each printing its own JSON line of the same form (their
steps are launched one by one; with --launch graph, the default, the replay of
a HIP graph holding the same K steps is added and is the reported figure,
which also keeps the stream busy under a kernel tracer that slows the host's
launches):
  quantize     the BF16 -> NVFP4 activation quantiser on a bf16 activation
               batch (--act-config tokens | decode_x)
  gemv_bf16x   the GEMV fed by a bf16 activation: quantiser + GEMV per step
  smalln       the small-N GEMM: one weight matrix against n vectors
               (--smalln-config decode_n2 | decode_n4 | decode_n16 | tiny_n3)
  grouped      the grouped (MoE) GEMV: routed tokens against their experts'
               weights (--moe-config moe_decode | moe_tiny)
  --packed     with smalln / grouped: the weights are packed once into the
               matrix-core tile layout (not timed) and the packed calls timed

--trace-cold runs only the warm-up and the timed steps (no cache-resident
loop, single launches, probes or CPU baseline), for rocprofv3 kernel traces
whose averages then cover HBM-cold launches only.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--config all|decode|...]
                       [--launch graph|stream] [--trace-cold]
                       [--path gemv|quantize|gemv_bf16x|smalln|grouped] [--packed]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "achieved HBM GB/s and % of MI355X peak for NVFP4 batched GEMV; \u00b5s/call"
# GEMV workloads of --config all, in print order: the batched workload's line last
GEMV_ORDER = ("tiny", "decode", "shortk", "gaussian", "batched")
# GPU-side delay before a timed region (clock cycles of torch's spin kernel)
PREROLL_CYCLES = 2_000_000
# at most this many input copies (the tiny workload would otherwise need 50000)
MAX_REPLICAS = 64
MAX_GRAPH_STEPS = 20000     # kernel nodes in one captured graph
CSRC = os.path.join(ROOT, "precision_decode_amd", "csrc")
PROFILES = os.path.join(ROOT, "profiles")
# counter summaries under profiles/ are valid only for the source they were taken on
# (the GEMV's device code is gemv_kernels.h with its helpers in device_common.h)
KERNEL_SOURCES = {"gemv": ("gemv_kernels.h", "device_common.h"),
                  "quantize_blocks": ("nvfp4_quantize.hip", "quant_arith.h", "device_common.h"),
                  "mma_stream": ("mma_kernels.h", "device_common.h"),
                  "mma_lds": ("mma_kernels.h", "device_common.h"),
                  "mma_generic": ("mma_kernels.h", "device_common.h"),
                  "vec_tile": ("mma_kernels.h", "device_common.h"),
                  "mma_stream_packed": ("mma_kernels.h", "device_common.h")}


def parse_args(argv=None):
    p = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=2000)
    p.add_argument("--warmup", type=int, default=100)
    p.add_argument("--path", default="gemv",
                   choices=["gemv", "quantize", "gemv_bf16x", "smalln", "grouped"])
    p.add_argument("--config", default="all",
                   help="GEMV workload from workloads.CONFIGS (decode, batched, shortk, tiny, or "
                        "gaussian: bf16 draws quantised by the library's device quantiser, untimed), "
                        "or all: each in turn, one JSON line each, batched last")
    p.add_argument("--launch", default="graph", choices=["graph", "stream"],
                   help="time the K steps as one replay of a HIP graph that holds them, or "
                        "launched one by one on the stream")
    p.add_argument("--trace-cold", action="store_true",
                   help="GEMV: only the warm-up and the timed steps (no cache-resident loop, "
                        "single launches, probes or CPU baseline), for kernel traces")
    p.add_argument("--act-config", default="tokens",
                   help="activation workload of --path quantize (workloads.ACT_CONFIGS)")
    p.add_argument("--smalln-config", default="decode_n16",
                   help="workload of --path smalln (workloads.SMALLN_CONFIGS)")
    p.add_argument("--moe-config", default="moe_decode",
                   help="workload of --path grouped (workloads.MOE_CONFIGS)")
    p.add_argument("--out-type", type=int, default=None,
                   help="output format of --path smalln / grouped: 0 fp16, 1 bf16 "
                        "(default fp16 for smalln, bf16 for grouped)")
    p.add_argument("--rule", type=int, default=0,
                   help="E2M1 rounding rule of the quantiser (0 half-step, 1 nearest-even, "
                        "2 nearest-lower)")
    p.add_argument("--replicas", type=int, default=0,
                   help="device copies of the inputs to rotate over (0: enough for >= 1 GB)")
    p.add_argument("--variant", type=int, default=0,
                   help="fast-kernel variant of the chosen path (0 = default plan)")
    p.add_argument("--ksplit", type=int, default=0, help="K split (0 = default plan)")
    p.add_argument("--packed", action="store_true",
                   help="--path smalln / grouped: weights pre-packed once (nvfp4_mma_pack_weight, "
                        "outside the timed region) and the packed launches timed")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-probe", action="store_true")
    p.add_argument("--single-launches", type=int, default=50,
                   help="GEMV: single launches, each after a 512 MiB streaming read, for per-launch "
                        "latency percentiles (0 = skip)")
    p.add_argument("--copy-mib", type=int, default=0,
                   help="after timing, run 4 plain device copies of this many MiB (the "
                        "known-size reference for HBM byte counters)")
    args = p.parse_args(argv)
    if args.steps < 1 or args.warmup < 0:
        p.error("--steps must be at least 1 and --warmup at least 0")
    if args.launch == "graph" and args.steps > MAX_GRAPH_STEPS:
        p.error(f"--launch graph captures the K steps in one HIP graph: --steps at most "
                f"{MAX_GRAPH_STEPS} (use --launch stream for more)")
    return args


def kernel_source_hash(kernel: str = "gemv") -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[kernel]:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def recorded_traffic(config: str, kernel: str = "gemv"):
    """HBM bytes per launch from a committed counter summary, if it was taken
    on the current kernel source; otherwise None."""
    path = os.path.join(PROFILES, f"{kernel}_{config}_hbm_counters.txt")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    h = re.search(r"^kernel_source_sha256_16:\s*(\w+)", text, re.M)
    t = re.search(r"^hbm_bytes_per_launch:\s*([0-9.eE+]+)", text, re.M)
    if not h or not t or h.group(1) != kernel_source_hash(kernel):
        return None
    return float(t.group(1))


def single_launch_percentiles(torch, stream, step, n, evict=None):
    """p10/p50/p90 of single launches (HIP events on the launch stream around one
    step).  Before each launch `evict(i)` runs on the same stream; by default it
    writes 512 MiB.  The GEMV bench passes a 512 MiB streaming read instead, which
    evicts the operands from L2 and the Infinity Cache without leaving dirty
    lines there, so each launch starts cold and alone."""
    if n <= 0:
        return None
    scratch = None
    if evict is None:
        scratch = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
        evict = lambda i: scratch.fill_(i & 0xFF)
    times = []
    for i in range(n):
        evict(i)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        step(i)
        e1.record(stream)
        e1.synchronize()
        times.append(e0.elapsed_time(e1) * 1e3)
    del scratch
    times.sort()

    def pct(q):
        return round(times[min(len(times) - 1, int(q * (len(times) - 1) + 0.5))], 2)

    return {"p10": pct(0.1), "p50": pct(0.5), "p90": pct(0.9), "launches": n}


class Timer:
    """HIP events on the launch stream around n back-to-back calls.  A GPU-side
    delay kernel runs first, so the stream is busy (not idle at the start
    event) while the host enqueues the first calls."""

    def __init__(self, torch, stream):
        self.torch, self.stream = torch, stream
        self.enqueue_s = 0.0

    def preroll(self):
        sleep = getattr(self.torch.cuda, "_sleep", None)
        if sleep is not None:
            try:
                sleep(PREROLL_CYCLES)
            except RuntimeError:
                self.torch.cuda._sleep = None     # not available in this torch: no delay

    def __call__(self, n, fn):
        torch = self.torch
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        self.preroll()
        start.record(self.stream)
        for i in range(n):
            fn(i)
        end.record(self.stream)
        self.enqueue_s = time.perf_counter() - t0
        torch.cuda.synchronize()
        return start.elapsed_time(end), time.perf_counter() - t0


def capture_steps(torch, n, step, state, cs=None):
    """A HIP graph holding steps 0 .. n-1, captured on the side stream `cs`
    (a new one when None; nothing runs).  `state["stream"]` is the stream the
    step function launches on."""
    g = torch.cuda.CUDAGraph()
    cs = torch.cuda.Stream() if cs is None else cs
    main = torch.cuda.current_stream()
    cs.wait_stream(main)
    try:
        with torch.cuda.graph(g, stream=cs):
            state["stream"] = cs.cuda_stream
            for i in range(n):
                step(i)
    finally:
        state["stream"] = main.cuda_stream
    main.wait_stream(cs)
    return g


def replicate(torch, base, nbytes, reps_arg):
    reps = reps_arg or min(MAX_REPLICAS, max(1, -(-1_000_000_000 // nbytes)))
    return [base] + [{n: t.clone() for n, t in base.items()} for _ in range(reps - 1)], reps


def pack_replicas(torch, pd, replicas, wkey, skey, groups, rows, k):
    """Adds the packed form of each replica's weights (an offline step, before
    any timing); the row-major weights are dropped so only packed bytes rotate."""
    cb, sb = pd.nvfp4_mma_packed_sizes(groups, rows, k)
    for r in replicas:
        wp = torch.empty(cb, dtype=torch.uint8, device="cuda")
        swp = torch.empty(sb, dtype=torch.uint8, device="cuda")
        pd.nvfp4_mma_pack_weight(r[wkey], r[skey], groups, rows, k, wp, swp)
        r[wkey + "_packed"], r[skey + "_packed"] = wp, swp
    torch.cuda.synchronize()
    for r in replicas:
        del r[wkey], r[skey]


def run_copies(torch, mib):
    if mib:
        src = torch.ones(mib << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(4):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(f"[bench] ran 4 device copies of {mib} MiB", flush=True)


def roofline(gbs, traffic, **extra):
    r = {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
         "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": traffic}
    r.update({k: (round(v, 4 if k.startswith("frac") else 2) if isinstance(v, float) else v)
              for k, v in extra.items()})
    return r


def parity_summary(np, got, want):
    """fp16 outputs of the GPU against the oracle's: how many are bit-identical
    and the largest distance in fp16 ulps (over the ordered bit patterns)."""
    got = np.asarray(got, dtype=np.uint16).reshape(-1)
    want = np.asarray(want, dtype=np.uint16).reshape(-1)

    def ordered(b):
        b = b.astype(np.int64)
        return np.where(b & 0x8000, -(b & 0x7FFF), b & 0x7FFF)

    dist = np.abs(ordered(got) - ordered(want))
    return {"outputs": int(got.size), "bit_identical": int(np.count_nonzero(got == want)),
            "max_ulp": int(dist.max()) if dist.size else 0}


def with_speedup(cpu, gbs):
    """The CPU baseline with the GPU's throughput ratio to it (None stays None)."""
    if cpu is None:
        return None
    return dict(cpu, gpu_speedup=round(gbs / cpu["value"], 1))


def common_fields(args, gbs, ms_step, dtype):
    return {"value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": round(ms_step, 6),
            "us_per_call": round(ms_step * 1e3, 3),
            "pct_of_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2), "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": dtype, "data": "synthetic"}


def timed_steps(args, timer, step, nbytes, label, state, capture_stream):
    """Warm-up, then the K steps launched one by one on the stream; with
    --launch graph, the same K steps are also captured into one HIP graph on
    `capture_stream` and its replay gives the step time.  `step` launches on
    state["stream"].  Returns (ms per step, GB/s, the timings in us)."""
    for i in range(args.warmup):
        step(i)
    timer.torch.cuda.synchronize()
    ms_total, wall = timer(args.steps, step)
    ms_step = ms_total / args.steps
    gbs = nbytes / (ms_step * 1e-3) / 1e9
    enqueue_us = timer.enqueue_s / args.steps * 1e6
    print(f"[bench] {label}: {args.steps} steps: {ms_step * 1e3:.2f} us/step, {gbs:.1f} GB/s "
          f"({100 * gbs / HBM_PEAK_GBS:.1f}% of peak), host wall {wall:.3f}s, host enqueue "
          f"{enqueue_us:.2f} us/step", flush=True)
    timing = {"graph_replay": None, "stream_launches": round(ms_step * 1e3, 3),
              "host_enqueue_per_launch": round(enqueue_us, 3)}
    if args.launch == "graph":
        g = capture_steps(timer.torch, args.steps, step, state, capture_stream)
        g.replay()                                   # untimed: uploads the graph
        timer.torch.cuda.synchronize()
        ms_total, _ = timer(1, lambda i: g.replay())
        ms_step = ms_total / args.steps
        gbs = nbytes / (ms_step * 1e-3) / 1e9
        timing["graph_replay"] = round(ms_step * 1e3, 3)
        print(f"[bench] {label}, one graph replay of {args.steps} steps: {ms_step * 1e3:.2f} us/step, "
              f"{gbs:.1f} GB/s ({100 * gbs / HBM_PEAK_GBS:.1f}% of peak)", flush=True)
    return ms_step, gbs, timing


def launch_label(args):
    return ("one HIP graph replay of the K steps" if args.launch == "graph"
            else "K launches on the stream")


def cpu_time(fn, runs=3):
    times = []
    for _ in range(runs):
        t0 = time.perf_counter()
        fn()
        times.append(time.perf_counter() - t0)
    return statistics.median(times)


# ------------------------------------------------------------------------------------ GEMV
def quantize_gaussian_on_device(torch, np, pd, raw, l, m, k):
    """NVFP4 operands of a Gaussian workload, quantised by the library's device
    weight quantiser (before any timing): each batch's A[b] and x[b] is a
    tensor of its own with its amax global scale, nearest-even codes, and
    alpha[b] = f32(gA[b] * gx[b])."""
    rule = pd.NVFP4_ROUND_NEAREST_EVEN
    out = {}
    scales = {}
    for name, rows in (("A", m), ("x", 1)):
        src = torch.from_numpy(np.ascontiguousarray(raw[name])).to(torch.bfloat16).cuda()
        codes = torch.empty((l, rows, k // 2), dtype=torch.uint8, device="cuda")
        sf = torch.empty((l, rows, k // 16), dtype=torch.uint8, device="cuda")
        g = torch.empty(l, dtype=torch.float32, device="cuda")
        pd.nvfp4_quantize_weight(src, l, rows, k, rule, codes, sf, g)
        shape = (l, m) if name == "A" else (l,)
        out[name] = codes.reshape(*shape, k // 2)
        out["sf" + name] = sf.reshape(*shape, k // 16)
        scales[name] = g
    out["alpha"] = scales["A"] * scales["x"]     # one fp32 rounding, as the workload defines
    torch.cuda.synchronize()
    return out


def launch_timer(timer, state, capture_stream, modes):
    """(n, call) -> ms for n calls of call(i), each launching on state["stream"]:
    launched one by one ("stream") or as one replay of a HIP graph holding the
    n calls ("graph"); with both modes, the faster of the two."""
    def run(n, call):
        best = None
        for mode in modes:
            if mode == "stream":
                ms, _ = timer(n, call)
            else:
                g = capture_steps(timer.torch, n, call, state, capture_stream)
                g.replay()                           # untimed: uploads the graph
                timer.torch.cuda.synchronize()
                ms, _ = timer(1, lambda i: g.replay())
            best = ms if best is None else min(best, ms)
        return best
    return run


def flat_probe_gbs(torch, pd, timed, state, shared):
    """The library's flat streaming-read probe over 1 GiB (measured once per run)."""
    if "flat_probe_gbs" not in shared:
        pbytes = 1 << 30
        pbuf = torch.empty(pbytes, dtype=torch.uint8, device="cuda")
        pbuf.fill_(1)
        sink = torch.empty(4096, dtype=torch.int32, device="cuda")
        for _ in range(3):
            pd.nvfp4_hbm_read_probe(pbuf, pbytes, sink, state["stream"])
        pn = 20
        pms = timed(pn, lambda i: pd.nvfp4_hbm_read_probe(pbuf, pbytes, sink, state["stream"]))
        shared["flat_probe_gbs"] = pbytes / (pms / pn * 1e-3) / 1e9
        del pbuf
        print(f"[bench] streaming-read probe (1 GiB): {shared['flat_probe_gbs']:.1f} GB/s", flush=True)
    return shared["flat_probe_gbs"]


def row_probe_gbs(torch, pd, timed, state, replicas, l, m, k):
    """The row-pattern read probe over every copy's A and sfA in turn: the read
    ceiling of the GEMV's load pattern for this weight, operands in HBM."""
    if k % 32 != 0:
        return None
    reps = len(replicas)
    rows = l * m
    sink = torch.empty(-(-rows // 14), dtype=torch.int32, device="cuda")
    nbytes = rows * (k // 2 + k // 16)
    for i in range(min(reps, 4)):
        pd.nvfp4_hbm_read_probe_rows(replicas[i]["A"], replicas[i]["sfA"], rows, k, sink,
                                     state["stream"])
    pn = max(8, 4 * reps)
    pms = timed(pn, lambda i: pd.nvfp4_hbm_read_probe_rows(replicas[i % reps]["A"],
                                                           replicas[i % reps]["sfA"], rows, k,
                                                           sink, state["stream"]))
    gbs = nbytes / (pms / pn * 1e-3) / 1e9
    print(f"[bench] row-pattern read probe over A and sfA ({nbytes / 1e6:.1f} MB, rotated): "
          f"{gbs:.1f} GB/s ({pms / pn * 1e3:.2f} us per read)", flush=True)
    return gbs


def flat_probe_same_size_gbs(torch, pd, timed, state, nbytes):
    """The flat streaming-read probe over contiguous copies of `nbytes` (the
    workload's A and sfA together), rotated over >= 1 GB (or over 64 copies,
    for operands below 16 MB): the read rate of a plain sequential read of
    this size, operands in HBM."""
    nb = -(-nbytes // 16) * 16
    reps = min(MAX_REPLICAS, max(2, -(-1_000_000_000 // nb)))   # at most 256 launches below
    bufs = [torch.ones(nb, dtype=torch.uint8, device="cuda") for _ in range(reps)]
    sink = torch.empty(4096, dtype=torch.int32, device="cuda")
    for i in range(reps):
        pd.nvfp4_hbm_read_probe(bufs[i], nb, sink, state["stream"])
    pn = max(8, 4 * reps)
    pms = timed(pn, lambda i: pd.nvfp4_hbm_read_probe(bufs[i % reps], nb, sink, state["stream"]))
    gbs = nb / (pms / pn * 1e-3) / 1e9
    del bufs
    print(f"[bench] flat read probe over {nb / 1e6:.1f} MB copies (rotated): {gbs:.1f} GB/s "
          f"({pms / pn * 1e3:.2f} us per read)", flush=True)
    return gbs


def bench_gemv(args, torch, np, pd, workloads, name=None, shared=None):
    shared = {} if shared is None else shared
    cfg = workloads.CONFIGS[name or args.config]
    l, m, k = cfg.l, cfg.m, cfg.k
    nbytes = cfg.bytes_moved
    print(f"[bench] workload {cfg.name}: l={l} m={m} k={k}, {nbytes} bytes per step", flush=True)

    if cfg.kind == "integer":
        raw = None
        ops = workloads.for_config(cfg)
        base = {n: torch.from_numpy(np.ascontiguousarray(v)).cuda() for n, v in ops.items()}
    else:
        raw = workloads.gaussian_bf16(l, m, k, seed=cfg.seed)
        base = quantize_gaussian_on_device(torch, np, pd, raw, l, m, k)
        print("[bench] Gaussian operands quantised on the device (not timed)", flush=True)
    replicas, reps = replicate(torch, base, nbytes, args.replicas)
    c = torch.empty((l, m), dtype=torch.int16, device="cuda")
    stream = torch.cuda.current_stream()
    state = {"stream": stream.cuda_stream}
    timer = Timer(torch, stream)

    tuned = args.variant or args.ksplit
    tuning = {"variant": args.variant, "ksplit": args.ksplit}
    plan, ws_bytes = pd.nvfp4_gemv_plan(l, m, k, aligned=True, tuning=tuning if tuned else None)
    ws = torch.empty(max(ws_bytes, 4), dtype=torch.uint8, device="cuda")
    capture_stream = torch.cuda.Stream()
    if not tuned and ws_bytes:
        # the library's split-K workspace, sized before any capture on both streams
        pd.nvfp4_workspace_reserve(ws_bytes, stream)
        pd.nvfp4_workspace_reserve(ws_bytes, capture_stream)

    def step(i):
        r = replicas[i % reps]
        if tuned:
            pd.nvfp4_gemv_launch_tuned(r["A"], r["sfA"], r["x"], r["sfx"], r["alpha"], c, l, m, k,
                                       tuning, ws, ws_bytes, state["stream"])
        else:
            pd.nvfp4_gemv_launch(r["A"], r["sfA"], r["x"], r["sfx"], r["alpha"], c, l, m, k,
                                 state["stream"])

    footprint = reps * nbytes
    operands = ("HBM (rotated over >= 1 GB of copies)" if footprint >= 1_000_000_000 else
                f"rotated over {reps} copies ({footprint / 1e6:.1f} MB, cache-resident: "
                f"launch-bound workload)")
    print(f"[bench] plan path={plan.path} variant={plan.variant} ksplit={plan.ksplit}; "
          f"{reps} replicas ({footprint / 1e9:.3f} GB)", flush=True)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    # the K steps launched one by one from the host
    ms_total, wall = timer(args.steps, step)
    stream_us = ms_total / args.steps * 1e3
    enqueue_us = timer.enqueue_s / args.steps * 1e6
    print(f"[bench] gemv, stream launches: {args.steps} steps: {stream_us:.2f} us/step "
          f"({nbytes / stream_us / 1e3:.1f} GB/s), host enqueue {enqueue_us:.2f} us/step", flush=True)
    graph_us = None
    if not args.trace_cold or args.launch == "graph":
        g = capture_steps(torch, args.steps, step, state, capture_stream)
        g.replay()                                   # untimed: uploads the graph
        torch.cuda.synchronize()
        ms_total, wall = timer(1, lambda i: g.replay())
        graph_us = ms_total / args.steps * 1e3
        print(f"[bench] gemv, one graph replay of {args.steps} steps: {graph_us:.2f} us/step "
              f"({nbytes / graph_us / 1e3:.1f} GB/s)", flush=True)
    us_step = graph_us if args.launch == "graph" else stream_us
    ms_step = us_step * 1e-3
    gbs = nbytes / (ms_step * 1e-3) / 1e9
    print(f"[bench] gemv {cfg.name}: {us_step:.2f} us/step, {gbs:.1f} GB/s "
          f"({100 * gbs / HBM_PEAK_GBS:.1f}% of peak)", flush=True)
    # the last timed call's output, before anything else writes c
    got = c.cpu().numpy().view(np.uint16).copy()

    warm_gbs = single = probe_gbs = probe_rows = probe_flat = None
    if not args.trace_cold:
        nw = min(args.steps, 500)
        warm_ms = launch_timer(timer, state, capture_stream, (args.launch,))(nw, lambda i: step(0))
        # the read probes' ceiling: each timed both ways, the faster counts
        timed = launch_timer(timer, state, capture_stream, ("stream", "graph"))
        warm_gbs = nbytes / (warm_ms / nw * 1e-3) / 1e9
        print(f"[bench] cache-resident (same buffers every step): {warm_gbs:.1f} GB/s", flush=True)

        ebytes = 512 << 20
        ebuf = torch.ones(ebytes, dtype=torch.uint8, device="cuda")
        esink = torch.empty(4096, dtype=torch.int32, device="cuda")
        single = single_launch_percentiles(
            torch, stream, step, args.single_launches,
            evict=lambda i: pd.nvfp4_hbm_read_probe(ebuf, ebytes, esink, state["stream"]))
        del ebuf
        if single:
            print(f"[bench] single launches after a 512 MiB streaming read: p10 {single['p10']} us, "
                  f"p50 {single['p50']} us, p90 {single['p90']} us", flush=True)
        if not args.no_probe:
            probe_gbs = flat_probe_gbs(torch, pd, timed, state, shared)
            probe_rows = row_probe_gbs(torch, pd, timed, state, replicas, l, m, k)
            probe_flat = flat_probe_same_size_gbs(torch, pd, timed, state,
                                                  l * m * (k // 2 + k // 16))
    run_copies(torch, args.copy_mib)

    cpu = None
    quantised = None
    if not args.no_cpu_baseline and not args.trace_cold:
        from oracle import reference as ref

        if raw is not None:
            # the oracle's own quantisation of the same draws, byte for byte
            from oracle import quantize as oq

            ops = oq.gaussian_operands(raw, l, m, k)
            quantised = all(np.array_equal(base[n].cpu().numpy().reshape(ops[n].shape), ops[n])
                            for n in ("A", "sfA", "x", "sfx")) and \
                np.array_equal(base["alpha"].cpu().numpy().view(np.uint32), ops["alpha"].view(np.uint32))
            print(f"[bench] device-quantised operands identical to the oracle's: {quantised}",
                  flush=True)
        threads = ref.default_threads()
        results = []
        t_med = cpu_time(lambda: results.append(ref.gemv(ops["A"], ops["sfA"], ops["x"], ops["sfx"],
                                                         ops["alpha"], l, m, k, nthreads=threads)))
        parity = parity_summary(np, got, results[-1])
        print(f"[bench] parity of the last timed call with the oracle: {parity}", flush=True)
        cpu = {"value": round(nbytes / t_med / 1e9, 4), "unit": "GB/s", "cores": threads,
               "kind": "oracle",
               "sample": f"the whole {cfg.name} workload (l={l}, m={m}, k={k}), median of 3 runs "
                         f"of {t_med:.3f}s, fp64 sums + fp32/fp16 epilogue, inputs in host memory",
               "seconds": round(t_med, 4),
               "elements_per_s_per_core": round(l * m * k / t_med / threads, 1),
               "parity": parity}
        if quantised is not None:
            cpu["quantised_operands_identical"] = quantised
        print(f"[bench] CPU oracle: {t_med:.3f}s per GEMV on {threads} threads", flush=True)

    out = {"metric": METRIC}
    out.update(common_fields(args, gbs, ms_step, "f32"))
    inputs = {"one": "integer-coded, alpha=1", "uniform": "integer-coded, alpha U[0.5,2]",
              "quantizer": "bf16 N(0,1) quantised on the device, alpha = gA*gx"}[cfg.alpha]
    out["config"] = {"workload": f"{cfg.name}: NVFP4 GEMV l={l} m={m} k={k}, {inputs} ({cfg.note})",
                     "l": l, "m": m, "k": k, "bytes_per_step": nbytes,
                     "replicas": reps, "operands": operands,
                     "launch": ("one HIP graph replay of the K steps" if args.launch == "graph"
                                else "K stream launches"),
                     "plan": {"path": plan.path, "variant": plan.variant, "ksplit": plan.ksplit}}
    out["timing_us"] = {"graph_replay": None if graph_us is None else round(graph_us, 3),
                        "stream_launches": round(stream_us, 3),
                        "host_enqueue_per_launch": round(enqueue_us, 3)}
    # the GEMV's rate against the best read probe of its own size, in the same run
    best = max([g for g in (probe_rows, probe_flat) if g] or [0.0]) or None
    out["roofline"] = roofline(gbs, recorded_traffic(cfg.name), kernel=plan_kernel_name(pd, plan),
                               probe_read_gbs=probe_gbs, probe_rows_same_size_gbs=probe_rows,
                               probe_flat_same_size_gbs=probe_flat,
                               frac_of_best_same_size_probe=(gbs / best) if best else None,
                               cache_resident_gbs=warm_gbs)
    out["single_launch_us"] = single
    out["cpu_baseline"] = with_speedup(cpu, gbs)
    if cpu is not None:
        out["parity"] = cpu["parity"]
    return out


def mma_kernel_name(pd, plan, packed):
    """The kernel a small-N or grouped plan runs, by its committed-profile
    name: matrix cores on packed weights, or by the variant's form."""
    if packed:
        return "mma_stream_packed"
    if plan.path != pd.NVFP4_GEMV_PATH_FAST:
        return "mma_generic"
    form = pd.nvfp4_mma_variant_form(plan.variant)
    return {pd.NVFP4_MMA_FORM_VALU_TILES: "vec_tile",
            pd.NVFP4_MMA_FORM_LDS_STAGED: "mma_lds",
            pd.NVFP4_MMA_FORM_LDS_VECTOR_REGS: "mma_lds"}.get(form, "mma_stream")


def plan_kernel_name(pd, plan):
    """The GEMV kernel a plan launches, as the profiles name it."""
    if plan.path != pd.NVFP4_GEMV_PATH_FAST:
        return "gemv_generic"
    r, u, w, xs = pd.nvfp4_gemv_variant_info(plan.variant)
    if xs == 3:
        return f"gemv_tile<{w}, {r}>"
    return f"{('gemv_fast', 'gemv_fastp', 'gemv_fastg')[xs]}<{r}, {u}, {w}>"


# ------------------------------------------------------------------------------ quantiser
def bench_quantize(args, torch, np, pd, workloads):
    cfg = workloads.ACT_CONFIGS[args.act_config]
    rows, d = cfg.rows, cfg.d
    nbytes = cfg.bytes_moved
    print(f"[bench] activation workload {cfg.name}: rows={rows} d={d}, {nbytes} bytes per step, "
          f"rule {args.rule}", flush=True)
    vals = workloads.activation_bf16(cfg)
    # the global scale a warm-up pass would cache: amax / (6 * 448) per row
    gs = (np.maximum(np.abs(vals).max(axis=1), np.float32(1e-8)) / np.float32(2688.0)).astype(np.float32)
    base = {"x": torch.from_numpy(workloads.bf16_bits(vals).view(np.int16)).cuda(),
            "gs": torch.from_numpy(gs).cuda(),
            "q": torch.empty((rows, d // 2), dtype=torch.uint8, device="cuda"),
            "sf": torch.empty((rows, d // 16), dtype=torch.uint8, device="cuda")}
    replicas, reps = replicate(torch, base, nbytes, args.replicas)
    stream = torch.cuda.current_stream()
    state = {"stream": stream.cuda_stream}
    capture_stream = torch.cuda.Stream()
    timer = Timer(torch, stream)

    def step(i):
        r = replicas[i % reps]
        pd.nvfp4_quantize_activation(r["x"], r["gs"], 1 if rows > 1 else 0, r["q"], r["sf"], rows, d,
                                     args.rule, state["stream"])

    print(f"[bench] {reps} replicas ({reps * nbytes / 1e9:.2f} GB)", flush=True)
    ms_step, gbs, timing = timed_steps(args, timer, step, nbytes, "quantize", state, capture_stream)
    run_copies(torch, args.copy_mib)

    cpu = None
    if not args.no_cpu_baseline:
        from oracle import quantize as oq

        sample = min(rows, 256)
        with np.errstate(all="ignore"):
            t_med = cpu_time(lambda: oq.quantize_with_scale(vals[:sample], gs[:sample], args.rule))
        sbytes = nbytes * sample / rows
        cpu = {"value": round(sbytes / t_med / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
               "sample": f"{sample} of the {rows} rows (d={d}), median of 3 runs of {t_med:.3f}s, "
                         f"numpy fp32 steps, one thread"}
        print(f"[bench] CPU oracle: {t_med:.3f}s for {sample} rows", flush=True)

    out = {"metric": "achieved HBM GB/s of the BF16 -> NVFP4 activation quantiser (us/call alongside)"}
    out.update(common_fields(args, gbs, ms_step, "f32"))
    out["config"] = {"workload": f"{cfg.name}: quantise rows={rows} d={d} bf16 N(0,1), per-row "
                                 f"global scale, rule {args.rule} ({cfg.note})",
                     "rows": rows, "d": d, "rule": args.rule, "bytes_per_step": nbytes,
                     "replicas": reps, "operands": "HBM (rotated over >= 1 GB of copies)"}
    out["roofline"] = roofline(gbs, recorded_traffic(cfg.name, "quantize_blocks"))
    out["config"]["launch"] = launch_label(args)
    out["timing_us"] = timing
    out["cpu_baseline"] = with_speedup(cpu, gbs)
    return out


# ------------------------------------------------------------- GEMV fed by a bf16 activation
def bench_bf16x(args, torch, np, pd, workloads):
    cfg = workloads.CONFIGS["decode" if args.config == "all" else args.config]
    if cfg.kind != "integer":
        print(f"{cfg.name} is not an integer-coded workload", file=sys.stderr)
        return None
    l, m, k = cfg.l, cfg.m, cfg.k
    # A + sfA + bf16 x in; c, the quantised x, its scales and alpha out
    nbytes = l * m * k // 2 + l * m * k // 16 + 2 * l * k + 2 * l * m + l * k // 2 + l * k // 16 + 8 * l
    print(f"[bench] workload {cfg.name} with a bf16 activation: l={l} m={m} k={k}, {nbytes} bytes "
          f"per step, rule {args.rule}", flush=True)
    ops = workloads.for_config(cfg)
    xv = workloads.gaussian_bf16(l, 1, k, seed=cfg.seed + 1)["x"]
    xs = (np.maximum(np.abs(xv).max(axis=1), np.float32(1e-8)) / np.float32(2688.0)).astype(np.float32)
    base = {"A": torch.from_numpy(ops["A"]).cuda(), "sfA": torch.from_numpy(ops["sfA"]).cuda(),
            "x": torch.from_numpy(workloads.bf16_bits(xv).view(np.int16)).cuda(),
            "xs": torch.from_numpy(xs).cuda(),
            "xq": torch.empty((l, k // 2), dtype=torch.uint8, device="cuda"),
            "sfx": torch.empty((l, k // 16), dtype=torch.uint8, device="cuda"),
            "alpha": torch.empty(l, dtype=torch.float32, device="cuda")}
    replicas, reps = replicate(torch, base, nbytes, args.replicas)
    c = torch.empty((l, m), dtype=torch.int16, device="cuda")
    stream = torch.cuda.current_stream()
    state = {"stream": stream.cuda_stream}
    capture_stream = torch.cuda.Stream()
    timer = Timer(torch, stream)
    _, ws_bytes = pd.nvfp4_gemv_plan(l, m, k, aligned=True)
    if ws_bytes:
        # the GEMV's split-K workspace, sized before any capture on both streams
        pd.nvfp4_workspace_reserve(ws_bytes, stream)
        pd.nvfp4_workspace_reserve(ws_bytes, capture_stream)

    def step(i):
        r = replicas[i % reps]
        pd.nvfp4_gemv_bf16x_launch(r["A"], r["sfA"], None, r["x"], r["xs"], args.rule, r["xq"],
                                   r["sfx"], r["alpha"], c, l, m, k, state["stream"])

    print(f"[bench] {reps} replicas ({reps * nbytes / 1e9:.2f} GB)", flush=True)
    ms_step, gbs, timing = timed_steps(args, timer, step, nbytes, "gemv_bf16x", state, capture_stream)
    run_copies(torch, args.copy_mib)

    cpu = None
    if not args.no_cpu_baseline:
        from oracle import quantize as oq
        from oracle import reference as ref

        threads = ref.default_threads()
        with np.errstate(all="ignore"):
            t_med = cpu_time(lambda: oq.activation_gemv(ops["A"], ops["sfA"], None, xv, xs, args.rule,
                                                        l, m, k))
        cpu = {"value": round(nbytes / t_med / 1e9, 4), "unit": "GB/s", "cores": threads,
               "kind": "oracle",
               "sample": f"the whole {cfg.name} workload with a bf16 activation, median of 3 runs of "
                         f"{t_med:.3f}s (numpy quantiser, C fp64 GEMV on {threads} threads)"}
        print(f"[bench] CPU oracle: {t_med:.3f}s per call", flush=True)

    out = {"metric": "achieved HBM GB/s of the NVFP4 GEMV fed by a bf16 activation (quantiser + "
                     "GEMV per call)"}
    out.update(common_fields(args, gbs, ms_step, "f32"))
    out["config"] = {"workload": f"{cfg.name}: bf16 x quantised (rule {args.rule}) then NVFP4 GEMV "
                                 f"l={l} m={m} k={k}, integer-coded A ({cfg.note})",
                     "l": l, "m": m, "k": k, "rule": args.rule, "bytes_per_step": nbytes,
                     "replicas": reps, "operands": "HBM (rotated over >= 1 GB of copies)"}
    out["roofline"] = roofline(gbs, None)
    out["config"]["launch"] = launch_label(args)
    out["timing_us"] = timing
    out["cpu_baseline"] = with_speedup(cpu, gbs)
    return out


# ------------------------------------------------------------------------- small-N GEMM
def bench_smalln(args, torch, np, pd, workloads):
    cfg = workloads.SMALLN_CONFIGS[args.smalln_config]
    l, m, n, k = cfg.l, cfg.m, cfg.n, cfg.k
    out_type = pd.NVFP4_OUT_F16 if args.out_type is None else args.out_type
    nbytes = cfg.bytes_moved
    print(f"[bench] small-N workload {cfg.name}: l={l} m={m} n={n} k={k}, {nbytes} bytes per step",
          flush=True)
    ops = workloads.smalln_operands(cfg)
    base = {name: torch.from_numpy(np.ascontiguousarray(v)).cuda() for name, v in ops.items()}
    replicas, reps = replicate(torch, base, nbytes, args.replicas)
    c = torch.empty((l, m, n), dtype=torch.int16, device="cuda")
    stream = torch.cuda.current_stream()
    state = {"stream": stream.cuda_stream}
    capture_stream = torch.cuda.Stream()
    timer = Timer(torch, stream)
    tuned = args.variant or args.ksplit
    tuning = {"variant": args.variant, "ksplit": args.ksplit}
    plan, ws_bytes = pd.nvfp4_gemm_smalln_plan(l, m, n, k, tuning=tuning if tuned else None)
    ws = torch.empty(max(ws_bytes, 4), dtype=torch.uint8, device="cuda")
    if not tuned and ws_bytes:
        # the library's split-K workspace, sized before any capture on both streams
        pd.nvfp4_workspace_reserve(ws_bytes, stream)
        pd.nvfp4_workspace_reserve(ws_bytes, capture_stream)
    if args.packed:
        pack_replicas(torch, pd, replicas, "A", "sfA", l, m, k)

    def step(i):
        r = replicas[i % reps]
        if args.packed:
            pd.nvfp4_gemm_smalln_launch_packed(r["A_packed"], r["sfA_packed"], r["B"], r["sfB"],
                                               r["alpha"], c, l, m, n, k, out_type,
                                               tuning if tuned else None, state["stream"])
        elif tuned:
            pd.nvfp4_gemm_smalln_launch_tuned(r["A"], r["sfA"], r["B"], r["sfB"], r["alpha"], c, l, m,
                                              n, k, out_type, tuning, ws, ws_bytes, state["stream"])
        else:
            pd.nvfp4_gemm_smalln_launch(r["A"], r["sfA"], r["B"], r["sfB"], r["alpha"], c, l, m, n, k,
                                        out_type, state["stream"])

    print(f"[bench] plan path={plan.path} variant={plan.variant} ksplit={plan.ksplit}"
          f"{' (row-major plan; packed weights)' if args.packed else ''}; "
          f"{reps} replicas ({reps * nbytes / 1e9:.2f} GB)", flush=True)
    ms_step, gbs, timing = timed_steps(args, timer, step, nbytes, "smalln", state, capture_stream)
    run_copies(torch, args.copy_mib)

    cpu = None
    if not args.no_cpu_baseline:
        from oracle import multi
        from oracle import reference as ref

        threads = ref.default_threads()
        fmt = "bf16" if out_type == pd.NVFP4_OUT_BF16 else "f16"
        t_med = cpu_time(lambda: multi.gemm_smalln(ops["A"], ops["sfA"], ops["B"], ops["sfB"],
                                                   ops["alpha"], l, m, n, k, fmt, nthreads=threads))
        cpu = {"value": round(nbytes / t_med / 1e9, 4), "unit": "GB/s", "cores": threads,
               "kind": "oracle",
               "sample": f"the whole {cfg.name} workload, median of 3 runs of {t_med:.3f}s "
                         f"(C fp64 sums, one vector at a time, {threads} threads)"}
        print(f"[bench] CPU oracle: {t_med:.3f}s per call", flush=True)

    flops = 2 * l * m * n * k
    out = {"metric": "achieved HBM GB/s of the NVFP4 small-N block-scaled GEMM (us/call alongside)"}
    out.update(common_fields(args, gbs, ms_step, "f32"))
    out["config"] = {"workload": f"{cfg.name}: NVFP4 GEMM l={l} m={m} n={n} k={k}, integer-coded, "
                                 f"alpha U[0.5,2] ({cfg.note})",
                     "l": l, "m": m, "n": n, "k": k, "out": "bf16" if out_type else "f16",
                     "bytes_per_step": nbytes, "replicas": reps,
                     "operands": "HBM (rotated over >= 1 GB of copies)",
                     "plan": {"path": plan.path, "variant": plan.variant, "ksplit": plan.ksplit},
                     "weights": "packed once by nvfp4_mma_pack_weight (not timed)" if args.packed
                                else "row-major"}
    if args.packed:
        del out["config"]["plan"]
    kernel = mma_kernel_name(pd, plan, args.packed)
    extra = {} if kernel == "vec_tile" else {"mfma_tflops": flops / (ms_step * 1e-3) / 1e12}
    out["roofline"] = roofline(gbs, recorded_traffic(cfg.name, kernel), kernel=kernel, **extra)
    out["config"]["launch"] = launch_label(args)
    out["timing_us"] = timing
    out["cpu_baseline"] = with_speedup(cpu, gbs)
    return out


# ------------------------------------------------------------------- grouped (MoE) GEMV
def bench_grouped(args, torch, np, pd, workloads):
    cfg = workloads.MOE_CONFIGS[args.moe_config]
    out_type = pd.NVFP4_OUT_BF16 if args.out_type is None else args.out_type
    ops = workloads.moe_operands(cfg)
    E, n, k, T = cfg.experts, cfg.n, cfg.k, cfg.tokens
    nbytes = workloads.moe_bytes_moved(cfg, ops["offsets"])
    active = int((np.diff(np.concatenate([[0], ops["offsets"]])) > 0).sum())
    print(f"[bench] grouped workload {cfg.name}: {E} experts ({active} with tokens) of n={n} k={k}, "
          f"{T} tokens, {nbytes} bytes per step", flush=True)
    base = {name: torch.from_numpy(np.ascontiguousarray(v)).cuda() for name, v in ops.items()}
    replicas, reps = replicate(torch, base, nbytes, args.replicas)
    c = torch.empty((T, n), dtype=torch.int16, device="cuda")
    stream = torch.cuda.current_stream()
    state = {"stream": stream.cuda_stream}
    capture_stream = torch.cuda.Stream()
    timer = Timer(torch, stream)
    tuning = {"variant": args.variant}
    if args.packed:
        pack_replicas(torch, pd, replicas, "W", "sfW", E, n, k)

    def step(i):
        r = replicas[i % reps]
        if args.packed:
            pd.nvfp4_grouped_gemv_launch_packed(r["X"], r["sfX"], r["W_packed"], r["sfW_packed"],
                                                r["offsets"], r["gs_x"], r["gs_w"], c, T, E, n, k,
                                                out_type, tuning, state["stream"])
        else:
            pd.nvfp4_grouped_gemv_launch_tuned(r["X"], r["sfX"], r["W"], r["sfW"], r["offsets"],
                                               r["gs_x"], r["gs_w"], c, T, E, n, k, out_type, tuning,
                                               state["stream"])

    print(f"[bench] variant={args.variant or 'default'}; {reps} replicas "
          f"({reps * nbytes / 1e9:.2f} GB)", flush=True)
    ms_step, gbs, timing = timed_steps(args, timer, step, nbytes, "grouped", state, capture_stream)
    run_copies(torch, args.copy_mib)

    cpu = None
    if not args.no_cpu_baseline:
        from oracle import multi
        from oracle import reference as ref

        threads = ref.default_threads()
        fmt = "bf16" if out_type == pd.NVFP4_OUT_BF16 else "f16"
        t_med = cpu_time(lambda: multi.grouped_gemv(ops["X"], ops["sfX"], ops["W"], ops["sfW"],
                                                    ops["offsets"], ops["gs_x"], ops["gs_w"], T, E,
                                                    n, k, fmt, nthreads=threads))
        cpu = {"value": round(nbytes / t_med / 1e9, 4), "unit": "GB/s", "cores": threads,
               "kind": "oracle",
               "sample": f"the whole {cfg.name} workload, median of 3 runs of {t_med:.3f}s "
                         f"(C fp64 sums token by token, {threads} threads)"}
        print(f"[bench] CPU oracle: {t_med:.3f}s per call", flush=True)

    out = {"metric": "achieved HBM GB/s of the NVFP4 grouped (MoE) GEMV (us/call alongside)"}
    out.update(common_fields(args, gbs, ms_step, "f32"))
    out["config"] = {"workload": f"{cfg.name}: {E} experts of n={n} k={k}, {T} routed tokens "
                                 f"(multinomial counts, {active} experts active), integer-coded "
                                 f"({cfg.note})",
                     "experts": E, "active_experts": active, "n": n, "k": k, "tokens": T,
                     "out": "bf16" if out_type else "f16", "bytes_per_step": nbytes,
                     "replicas": reps, "operands": "HBM (rotated over >= 1 GB of copies)",
                     "weights": "packed once by nvfp4_mma_pack_weight (not timed)" if args.packed
                                else "row-major"}
    plan = pd.nvfp4_grouped_gemv_plan(E, n, k, T, packed=args.packed,
                                      tuning={"variant": args.variant} if args.variant else None)
    kernel = mma_kernel_name(pd, plan, args.packed)
    out["config"]["plan"] = {"path": plan.path, "variant": plan.variant,
                             "rows_per_block": plan.rows_per_block}
    out["roofline"] = roofline(gbs, recorded_traffic(cfg.name, kernel), kernel=kernel)
    out["config"]["launch"] = launch_label(args)
    out["timing_us"] = timing
    out["cpu_baseline"] = with_speedup(cpu, gbs)
    return out


def main(argv=None) -> int:
    args = parse_args(argv)
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the NVFP4 GEMV runs on a single MI355X and the "
              "library has no multi-GPU path (the design notes describe sharding along M). "
              "Run with --gpus 1.", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import precision_decode_amd as pd
    import workloads

    if not os.path.exists(pd.LIB_PATH):
        from precision_decode_amd import build as lib_build
        lib_build.build()
    pd.load()
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    torch.cuda.set_device(0)

    if args.path == "gemv":
        names = GEMV_ORDER if args.config == "all" else (args.config,)
        shared = {}
        for name in names:
            out = bench_gemv(args, torch, np, pd, workloads, name, shared)
            print(json.dumps(out), flush=True)
            torch.cuda.synchronize()
            torch.cuda.empty_cache()
        return 0
    fn = {"quantize": bench_quantize, "gemv_bf16x": bench_bf16x,
          "smalln": bench_smalln, "grouped": bench_grouped}[args.path]
    out = fn(args, torch, np, pd, workloads)
    if out is None:
        return 2
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
