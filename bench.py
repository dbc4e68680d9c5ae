#!/usr/bin/env python3
"""Throughput of the NVFP4 block-scaled batched GEMV on one MI355X.

One step = one call of the GEMV (all of its kernels) on one batch of inputs.
The default workload is the decode-style single large weight: l=1, m=7168,
k=16384, integer-coded (nibbles uniform over all 16 E2M1 codes, block scales
from {0, 1, 2}), alpha = 1.  Its 66 MB footprint fits in MI355X's 256 MB
Infinity Cache, so the timed loop rotates over enough device copies of the
inputs (>= 1 GB together) that every step reads its operands from HBM; a
cache-resident ("warm") figure is reported separately and labelled as such.

Prints one JSON line:
  value        algorithmic bytes per step (A + sfA + x + sfx + c) / time, GB/s
  roofline     the same rate against the 8 TB/s HBM peak, the kernel's HBM
               traffic from rocprofv3 counters when they were taken on this
               kernel source, and the achievable read rate of a plain
               streaming-read probe measured in the same run
  cpu_baseline the CPU oracle (plain C, fp64, OpenMP over rows) on the same
               workload on this host's cores

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--config decode]
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
KERNEL_SRC = os.path.join(ROOT, "precision_decode_amd", "csrc", "nvfp4_gemv.hip")
PROFILES = os.path.join(ROOT, "profiles")


def parse_args(argv=None):
    p = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=2000)
    p.add_argument("--warmup", type=int, default=100)
    p.add_argument("--config", default="decode",
                   help="integer-coded workload name from workloads.CONFIGS")
    p.add_argument("--replicas", type=int, default=0,
                   help="device copies of the inputs to rotate over (0: enough for >= 1 GB)")
    p.add_argument("--variant", type=int, default=0, help="fast-kernel variant (0 = default plan)")
    p.add_argument("--ksplit", type=int, default=0, help="K split (0 = default plan)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-probe", action="store_true")
    p.add_argument("--copy-mib", type=int, default=0,
                   help="after timing, run 4 plain device copies of this many MiB (the "
                        "known-size reference for HBM byte counters)")
    return p.parse_args(argv)


def kernel_source_hash() -> str:
    with open(KERNEL_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def recorded_traffic(config: str):
    """HBM bytes per launch from a committed counter summary, if it was taken
    on the current kernel source; otherwise None."""
    path = os.path.join(PROFILES, f"gemv_fast_{config}_hbm_counters.txt")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    h = re.search(r"^kernel_source_sha256_16:\s*(\w+)", text, re.M)
    t = re.search(r"^hbm_bytes_per_launch:\s*([0-9.eE+]+)", text, re.M)
    if not h or not t or h.group(1) != kernel_source_hash():
        return None
    return float(t.group(1))


def main(argv=None) -> int:
    args = parse_args(argv)
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the NVFP4 GEMV runs on a single MI355X and this "
              "build has no multi-GPU path (sharding along M is described in DESIGN.md). "
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

    cfg = workloads.CONFIGS[args.config]
    if cfg.kind != "integer":
        print(f"{cfg.name} is not an integer-coded workload; bench it with an integer config",
              file=sys.stderr)
        return 2
    l, m, k = cfg.l, cfg.m, cfg.k
    nbytes = cfg.bytes_moved
    print(f"[bench] workload {cfg.name}: l={l} m={m} k={k}, {nbytes} bytes per step", flush=True)

    ops = workloads.for_config(cfg)
    base = {n: torch.from_numpy(np.ascontiguousarray(v)).cuda() for n, v in ops.items()}
    reps = args.replicas or max(1, -(-1_000_000_000 // nbytes))
    replicas = [base] + [{n: t.clone() for n, t in base.items()} for _ in range(reps - 1)]
    c = torch.empty((l, m), dtype=torch.int16, device="cuda")
    stream = torch.cuda.current_stream()
    sptr = stream.cuda_stream

    tuned = args.variant or args.ksplit
    tuning = {"variant": args.variant, "ksplit": args.ksplit}
    plan, ws_bytes = pd.nvfp4_gemv_plan(l, m, k, aligned=True, tuning=tuning if tuned else None)
    ws = torch.empty(max(ws_bytes, 4), dtype=torch.uint8, device="cuda")

    def step(i):
        r = replicas[i % reps]
        if tuned:
            pd.nvfp4_gemv_launch_tuned(r["A"], r["sfA"], r["x"], r["sfx"], r["alpha"], c, l, m, k,
                                       tuning, ws, ws_bytes, sptr)
        else:
            pd.nvfp4_gemv_launch(r["A"], r["sfA"], r["x"], r["sfx"], r["alpha"], c, l, m, k, sptr)

    def timed(n, fn):
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        start.record(stream)
        for i in range(n):
            fn(i)
        end.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        return start.elapsed_time(end), wall

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    print(f"[bench] warmup {args.warmup} done; plan path={plan.path} variant={plan.variant} "
          f"ksplit={plan.ksplit}; {reps} replicas ({reps * nbytes / 1e9:.2f} GB)", flush=True)

    ms_total, wall = timed(args.steps, step)
    ms_step = ms_total / args.steps
    gbs = nbytes / (ms_step * 1e-3) / 1e9
    print(f"[bench] {args.steps} steps: {ms_step * 1e3:.2f} us/step, {gbs:.1f} GB/s "
          f"({100 * gbs / HBM_PEAK_GBS:.1f}% of peak), host wall {wall:.3f}s", flush=True)

    warm_ms, _ = timed(min(args.steps, 500), lambda i: step(0))
    warm_gbs = nbytes / (warm_ms / min(args.steps, 500) * 1e-3) / 1e9
    print(f"[bench] cache-resident (same buffers every step): {warm_gbs:.1f} GB/s", flush=True)

    probe_gbs = probe_ws_gbs = None
    if not args.no_probe:
        pbytes = 1 << 30
        pbuf = torch.empty(pbytes, dtype=torch.uint8, device="cuda")
        pbuf.fill_(1)
        sink = torch.empty(4096, dtype=torch.int32, device="cuda")
        for _ in range(3):
            pd.nvfp4_hbm_read_probe(pbuf, pbytes, sink, sptr)
        pn = 20
        pms, _ = timed(pn, lambda i: pd.nvfp4_hbm_read_probe(pbuf, pbytes, sink, sptr))
        probe_gbs = pbytes / (pms / pn * 1e-3) / 1e9
        del pbuf
        print(f"[bench] streaming-read probe (1 GiB): {probe_gbs:.1f} GB/s", flush=True)
        # the same probe over each copy's A in turn: the achievable read rate
        # for a read of this workload's size, operands in HBM
        abytes = replicas[0]["A"].numel()
        pn = 4 * reps
        pms, _ = timed(pn, lambda i: pd.nvfp4_hbm_read_probe(replicas[i % reps]["A"], abytes, sink, sptr))
        probe_ws_gbs = abytes / (pms / pn * 1e-3) / 1e9
        print(f"[bench] streaming-read probe over A ({abytes / 1e6:.1f} MB, rotated): "
              f"{probe_ws_gbs:.1f} GB/s", flush=True)

    if args.copy_mib:
        src = torch.ones(args.copy_mib << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(4):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(f"[bench] ran 4 device copies of {args.copy_mib} MiB", flush=True)

    cpu = None
    if not args.no_cpu_baseline:
        from oracle import reference as ref

        threads = ref.default_threads()
        times = []
        for _ in range(3):
            t0 = time.perf_counter()
            ref.gemv(ops["A"], ops["sfA"], ops["x"], ops["sfx"], ops["alpha"], l, m, k, nthreads=threads)
            times.append(time.perf_counter() - t0)
        t_med = statistics.median(times)
        cpu = {"value": round(nbytes / t_med / 1e9, 4), "unit": "GB/s", "cores": threads,
               "kind": "oracle",
               "sample": f"the whole {cfg.name} workload (l={l}, m={m}, k={k}), median of 3 runs "
                         f"of {t_med:.3f}s, fp64 sums + fp32/fp16 epilogue, inputs in host memory"}
        print(f"[bench] CPU oracle: {t_med:.3f}s per GEMV on {threads} threads", flush=True)

    traffic = recorded_traffic(cfg.name)
    out = {
        "metric": "achieved HBM GB/s for the NVFP4 block-scaled batched GEMV (us/call and % of "
                  "MI355X peak alongside)",
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 6),
        "us_per_call": round(ms_step * 1e3, 3),
        "pct_of_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"{cfg.name}: NVFP4 GEMV l={l} m={m} k={k}, integer-coded, "
                               f"alpha=1 ({cfg.note})",
                   "l": l, "m": m, "k": k, "bytes_per_step": nbytes,
                   "replicas": reps, "operands": "HBM (rotated over >= 1 GB of copies)",
                   "plan": {"path": plan.path, "variant": plan.variant, "ksplit": plan.ksplit}},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4),
                     "traffic": traffic,
                     "probe_read_gbs": round(probe_gbs, 2) if probe_gbs else None,
                     "probe_read_same_size_gbs": round(probe_ws_gbs, 2) if probe_ws_gbs else None,
                     "cache_resident_gbs": round(warm_gbs, 2)},
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
