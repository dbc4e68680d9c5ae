"""Ahead-of-time build of the HIP library for gfx950.

``python -m precision_decode_amd.build`` compiles the HIP sources under
``csrc/`` with hipcc into ``precision_decode_amd/libnvfp4_gemv.so`` (in the source tree, so the
built library travels with the tree).  Packed-FP32 VALU instructions are
disabled for device code; floating-point contraction is off so every multiply
and add rounds where the source says it does.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRCS = [os.path.join(HERE, "csrc", n) for n in ("nvfp4_gemv.hip", "nvfp4_quantize.hip", "nvfp4_mma.hip")]
LIB = os.path.join(HERE, "libnvfp4_gemv.so")
INCLUDE = os.path.join(ROOT, "include")
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    return "hipcc"


def command(out: str) -> list:
    return [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
            "-ffp-contract=off", "-Wall", "-Wextra",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", INCLUDE, *SRCS, "-o", out]


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = command(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the device-only feature flag; drop that line.
    noise = "is not a recognized feature for this target"
    err = "\n".join(line for line in res.stderr.splitlines() if noise not in line)
    if res.returncode != 0:
        sys.stderr.write(err + "\n")
        raise RuntimeError(f"hipcc failed with status {res.returncode}")
    if err.strip() and verbose:
        sys.stderr.write(err + "\n")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
