"""Builds the device checks under ``tests/device`` (hipcc for gfx950, in the
source tree next to their sources, so they travel with it).  They include the
library's device headers directly and are run by the GPU tests."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
CSRC = os.path.join(ROOT, "precision_decode_amd", "csrc")
CHECKS = ("quant_arith_check",)


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    return "hipcc"


def build() -> list:
    built = []
    for name in CHECKS:
        out = os.path.join(HERE, name)
        cmd = [hipcc(), "--offload-arch=gfx950", "-O3", "-std=c++17", "-ffp-contract=off",
               "-Wall", "-Wextra", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-I", os.path.join(ROOT, "include"), "-I", CSRC,
               os.path.join(HERE, name + ".hip"), "-o", out + ".tmp"]
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"hipcc failed for {name}:\n{res.stderr[-4000:]}")
        os.replace(out + ".tmp", out)
        built.append(out)
    return built


if __name__ == "__main__":
    for p in build():
        print(p)
