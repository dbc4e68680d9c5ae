"""Host code under the address and undefined-behaviour sanitizers (no GPU).

* ``tests/host/plan_check.cpp`` compiles the library's host logic
  (``precision_decode_amd/csrc/gemv_plan.h``: validation, launch plan, and the
  order in which an entry point validates, plans, takes its workspace and
  launches) with g++ and runs it against a mock backend that fails the device
  query, the workspace allocation and the launch on purpose: the statuses are
  DEVICE, WORKSPACE and LAUNCH, and invalid calls never reach the backend.
* ``tests/host/mma_plan_check.cpp`` compiles the small-N GEMM and grouped
  GEMV plan (``precision_decode_amd/csrc/mma_plan.h``: shape rules, variants,
  defaults, launch plan) and checks 200000 random shapes and tunings against
  what the kernels assume, and the default rules.
* ``tests/host/oracle_check.c`` compiles the oracle's C sums
  (``oracle/nvfp4_ref.c``) with gcc and runs them on exact-size buffers.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HOST = os.path.join(ROOT, "tests", "host")
SAN = ["-O1", "-g", "-Wall", "-Wextra", "-Werror", "-fsanitize=address,undefined",
       "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
           UBSAN_OPTIONS="print_stacktrace=1")


def build_and_run(cmd, exe):
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-4000:]
    run = subprocess.run([exe], capture_output=True, text=True, env=ENV, timeout=120)
    return run


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_plan_and_orchestration_under_sanitizers(tmp_path):
    exe = str(tmp_path / "plan_check")
    cmd = ["g++", "-std=c++17", *SAN, "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(ROOT, "precision_decode_amd", "csrc"),
           os.path.join(HOST, "plan_check.cpp"), "-o", exe]
    run = build_and_run(cmd, exe)
    assert run.returncode == 0 and "plan_check ok" in run.stdout, run.stdout + run.stderr


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_mma_plan_under_sanitizers(tmp_path):
    exe = str(tmp_path / "mma_plan_check")
    cmd = ["g++", "-std=c++17", *SAN, "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(ROOT, "precision_decode_amd", "csrc"),
           os.path.join(HOST, "mma_plan_check.cpp"), "-o", exe]
    run = build_and_run(cmd, exe)
    assert run.returncode == 0 and "mma_plan_check ok" in run.stdout, run.stdout + run.stderr


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_sums_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_check")
    cmd = ["gcc", "-std=c11", *SAN, "-fopenmp", "-ffp-contract=off",
           os.path.join(ROOT, "oracle", "nvfp4_ref.c"), os.path.join(HOST, "oracle_check.c"),
           "-o", exe, "-lm"]
    run = build_and_run(cmd, exe)
    assert run.returncode == 0 and "oracle_check ok" in run.stdout, run.stdout + run.stderr
