"""The quantiser's division-free quotients (``csrc/quant_arith.h``) against
IEEE division on the device, over the whole range in which its fast path
relies on them (``tests/device/quant_arith_check.hip``): every fp32 global
scale for the fp64 reciprocal, every bf16-by-fp32 significand pair for x/g,
and every quotient by a nonzero E4M3 block scale that decides an E2M1 code.
The check is a separate program started as a child process."""
import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
EXE = os.path.join(ROOT, "tests", "device", "quant_arith_check")


def test_quantiser_quotients_match_ieee_division():
    if not os.path.exists(EXE):
        pytest.fail(f"{EXE} is missing: build it with `python -c 'import __graft_entry__ as g; g.build()'`")
    res = subprocess.run([EXE], capture_output=True, text=True, timeout=300)
    print(res.stdout)
    assert res.returncode == 0 and "quant_arith_check ok" in res.stdout, res.stdout + res.stderr
