"""The no-allocation GEMV entry point (nvfp4_gemv_launch_noalloc) against the
caller-workspace entry point (nvfp4_gemv_launch_ws) and the oracle, through
the C ABI: two split-K calls in a row, the second smaller (the fixed scratch
array keeps the first call's partial sums, which the second must not see),
then an unsplit call, and a shape whose partial sums exceed the array."""
import ctypes

import numpy as np
import pytest
import torch

import precision_decode_amd as pd
import workloads
from gpu_util import assert_bits_equal, to_device
from oracle import reference as ref

pytestmark = pytest.mark.gpu

# one GPU's eighth of the decode weight (K split 8), then a smaller split shape
# (fewer rows, shorter K), then a shape with no split
SHAPES = [(1, 896, 16384), (1, 300, 8192), (2, 100, 2048)]


@pytest.fixture(scope="module", autouse=True)
def gpu_ready():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    pd.load()


def call(fn, d, c, l, m, k, *extra):
    lib = pd.load()
    st = getattr(lib, fn)(d["A"].data_ptr(), d["sfA"].data_ptr(), d["x"].data_ptr(),
                          d["sfx"].data_ptr(), d["alpha"].data_ptr(), c.data_ptr(), l, m, k, *extra,
                          torch.cuda.current_stream().cuda_stream)
    assert st == pd.NVFP4_GEMV_OK, (fn, st, pd.nvfp4_gemv_status_string(st))


def test_noalloc_matches_caller_workspace_entry_point():
    for i, (l, m, k) in enumerate(SHAPES):
        print(f"noalloc case {(l, m, k)}", flush=True)
        ops = workloads.integer_coded(l, m, k, seed=60 + i, alpha="uniform")
        d = to_device(ops)
        ws_bytes = pd.nvfp4_gemv_workspace_size(l, m, k)
        assert (ws_bytes > 0) == (i < 2)
        assert ws_bytes <= pd.NVFP4_GEMV_NOALLOC_SCRATCH_BYTES
        ws = torch.empty(max(ws_bytes, 4), dtype=torch.uint8, device="cuda")
        c_ws = torch.full((l, m), -1, dtype=torch.int16, device="cuda")
        c_na = torch.full((l, m), -1, dtype=torch.int16, device="cuda")
        call("nvfp4_gemv_launch_ws", d, c_ws, l, m, k, ctypes.c_void_p(ws.data_ptr()),
             ctypes.c_size_t(ws_bytes))
        call("nvfp4_gemv_launch_noalloc", d, c_na, l, m, k)
        torch.cuda.synchronize()
        got_ws = c_ws.cpu().numpy().view(np.uint16)
        got_na = c_na.cpu().numpy().view(np.uint16)
        want = ref.gemv(ops["A"], ops["sfA"], ops["x"], ops["sfx"], ops["alpha"], l, m, k)
        assert_bits_equal(got_ws, want, f"launch_ws {(l, m, k)}")
        assert_bits_equal(got_na, got_ws, f"noalloc vs launch_ws {(l, m, k)}")


def test_noalloc_refuses_partial_sums_above_the_array():
    # K split 2 over 524352 rows: 4 MiB + 2 KiB of partial sums.  The buffers are
    # allocated (uninitialised, never read: the call is refused before launching).
    l, m, k = 1, 524352, 32768
    assert pd.nvfp4_gemv_workspace_size(l, m, k) > pd.NVFP4_GEMV_NOALLOC_SCRATCH_BYTES
    d = {"A": torch.empty(l * m * k // 2, dtype=torch.uint8, device="cuda"),
         "sfA": torch.empty(l * m * k // 16, dtype=torch.uint8, device="cuda"),
         "x": torch.empty(l * k // 2, dtype=torch.uint8, device="cuda"),
         "sfx": torch.empty(l * k // 16, dtype=torch.uint8, device="cuda"),
         "alpha": torch.ones(l, dtype=torch.float32, device="cuda")}
    c = torch.full((l, m), -1, dtype=torch.int16, device="cuda")
    lib = pd.load()
    st = lib.nvfp4_gemv_launch_noalloc(d["A"].data_ptr(), d["sfA"].data_ptr(), d["x"].data_ptr(),
                                       d["sfx"].data_ptr(), d["alpha"].data_ptr(), c.data_ptr(),
                                       l, m, k, torch.cuda.current_stream().cuda_stream)
    assert st == pd.NVFP4_GEMV_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert bool((c == -1).all())
    del d
    torch.cuda.empty_cache()
