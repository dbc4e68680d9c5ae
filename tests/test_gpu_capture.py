"""GEMV calls inside a HIP graph: the library-owned split-K workspace is sized
before capture (nvfp4_workspace_reserve), two split-K calls of different
sizes and one unsplit call are captured on one stream, and every replay is
checked against the oracle, with eager work and synchronisations between
replays.  A call that would have to grow the workspace during capture
returns NVFP4_GEMV_ERR_WORKSPACE and enqueues nothing."""
import numpy as np
import pytest
import torch

import precision_decode_amd as pd
import workloads
from gpu_util import assert_bits_equal, to_device
from oracle import reference as ref

pytestmark = pytest.mark.gpu

# (l, m, k): one GPU's eighth of the decode weight (K split), a smaller split
# shape, and the short-K workload's shape with fewer rows (no split)
SHAPES = [(1, 896, 16384), (1, 300, 8192), (2, 512, 2048)]


@pytest.fixture(scope="module", autouse=True)
def gpu_ready():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    pd.load()


def test_captured_split_k_calls_after_reserve():
    cases = []
    for i, (l, m, k) in enumerate(SHAPES):
        ops = workloads.integer_coded(l, m, k, seed=40 + i, alpha="uniform")
        want = ref.gemv(ops["A"], ops["sfA"], ops["x"], ops["sfx"], ops["alpha"], l, m, k)
        c = torch.full((l, m), -1, dtype=torch.int16, device="cuda")
        cases.append((l, m, k, to_device(ops), c, want))
    assert pd.nvfp4_gemv_workspace_size(*SHAPES[0]) > pd.nvfp4_gemv_workspace_size(*SHAPES[1]) > 0
    assert pd.nvfp4_gemv_workspace_size(*SHAPES[2]) == 0

    s = torch.cuda.Stream()
    need = max(pd.nvfp4_gemv_workspace_size(l, m, k) for l, m, k in SHAPES)
    pd.nvfp4_workspace_reserve(need, stream=s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    print("capturing 3 GEMV calls", flush=True)
    with torch.cuda.graph(g, stream=s):
        for l, m, k, d, c, _ in cases:
            pd.nvfp4_gemv_launch(d["A"], d["sfA"], d["x"], d["sfx"], d["alpha"], c, l, m, k)
    torch.cuda.synchronize()
    for replay in range(3):
        for *_, c, _ in cases:
            c.fill_(-1)                                 # eager work between replays
        torch.cuda.synchronize()
        print(f"replay {replay}", flush=True)
        g.replay()
        torch.cuda.synchronize()
        for l, m, k, _, c, want in cases:
            assert_bits_equal(c.cpu().numpy().view(np.uint16), want, f"replay {replay} {(l, m, k)}")


def test_growing_during_capture_is_refused():
    l, m, k = 1, 896, 16384                              # needs a split-K workspace
    ops = workloads.integer_coded(l, m, k, seed=50)
    d = to_device(ops)
    c = torch.full((l, m), -1, dtype=torch.int16, device="cuda")
    l2, m2, k2 = SHAPES[2]                               # no workspace: captured normally
    ops2 = workloads.integer_coded(l2, m2, k2, seed=51)
    d2 = to_device(ops2)
    c2 = torch.full((l2, m2), -1, dtype=torch.int16, device="cuda")
    s = torch.cuda.Stream()                              # a fresh stream: no workspace yet
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    statuses = []
    with torch.cuda.graph(g, stream=s):
        statuses.append(pd.load().nvfp4_gemv_launch(d["A"].data_ptr(), d["sfA"].data_ptr(),
                                                    d["x"].data_ptr(), d["sfx"].data_ptr(),
                                                    d["alpha"].data_ptr(), c.data_ptr(), l, m, k,
                                                    s.cuda_stream))
        pd.nvfp4_gemv_launch(d2["A"], d2["sfA"], d2["x"], d2["sfx"], d2["alpha"], c2, l2, m2, k2)
    assert statuses == [pd.NVFP4_GEMV_ERR_WORKSPACE]
    g.replay()
    torch.cuda.synchronize()
    want2 = ref.gemv(ops2["A"], ops2["sfA"], ops2["x"], ops2["sfx"], ops2["alpha"], l2, m2, k2)
    assert_bits_equal(c2.cpu().numpy().view(np.uint16), want2, "unsplit call in the same graph")
    assert (c.cpu().numpy().view(np.uint16) == 0xFFFF).all()   # the refused call wrote nothing
    # outside capture the same call grows the workspace and runs
    want = ref.gemv(ops["A"], ops["sfA"], ops["x"], ops["sfx"], ops["alpha"], l, m, k)
    pd.nvfp4_gemv_launch(d["A"], d["sfA"], d["x"], d["sfx"], d["alpha"], c, l, m, k, stream=s)
    torch.cuda.synchronize()
    assert_bits_equal(c.cpu().numpy().view(np.uint16), want, "after capture")
