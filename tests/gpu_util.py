"""Helpers shared by the GPU tests: move inputs to the device, call the HIP
library through its C ABI, compare fp16 bit patterns, build edge-case inputs."""
import numpy as np
import torch

import precision_decode_amd as pd
import workloads


def to_device(ops):
    # np.array copies: some fixtures are read-only arrays, which torch will not wrap
    return {k: torch.from_numpy(np.array(v, order="C")).cuda() for k, v in ops.items()}


def run_gpu(dops, l, m, k, tuning=None, use_alpha=True, mode="launch", stream=None):
    """Runs one GEMV on the GPU and returns the fp16 bits as a uint16 numpy array."""
    c = torch.full((l, m), -1, dtype=torch.int16, device="cuda")   # 0xFFFF: a NaN pattern
    alpha = dops["alpha"] if use_alpha else None
    args = (dops["A"], dops["sfA"], dops["x"], dops["sfx"], alpha, c, l, m, k)
    if mode == "launch" and tuning is None:
        pd.nvfp4_gemv_launch(*args, stream=stream)
    else:
        _, ws_bytes = pd.nvfp4_gemv_plan(l, m, k, aligned=True, tuning=tuning)
        ws = torch.empty(max(ws_bytes, 4), dtype=torch.uint8, device="cuda")
        if mode == "ws" and tuning is None:
            pd.nvfp4_gemv_launch_ws(*args, ws, ws_bytes, stream=stream)
        else:
            pd.nvfp4_gemv_launch_tuned(*args, tuning, ws, ws_bytes, stream=stream)
    torch.cuda.synchronize()
    return c.cpu().numpy().view(np.uint16)


def f16_ordered(bits):
    """Map fp16 (or bf16) bit patterns to integers whose difference counts ulps."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.int64)
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)


def nan_mask(bits, fmt="f16"):
    """NaN positions of fp16 or bf16 bit patterns."""
    b = np.asarray(bits, dtype=np.uint16)
    if fmt == "bf16":
        return (b & 0x7FFF) > 0x7F80
    return (b & 0x7FFF) > 0x7C00


def assert_bits_equal(got, want, what="", fmt="f16"):
    got = np.asarray(got, dtype=np.uint16)
    want = np.asarray(want, dtype=np.uint16)
    gnan = nan_mask(got, fmt)
    wnan = nan_mask(want, fmt)
    assert np.array_equal(gnan, wnan), f"{what}: NaN positions differ"
    diff = (got != want) & ~gnan
    if diff.any():
        idx = np.argwhere(diff)[:5]
        details = [(tuple(i), hex(int(got[tuple(i)])), hex(int(want[tuple(i)]))) for i in idx]
        raise AssertionError(f"{what}: {int(diff.sum())} of {got.size} outputs differ, e.g. {details}")


def bits_to_f64(bits, fmt="f16"):
    b = np.asarray(bits, dtype=np.uint16)
    if fmt == "bf16":
        return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return b.view(np.float16).astype(np.float64)


def assert_within_tolerance(got, want, ulps=2, rel=1e-3, what="", fmt="f16"):
    """|got - want| <= max(ulps ulps of the output format, rel * |want|), NaN where the
    oracle has NaN."""
    got = np.asarray(got, dtype=np.uint16)
    want = np.asarray(want, dtype=np.uint16)
    g = bits_to_f64(got, fmt)
    w = bits_to_f64(want, fmt)
    assert np.array_equal(np.isnan(g), np.isnan(w)), f"{what}: NaN positions differ"
    fin = ~np.isnan(w)
    ulp_ok = np.abs(f16_ordered(got) - f16_ordered(want)) <= ulps
    with np.errstate(invalid="ignore"):
        rel_ok = np.abs(g - w) <= rel * np.abs(w)
    ok = ulp_ok | rel_ok | ~fin
    assert ok.all(), f"{what}: {int((~ok).sum())} outputs outside tolerance"


def grouped_special_ops(counts, n, k, seed):
    """Arbitrary code bytes with every finite scale code (subnormal, negative,
    up to 448), a NaN scale code planted in one expert's weight row and in one
    token; per-expert global scales U[0.5, 2]."""
    experts, tokens = len(counts), int(sum(counts))
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    w = workloads.random_bytes(experts, n, k, seed=seed, scale_codes=finite)
    x = workloads.random_bytes(1, tokens, k, seed=seed + 1, scale_codes=finite)
    rng = np.random.default_rng(seed + 2)
    ops = {"X": x["A"][0], "sfX": x["sfA"][0], "W": w["A"], "sfW": w["sfA"],
           "offsets": np.cumsum(counts).astype(np.int32),
           "gs_x": rng.uniform(0.5, 2, experts).astype(np.float32),
           "gs_w": rng.uniform(0.5, 2, experts).astype(np.float32)}
    ops["sfW"][1, 3, 2] = 0x7F                     # expert 1, weight row 3
    ops["sfX"][tokens - 1, 5] = 0xFF               # the last token
    return ops
