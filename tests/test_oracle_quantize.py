"""Property pins of the oracle's BF16 -> NVFP4 quantiser (no GPU needed).

The pages print no quantised values, so the exact bytes are "parity unpinned";
these tests pin the properties the bridge page's recipe implies: values already
on the grid survive a round trip exactly, every code is a nearest E2M1 value
(the page's argmin rule), ties go to the even code (the reading taken),
block scales stay finite and at most 448, and the global scale is amax / 2688.
"""
import numpy as np
import pytest
import torch

import workloads
from oracle import quantize as q
from oracle import reference as ref
from golden_io import e2m1_magnitudes


def grid():
    return np.array([float(v) for v in e2m1_magnitudes()])


def test_nearest_index_ties_to_even():
    mags = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], dtype=np.float32)
    assert list(q.e2m1_nearest_index(mags)) == [0, 2, 2, 4, 4, 6, 6]


def test_nearest_index_is_argmin_off_ties():
    rng = np.random.default_rng(0)
    mags = rng.uniform(0, 6, size=20000).astype(np.float32)
    idx = q.e2m1_nearest_index(mags)
    d = np.abs(mags.astype(np.float64)[:, None] - grid()[None, :])
    assert np.all(d[np.arange(len(mags)), idx] == d.min(axis=1))
    assert np.array_equal(idx[d.min(axis=1) < np.sort(d, axis=1)[:, 1]],
                          d.argmin(axis=1)[d.min(axis=1) < np.sort(d, axis=1)[:, 1]])


def test_grid_values_round_trip_exactly():
    """A tensor whose amax is 6*448 has global scale exactly 1; blocks made of
    E2M1 values times an E4M3-representable scale, each containing +-6*scale,
    must come back bit for bit."""
    rng = np.random.default_rng(1)
    e4 = ref.e4m3_table()
    scales = e4[[0x7E, 0x38, 0x40, 0x21, 0x55, 0x0C, 0x6B, 0x30]]
    g = grid()
    blocks = []
    for s in scales:
        vals = g[rng.integers(0, 8, size=16)] * np.where(rng.random(16) < 0.5, -1, 1)
        vals[rng.integers(0, 16)] = 6.0 * (1 if rng.random() < 0.5 else -1)
        blocks.append(vals * s)
    t = np.concatenate(blocks).astype(np.float32)
    assert np.abs(t).max() == 6 * 448
    packed, sc, gs = q.quantize_nvfp4(t)
    assert gs == np.float32(1.0)
    assert np.array_equal(q.dequantize(packed, sc, gs), t.astype(np.float64))


def test_scale_range_and_global_scale():
    raw = workloads.gaussian_bf16(2, 64, 256, seed=3)
    for b in range(2):
        packed, sc, g = q.quantize_nvfp4(raw["A"][b])
        amax = np.float32(np.abs(raw["A"][b]).max())
        assert g == np.float32(amax / np.float32(2688.0))
        vals = ref.e4m3_table()[sc]
        assert np.isfinite(vals).all() and (vals >= 0).all() and vals.max() <= 448.0
        assert vals.max() == 448.0        # the block holding amax maps to the top scale


def test_quantised_codes_are_nearest_after_scaling():
    raw = workloads.gaussian_bf16(1, 32, 512, seed=4)
    t = raw["A"][0]
    packed, sc, g = q.quantize_nvfp4(t)
    e4 = ref.e4m3_table().astype(np.float32)
    tn = t / g
    v = tn.reshape(32, 32, 16) / np.maximum(e4[sc], np.float32(1e-8))[..., None]
    mag = np.minimum(np.abs(v), np.float32(6.0)).astype(np.float64)
    codes = np.stack([packed & 15, packed >> 4], -1).reshape(32, 512)
    got_mag = grid()[codes & 7].reshape(32, 32, 16)
    d_best = np.abs(mag[..., None] - grid()).min(-1)
    assert np.all(np.abs(mag - got_mag) == d_best)
    neg = (codes & 8).astype(bool).reshape(32, 32, 16)
    assert np.array_equal(neg, v < 0)


def test_sign_of_small_negatives_and_zero():
    t = np.zeros(32, dtype=np.float32)
    t[0] = 6.0
    t[1] = -1e-4        # rounds to magnitude 0 but keeps the sign code (8)
    t[2] = -0.0         # not < 0: code 0
    packed, sc, g = q.quantize_nvfp4(t)
    codes = np.stack([packed & 15, packed >> 4], -1).reshape(-1)
    assert codes[0] == 7 and codes[1] == 8 and codes[2] == 0


def test_packing_even_element_low_nibble():
    t = np.zeros(16, dtype=np.float32)
    t[0], t[1] = 6.0, 1.0
    packed, sc, g = q.quantize_nvfp4(t)
    assert packed[0] == (0x2 << 4) | 0x7


def test_gaussian_operands_alpha_and_shapes():
    raw = workloads.gaussian_bf16(3, 16, 64, seed=5)
    ops = q.gaussian_operands(raw, 3, 16, 64)
    assert ops["A"].shape == (3, 16, 32) and ops["sfA"].shape == (3, 16, 4)
    assert ops["x"].shape == (3, 32) and ops["sfx"].shape == (3, 4)
    for b in range(3):
        _, _, ga = q.quantize_nvfp4(raw["A"][b])
        _, _, gx = q.quantize_nvfp4(raw["x"][b])
        assert ops["alpha"][b] == np.float32(ga * gx)


def test_gaussian_gemv_close_to_unquantised_product():
    """End-to-end sanity of the quantised workload: the GEMV of the quantised
    operands tracks the bf16 product within NVFP4's relative error."""
    l, m, k = 2, 64, 1024
    raw = workloads.gaussian_bf16(l, m, k, seed=6)
    ops = q.gaussian_operands(raw, l, m, k)
    c = ref.gemv(**ops, l=l, m=m, k=k).view(np.float16).astype(np.float64)
    exact = np.einsum("bmk,bk->bm", raw["A"].astype(np.float64), raw["x"].astype(np.float64))
    err = np.abs(c - exact)
    assert np.median(err / np.sqrt(k)) < 0.25


def test_bf16_rounding_of_gaussian_draws():
    raw = workloads.gaussian_bf16(1, 4, 32, seed=7)
    a = torch.from_numpy(raw["A"])
    assert torch.equal(a.to(torch.bfloat16).float(), a)
