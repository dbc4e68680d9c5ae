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


# ---- quantiser with a given global scale (the page's graph-safe activation path) and the
# ---- three rounding rules

from golden_io import quant_examples  # noqa: E402


def codes_of(packed):
    packed = np.asarray(packed)
    return np.stack([packed & 15, packed >> 4], -1).reshape(*packed.shape[:-1], -1)


@pytest.mark.parametrize("ex", quant_examples(), ids=lambda e: f"{e['name']}-{e['rule']}")
def test_hand_derived_quant_examples(ex):
    packed, sf = q.quantize_with_scale(ex["values"], ex["gs"], q.RULE_NAMES[ex["rule"]])
    assert int(sf[0]) == ex["sf"]
    assert np.array_equal(packed, ex["packed"]), (packed.tobytes().hex(), ex["packed"].tobytes().hex())


def dense_magnitudes():
    """Every multiple of 2^-12 in [0, 6.5] plus the float32 neighbours of every
    quarter point (where the rules' boundaries lie)."""
    a = np.arange(0, 6.5 * 4096 + 1, dtype=np.float64) / 4096
    q4 = np.arange(0, 27, dtype=np.float32) / np.float32(4)
    nb = np.concatenate([np.nextafter(q4, np.float32(-1)), q4, np.nextafter(q4, np.float32(7))])
    return np.unique(np.concatenate([a.astype(np.float32), nb[nb >= 0]]))


def test_half_step_table_departs_from_nearest_on_three_intervals():
    """Derived by hand from the table: doubling and rounding puts (2.25, 2.75) on step 5,
    (3.25, 3.75) on step 7 and [4.75, 5.25] on step 10, which the table sends to 2, 3 and 4;
    nearest rounding sends (2.5, 2.75), [3.5, 3.75) and (5, 5.25] one code higher."""
    a = dense_magnitudes()
    hs = q.e2m1_index(a, q.ROUND_HALF_STEP).astype(int)
    ne = q.e2m1_index(a, q.ROUND_NEAREST_EVEN).astype(int)
    a64 = a.astype(np.float64)
    off = ((a64 > 2.5) & (a64 < 2.75)) | ((a64 >= 3.5) & (a64 < 3.75)) | ((a64 > 5) & (a64 <= 5.25))
    assert off.sum() > 1000
    assert np.array_equal(hs[~off], ne[~off])
    assert np.array_equal(hs[off], ne[off] - 1)


def test_nearest_lower_differs_from_even_only_on_upward_ties():
    """On a tie the even code is the upper neighbour at 0.75, 1.75 and 3.5 and the lower one
    at 0.25, 1.25, 2.5 and 5; away from ties both are the argmin of the exact distance."""
    a = dense_magnitudes()
    a = a[a <= 6]
    nl = q.e2m1_index(a, q.ROUND_NEAREST_LOWER).astype(int)
    ne = q.e2m1_index(a, q.ROUND_NEAREST_EVEN).astype(int)
    up = np.isin(a.astype(np.float64), [0.75, 1.75, 3.5])
    assert up.sum() == 3
    assert np.array_equal(nl[~up], ne[~up])
    assert np.array_equal(nl[up], ne[up] - 1)
    d = np.abs(a.astype(np.float64)[:, None] - grid()[None, :])
    assert np.array_equal(nl, d.argmin(axis=1))         # numpy argmin: first minimum


def test_unclamped_rules_above_six():
    a = np.array([6.0, 6.5, 100.0, 24414.0625, 5e5], dtype=np.float32)
    for rule in (q.ROUND_HALF_STEP, q.ROUND_NEAREST_EVEN, q.ROUND_NEAREST_LOWER):
        assert list(q.e2m1_index(a, rule)) == [7] * 5


def test_nan_gets_code_zero():
    v = np.array([np.nan, -np.nan], dtype=np.float32)
    for rule in (q.ROUND_HALF_STEP, q.ROUND_NEAREST_EVEN, q.ROUND_NEAREST_LOWER):
        assert list(q.e2m1_index(v, rule)) == [0, 0]


def test_e4m3_cast_rounds_to_nearest_even():
    """Pins torch's float -> float8_e4m3fn cast (the page's step) against the decode table:
    the code's value is a nearest finite E4M3 value, ties go to the even code, and past
    464 (halfway to the next step, 480, whose pattern is NaN) the result is 0x7F."""
    rng = np.random.default_rng(7)
    v = np.exp2(rng.uniform(-13, 9.5, size=200000)).astype(np.float32)
    e4 = ref.e4m3_table()
    finite = np.array([c for c in range(0x7F) if np.isfinite(e4[c])])
    mids = (e4[finite][:-1] + e4[finite][1:]) / 2
    v = np.concatenate([v, mids.astype(np.float32), np.float32([448, 463.9, 464, 464.1, 479, 480, 1e6])])
    codes = q.e4m3_encode(v)
    big = v.astype(np.float64) > 464
    assert np.all(codes[big] == 0x7F)
    v64 = v[~big].astype(np.float64)
    got = e4[codes[~big]]
    d = np.abs(v64[:, None] - e4[finite][None, :])
    dmin = d.min(axis=1)
    assert np.all(np.abs(v64 - got) == dmin)
    tie = (d == dmin[:, None]).sum(axis=1) == 2
    assert tie.sum() >= len(mids) - 1
    assert np.all(codes[~big][tie] % 2 == 0)


@pytest.mark.parametrize("rule", [0, 1, 2])
def test_grid_values_round_trip_for_every_rule(rule):
    rng = np.random.default_rng(11 + rule)
    e4 = ref.e4m3_table()
    g = grid()
    rows = []
    for s in e4[[0x7E, 0x38, 0x40, 0x21, 0x55, 0x0C, 0x6B, 0x30]]:
        vals = g[rng.integers(0, 8, size=16)] * np.where(rng.random(16) < 0.5, -1, 1)
        vals[rng.integers(0, 16)] = 6.0
        rows.append(vals * s)
    t = np.concatenate(rows).astype(np.float32)
    packed, sc = q.quantize_with_scale(t, np.float32(1.0), rule)
    assert np.array_equal(q.dequantize(packed, sc, 1.0), t.astype(np.float64))


@pytest.mark.parametrize("rule", [0, 1, 2])
def test_sign_symmetry(rule):
    raw = workloads.gaussian_bf16(1, 8, 256, seed=5)["A"][0]
    raw = np.where(raw == 0, np.float32(1.0), raw)
    p1, s1 = q.quantize_with_scale(raw, np.float32(0.01), rule)
    p2, s2 = q.quantize_with_scale(-raw, np.float32(0.01), rule)
    assert np.array_equal(s1, s2)
    assert np.array_equal(codes_of(p2), codes_of(p1) ^ 8)


@pytest.mark.parametrize("rule", [0, 1, 2])
def test_power_of_two_scale_invariance(rule):
    raw = workloads.gaussian_bf16(1, 8, 256, seed=6)["A"][0]
    base = q.quantize_with_scale(raw, np.float32(0.003), rule)
    for j in (-3, 5):
        f = np.float32(2.0 ** j)
        got = q.quantize_with_scale(raw * f, np.float32(0.003) * f, rule)
        assert np.array_equal(got[0], base[0]) and np.array_equal(got[1], base[1])


def test_per_row_scale_equals_row_by_row():
    raw = workloads.gaussian_bf16(1, 6, 128, seed=8)["A"][0]
    g = np.array([0.5, 0.01, 2.0, 1e-3, 3.0, 0.07], dtype=np.float32)
    p, s = q.quantize_with_scale(raw, g, q.ROUND_HALF_STEP)
    for r in range(6):
        pr, sr = q.quantize_with_scale(raw[r], g[r], q.ROUND_HALF_STEP)
        assert np.array_equal(p[r], pr) and np.array_equal(s[r], sr)


def test_given_scale_path_matches_amax_path():
    raw = workloads.gaussian_bf16(1, 4, 512, seed=9)["x"][0]
    packed, sc, g = q.quantize_nvfp4(raw)
    assert g == np.float32(np.float32(np.abs(raw).max()) / np.float32(2688.0))
    p2, s2 = q.quantize_with_scale(raw, g, q.ROUND_NEAREST_EVEN)
    assert np.array_equal(packed, p2) and np.array_equal(sc, s2)


def test_non_finite_input_poisons_only_its_block():
    t = np.ones(48, dtype=np.float32)
    t[20] = np.inf
    p, s = q.quantize_with_scale(t, np.float32(1.0), q.ROUND_HALF_STEP)
    # 1/6 = 1.333 * 2^-3 -> exponent field 4, mantissa 3 (2.67 rounded) -> 0x23 = 0.171875;
    # v = 1 / 0.171875 = 5.82 -> code 7.  The Inf block: scale 0x7F, v NaN -> codes 0.
    assert list(s) == [0x23, 0x7F, 0x23]
    c = codes_of(p)
    assert np.all(c[:16] == 7) and np.all(c[16:32] == 0) and np.all(c[32:] == 7)


def test_activation_gemv_composes_quantiser_and_gemv():
    """With x already on the grid (scale 1, amax 6 per block) the quantised x decodes to x
    itself, so the composite equals the plain float64 product, and alpha = A_scale * x_scale."""
    rng = np.random.default_rng(12)
    l, m, k = 2, 8, 64
    ops = workloads.integer_coded(l, m, k, seed=3)
    vals = grid()[rng.integers(0, 8, size=(l, k))] * np.where(rng.random((l, k)) < 0.5, -1, 1)
    vals.reshape(l, k // 16, 16)[:, :, 0] = 6.0
    xs = np.float32([0.5, 2.0])
    x = (vals * xs[:, None]).astype(np.float32)
    c, xp, sfx, alpha = q.activation_gemv(ops["A"], ops["sfA"], np.float32([3.0, 0.25]), x, xs,
                                          q.ROUND_HALF_STEP, l, m, k)
    assert list(alpha) == [1.5, 0.5]
    assert np.all(sfx == 0x38)
    A = ref.e2m1_table()[codes_of(ops["A"])] * np.repeat(ref.e4m3_table()[ops["sfA"]], 16, axis=-1)
    S = np.einsum("lmk,lk->lm", A, vals.astype(np.float64))
    assert np.array_equal(c, ref.epilogue(S, alpha))
