"""Pins of the CPU oracle against things other than itself (no GPU needed).

* the E2M1 table printed among the bridge page's constants (golden file);
* torch's float8_e4m3fn decode, for all 256 codes;
* hand-derived single-block examples (golden file, closed-form derivations);
* exact rational brute force on tiny shapes, with an independently written
  round-to-nearest-even to fp32 and fp16;
* an independent float64 matmul of separately decoded operands;
* invariants: zero scales, sign flips, block and batch permutations,
  power-of-two alpha, NaN scales.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import workloads
from oracle import reference as ref
from golden_io import e2m1_fraction, e2m1_magnitudes, hand_examples

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


# ---------------------------------------------------------------- helpers
def torch_e4m3_values():
    return torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def round_rne(value: Fraction, mant_bits: int, emin: int, max_finite: Fraction):
    """Round an exact rational to a binary float format, ties to even.

    Written here from the IEEE definition, independently of numpy's casts.
    Returns a Fraction, or +-inf as a float."""
    if value == 0:
        return Fraction(0)
    sign = -1 if value < 0 else 1
    a = abs(value)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    e = max(e, emin)
    ulp = Fraction(2) ** (e - mant_bits)
    q = a / ulp
    n = q.numerator // q.denominator
    r = q - n
    if r > Fraction(1, 2) or (r == Fraction(1, 2) and n % 2 == 1):
        n += 1
    v = n * ulp
    if v > max_finite:
        return sign * float("inf")
    return sign * v


F32_MAX = (2 - Fraction(1, 2 ** 23)) * Fraction(2) ** 127
F16_MAX = Fraction(65504)


def exact_output_bits(alpha: float, S: Fraction) -> int:
    """fp16 bits of f16(f32(alpha * S)) from exact arithmetic."""
    v32 = round_rne(Fraction(alpha) * S, 23, -126, F32_MAX)
    if isinstance(v32, float):
        v16 = v32
    else:
        v16 = round_rne(v32, 10, -14, F16_MAX)
    if isinstance(v16, float):
        return int(np.array(v16, dtype=np.float16).view(np.uint16))
    return int(np.array(float(v16), dtype=np.float16).view(np.uint16))


def exact_sums(ops, l, m, k):
    """Exact rational S[b][r] with E2M1 from the golden table and E4M3 from torch."""
    e4 = [Fraction(v) if np.isfinite(v) else None for v in torch_e4m3_values()]
    e2 = [e2m1_fraction(c) for c in range(16)]
    A, sfA, x, sfx = (ops[n] for n in ("A", "sfA", "x", "sfx"))
    out = []
    for b in range(l):
        row_vals = []
        for r in range(m):
            s = Fraction(0)
            for kk in range(k):
                an = (A[b, r, kk // 2] >> (4 * (kk % 2))) & 15
                xn = (x[b, kk // 2] >> (4 * (kk % 2))) & 15
                s += e2[an] * e4[sfA[b, r, kk // 16]] * e2[xn] * e4[sfx[b, kk // 16]]
            row_vals.append(s)
        out.append(row_vals)
    return out


def f16_values(bits):
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


# ---------------------------------------------------------------- decode pins
def test_e2m1_table_matches_page_constants():
    mags = e2m1_magnitudes()
    table = ref.e2m1_table()
    for code in range(16):
        want = float(mags[code & 7]) * (-1.0 if code & 8 else 1.0)
        assert table[code] == want
        assert np.signbit(table[code]) == bool(code & 8)   # code 8 is -0


def test_e4m3_decode_all_codes_match_torch():
    ours = ref.e4m3_table()
    theirs = torch_e4m3_values()
    nan = np.isnan(theirs)
    assert np.array_equal(np.isnan(ours), nan)
    assert set(np.nonzero(nan)[0]) == {0x7F, 0xFF}
    assert np.array_equal(ours[~nan], theirs[~nan])
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(theirs[~nan]))
    assert ours[0x7E] == 448.0          # the E4M3 maximum the quantiser divides by
    assert ours[0x01] == 2.0 ** -9      # smallest subnormal


def test_integer_scale_codes_are_e4m3_of_0_1_2():
    codes = torch.tensor([0.0, 1.0, 2.0]).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(codes, workloads.INT_SCALE_CODES)


# ---------------------------------------------------------------- hand examples
@pytest.mark.parametrize("ex", hand_examples(), ids=lambda e: e["name"])
def test_hand_examples(ex):
    k = ex["k"]
    S = ref.gemv_sums(ex["A"], ex["sfA"], ex["x"], ex["sfx"], 1, 1, k)
    assert Fraction(S[0, 0]) == ex["S"]
    c = ref.gemv(ex["A"], ex["sfA"], ex["x"], ex["sfx"], ex["alpha"], 1, 1, k)
    assert int(c[0, 0]) == ex["c"], hex(int(c[0, 0]))
    assert exact_output_bits(float(ex["alpha"][0]), ex["S"]) == ex["c"]


# ---------------------------------------------------------------- brute force
@pytest.mark.parametrize("seed", range(6))
def test_brute_force_exact_small_exponent_range(seed):
    """Scales with exponent fields 4..10 keep every sum within 53 bits, so the
    oracle's double sum must equal the exact rational and its output bits the
    exactly rounded value."""
    rng = np.random.default_rng(100 + seed)
    l, m = int(rng.integers(1, 3)), int(rng.integers(1, 6))
    k = int(rng.choice([16, 32, 48, 64]))
    codes = np.array([(s << 7) | (e << 3) | mt for s in (0, 1) for e in range(4, 11) for mt in range(8)],
                     dtype=np.uint8)
    ops = workloads.random_bytes(l, m, k, seed=seed, scale_codes=codes)
    ops["alpha"] = rng.choice(np.array([1.0, 0.5, 1.5, 0.75, 3.0, 1.25], dtype=np.float32), size=l)
    exact = exact_sums(ops, l, m, k)
    S = ref.gemv_sums(ops["A"], ops["sfA"], ops["x"], ops["sfx"], l, m, k)
    c = ref.gemv(ops["A"], ops["sfA"], ops["x"], ops["sfx"], ops["alpha"], l, m, k)
    for b in range(l):
        for r in range(m):
            assert Fraction(S[b, r]) == exact[b][r]
            assert int(c[b, r]) == exact_output_bits(float(ops["alpha"][b]), exact[b][r])


@pytest.mark.parametrize("seed", range(4))
def test_brute_force_all_finite_scale_codes(seed):
    """Every finite E4M3 code (subnormals, negatives, 448): the double sum stays
    within the sequential-summation error bound of the exact value."""
    rng = np.random.default_rng(200 + seed)
    l, m, k = 2, 3, int(rng.choice([16, 32, 64]))
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    ops = workloads.random_bytes(l, m, k, seed=50 + seed, scale_codes=codes)
    exact = exact_sums(ops, l, m, k)
    S = ref.gemv_sums(ops["A"], ops["sfA"], ops["x"], ops["sfx"], l, m, k)
    e4 = torch_e4m3_values()
    for b in range(l):
        for r in range(m):
            bound = k * 2.0 ** -52 * 448.0 ** 2 * 36 * k
            assert abs(Fraction(S[b, r]) - exact[b][r]) <= Fraction(bound)
    assert np.isfinite(S).all() and np.isfinite(e4[ops["sfA"]]).all()


def test_nan_scale_propagates():
    ops = workloads.integer_coded(1, 4, 64, seed=3)
    ops["sfA"][0, 2, 1] = 0x7F
    ops["sfx"][0, 3] = 0xFF
    c = ref.gemv(**ops, l=1, m=4, k=64)
    vals = f16_values(c)
    # the NaN sfx block reaches every row; the NaN sfA block only row 2
    assert np.isnan(vals).all()
    ops2 = workloads.integer_coded(1, 4, 64, seed=3)
    ops2["sfA"][0, 2, 1] = 0x7F
    vals2 = f16_values(ref.gemv(**ops2, l=1, m=4, k=64))
    assert np.isnan(vals2[0, 2]) and not np.isnan(vals2[0, [0, 1, 3]]).any()


# ---------------------------------------------------------------- independent matmul
def decoded_dense(ops, l, m, k):
    """Decode with the golden E2M1 table and torch's E4M3 into float64 arrays."""
    e2 = np.array([float(e2m1_fraction(c)) for c in range(16)])
    e4 = torch_e4m3_values()
    def unpack(p):
        return np.stack([p & 15, p >> 4], axis=-1).reshape(*p.shape[:-1], -1)
    a = e2[unpack(ops["A"])] * np.repeat(e4[ops["sfA"]], 16, axis=-1)
    xv = e2[unpack(ops["x"])] * np.repeat(e4[ops["sfx"]], 16, axis=-1)
    return a, xv


@pytest.mark.parametrize("name", ["tiny", "shortk"])
def test_matches_float64_matmul_integer_coded(name):
    cfg = workloads.CONFIGS[name]
    ops = workloads.for_config(cfg)
    l, m, k = cfg.l, min(cfg.m, 256), cfg.k
    ops = dict(ops, A=ops["A"][:, :m], sfA=ops["sfA"][:, :m])
    a, xv = decoded_dense(ops, l, m, k)
    S_mm = np.einsum("bmk,bk->bm", a, xv)      # exact: integer-coded sums are exact
    S = ref.gemv_sums(ops["A"], ops["sfA"], ops["x"], ops["sfx"], l, m, k)
    assert np.array_equal(S, S_mm)


def test_unit_scales_reduce_to_plain_fp4_gemv():
    """All block scales 1.0 and alpha = 1: the generic tensor-scaled FP4 GEMV."""
    ops = workloads.integer_coded(2, 33, 128, seed=9)
    ops["sfA"][:] = 0x38
    ops["sfx"][:] = 0x38
    e2 = np.array([float(e2m1_fraction(c)) for c in range(16)])
    codes_a = np.stack([ops["A"] & 15, ops["A"] >> 4], -1).reshape(2, 33, 128)
    codes_x = np.stack([ops["x"] & 15, ops["x"] >> 4], -1).reshape(2, 128)
    want = np.matmul(e2[codes_a], e2[codes_x][..., None])[..., 0]
    S = ref.gemv_sums(ops["A"], ops["sfA"], ops["x"], ops["sfx"], 2, 33, 128)
    assert np.array_equal(S, want)


# ---------------------------------------------------------------- invariants
@pytest.fixture(scope="module")
def medium():
    l, m, k = 3, 37, 96
    ops = workloads.integer_coded(l, m, k, seed=5, alpha="uniform")
    return l, m, k, ops, ref.gemv(**ops, l=l, m=m, k=k)


def test_zero_scales_give_positive_zero(medium):
    l, m, k, ops, _ = medium
    for key in ("sfA", "sfx"):
        o = {n: v.copy() for n, v in ops.items()}
        o[key][:] = 0
        assert (ref.gemv(**o, l=l, m=m, k=k) == 0).all()


def test_sign_flip_negates_row(medium):
    l, m, k, ops, c = medium
    o = {n: v.copy() for n, v in ops.items()}
    o["A"][1, 4] ^= 0x88
    c2 = ref.gemv(**o, l=l, m=m, k=k)
    want = c[1, 4] ^ 0x8000 if c[1, 4] != 0 else 0
    assert c2[1, 4] == want
    mask = np.ones_like(c, dtype=bool)
    mask[1, 4] = False
    assert np.array_equal(c2[mask], c[mask])


def test_block_permutation_invariance(medium):
    l, m, k, ops, c = medium
    perm = np.random.default_rng(1).permutation(k // 16)
    def perm_packed(p):
        return p.reshape(*p.shape[:-1], k // 16, 8)[..., perm, :].reshape(p.shape)
    o = dict(ops, A=perm_packed(ops["A"]), x=perm_packed(ops["x"]),
             sfA=ops["sfA"][..., perm], sfx=ops["sfx"][..., perm])
    assert np.array_equal(ref.gemv(**o, l=l, m=m, k=k), c)


def test_batch_permutation(medium):
    l, m, k, ops, c = medium
    perm = np.array([2, 0, 1])
    o = {n: v[perm] for n, v in ops.items()}
    assert np.array_equal(ref.gemv(**o, l=l, m=m, k=k), c[perm])


def test_power_of_two_alpha_scales_exactly(medium):
    l, m, k, ops, c = medium
    o = dict(ops, alpha=ops["alpha"] * np.float32(0.25))
    v1, v2 = f16_values(c), f16_values(ref.gemv(**o, l=l, m=m, k=k))
    normal = np.abs(v1 * 0.25) >= 2.0 ** -14
    assert np.array_equal(v2[normal], v1[normal] * 0.25)


# ---------------------------------------------------------------- epilogue rounding
def test_epilogue_rounding_matches_torch_casts():
    rng = np.random.default_rng(7)
    S = rng.standard_normal((4, 5000)) * 10.0 ** rng.integers(-6, 6, size=(4, 5000))
    alpha = rng.uniform(0.3, 3, size=4).astype(np.float32)
    ours = ref.epilogue(S, alpha)
    prod = torch.from_numpy(alpha.astype(np.float64)[:, None] * S)
    theirs = prod.to(torch.float32).to(torch.float16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, theirs)


def test_epilogue_overflow_and_ties():
    bits = ref.epilogue(np.array([[65519.0, 65520.0, -65520.0, 2305.0, 2307.0]]), np.ones(1, np.float32))
    assert list(bits[0]) == [0x7BFF, 0x7C00, 0xFC00, 0x6880, 0x6882]


def test_two_step_rounding_order():
    """alpha * S is rounded to fp32 first, then to fp16.  Find products where a
    single rounding of the exact value to fp16 would differ, and check the
    oracle follows the two-step definition (computed here exactly)."""
    rng = np.random.default_rng(11)
    alpha = rng.uniform(0.5, 2.0, size=400000).astype(np.float32)
    S = rng.integers(1, 4096, size=400000).astype(np.float64) * 0.25
    got = ref.epilogue(S[None, :], np.ones(1, np.float32) * 1.0)  # alpha=1 path
    assert np.array_equal(got[0], S.astype(np.float32).astype(np.float16).view(np.uint16))
    prods = [Fraction(float(a)) * Fraction(s) for a, s in zip(alpha[:4000], S[:4000])]
    differs = []
    for i, p in enumerate(prods):
        one = round_rne(p, 10, -14, F16_MAX)
        two = exact_output_bits(float(alpha[i]), Fraction(S[i]))
        one_bits = int(np.array(float(one), dtype=np.float16).view(np.uint16))
        if one_bits != two:
            differs.append(i)
    # widen the search cheaply until some double-rounding cases show up
    i0 = 4000
    while len(differs) < 2 and i0 < len(alpha):
        for i in range(i0, min(i0 + 20000, len(alpha))):
            p = Fraction(float(alpha[i])) * Fraction(S[i])
            one = round_rne(p, 10, -14, F16_MAX)
            two = exact_output_bits(float(alpha[i]), Fraction(S[i]))
            if int(np.array(float(one), dtype=np.float16).view(np.uint16)) != two:
                differs.append(i)
        i0 += 20000
    assert len(differs) >= 2
    for i in differs:
        got = int(ref.epilogue(np.array([[S[i]]]), alpha[i:i + 1])[0, 0])
        assert got == exact_output_bits(float(alpha[i]), Fraction(S[i]))


def test_gemv_rows_matches_full(medium):
    l, m, k, ops, c = medium
    br = np.array([[0, 0], [2, 36], [1, 17]])
    got = ref.gemv_rows(ops["A"], ops["sfA"], ops["x"], ops["sfx"], ops["alpha"], l, m, k, br)
    assert np.array_equal(got, c[br[:, 0], br[:, 1]])
