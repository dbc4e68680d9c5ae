"""The E2M1 rounding forms of the GPU quantiser, restated in numpy and checked
against the oracle's rules over every fp32 value where they can differ (no
GPU needed).

The quantiser kernel rounds every rule on gfx950's FP4 conversion, which
rounds to the nearest E2M1 magnitude with ties to the even code and
saturates at 6.  Two rules reach it through a rewrite of |v| that must not
move any value across a cut point:

* half step (the bridge page's activation quantiser, section
  "Quantization"): med3(RN(|v| (1 - 2^-24) - 0.25 + 5 2^-24), |v|, 2);
* nearest lower (its weight quantiser's argmin, first index on ties): one
  ulp towards zero for the fp32 patterns with mantissa bit 22 set and bits
  20..0 clear.

The GPU parity suite compares the kernel itself with the oracle on every
bf16 pattern and next to every cut; these tests cover every fp32 value of
the ranges in which the rewrites act.
"""
import numpy as np

from oracle import quantize as oq

HALF_STEP_SCALE = np.float32(1.0) - np.float32(2.0 ** -24)
HALF_STEP_SHIFT = np.float32(-0.25 + 5 * 2.0 ** -24)
CHUNK = 1 << 21


def fp32_range(lo_bits, hi_bits):
    """Every fp32 value with bit pattern in [lo_bits, hi_bits), in chunks."""
    for b in range(lo_bits, hi_bits, CHUNK):
        yield np.arange(b, min(b + CHUNK, hi_bits), dtype=np.uint32).view(np.float32)


def converter(a):
    """The FP4 conversion on |v|: nearest magnitude, ties to the even code, 6 above."""
    return oq.e2m1_nearest_index(np.minimum(a, np.float32(6.0)))


def half_step_rewrite(a):
    # a (24 bits) times the scale (24 bits) is exact in float64, and so is the
    # sum with the shift for a in [1, 8): the float32 cast is the fma's single
    # rounding
    f = (a.astype(np.float64) * np.float64(HALF_STEP_SCALE) + np.float64(HALF_STEP_SHIFT)).astype(np.float32)
    return np.maximum(np.minimum(f, a), np.minimum(np.maximum(f, a), np.float32(2.0)))   # med3(f, a, 2)


def nearest_lower_rewrite(a):
    b = a.view(np.uint32)
    return (b - ((b & np.uint32(0x005FFFFF)) == np.uint32(0x00400000)).astype(np.uint32)).view(np.float32)


def test_rewrite_constants_are_exact():
    assert float(HALF_STEP_SCALE) == 1.0 - 2.0 ** -24
    assert float(HALF_STEP_SHIFT) == -0.25 + 5 * 2.0 ** -24


def test_half_step_rewrite_matches_the_table_on_every_fp32_from_2_to_8():
    """Below 2 the rewrite returns |v| itself (f(a) < a there), and from 8 up
    both sides give the top code; in between every fp32 value is checked."""
    lo = int(np.float32(2.0).view(np.uint32))
    hi = int(np.float32(8.0).view(np.uint32))
    for a in fp32_range(lo, hi):
        want = oq.e2m1_index(a, oq.ROUND_HALF_STEP)
        got = converter(half_step_rewrite(a))
        bad = np.flatnonzero(want != got)
        assert bad.size == 0, f"{bad.size} mismatches, first at {a[bad[0]]!r}"


def test_half_step_rewrite_below_2_and_far_above():
    rng = np.random.default_rng(11)
    a = np.concatenate([rng.uniform(0, 2, 200000).astype(np.float32),
                        np.float32(2.0) ** rng.uniform(3, 20, 20000).astype(np.float32),
                        np.array([0.0, 2.0 ** -149, 1.0, 1.75, 1.9999999, 8.0, 3e38], np.float32)])
    assert np.array_equal(converter(half_step_rewrite(a)), oq.e2m1_index(a, oq.ROUND_HALF_STEP))
    small = a[a < 2]
    assert np.array_equal(half_step_rewrite(small), small)


def test_nearest_lower_rewrite_matches_the_argmin_on_every_fp32_from_0_125_to_8():
    lo = int(np.float32(0.125).view(np.uint32))
    hi = int(np.float32(8.0).view(np.uint32))
    for a in fp32_range(lo, hi):
        want = oq.e2m1_index(a, oq.ROUND_NEAREST_LOWER)
        got = converter(nearest_lower_rewrite(a))
        bad = np.flatnonzero(want != got)
        assert bad.size == 0, f"{bad.size} mismatches, first at {a[bad[0]]!r}"


def test_nearest_even_is_the_converter():
    rng = np.random.default_rng(12)
    a = rng.uniform(0, 7, 300000).astype(np.float32)
    a[:7] = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    assert np.array_equal(converter(a), oq.e2m1_index(a, oq.ROUND_NEAREST_EVEN))
