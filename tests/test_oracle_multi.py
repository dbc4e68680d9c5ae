"""Pins of the small-N GEMM and grouped-GEMV oracle (no GPU needed): the bf16
rounding against hand-derived bit patterns, the sums against an independent
float64 matrix product of the decoded operands, the expert ranges against the
page's cumulative-offset rule, and the untouched rows."""
import numpy as np
import pytest

import workloads
from oracle import multi
from oracle import reference as ref


def decode(packed, scales):
    """float64 values of packed E2M1 codes times their E4M3 block scales."""
    packed = np.asarray(packed)
    codes = np.stack([packed & 15, packed >> 4], -1).reshape(*packed.shape[:-1], -1)
    vals = ref.e2m1_table()[codes]
    sv = np.repeat(ref.e4m3_table()[np.asarray(scales)], 16, axis=-1)
    return vals * sv


def test_bf16_rounding_hand_values():
    # 1 + 2^-8: halfway between 1 (mantissa 0, even) and 1 + 2^-7 -> 0x3F80
    # 1 + 3*2^-8: halfway between 1 + 2^-7 (odd) and 1 + 2^-6 (even) -> 0x3F82
    # 1 + 2^-9: below halfway -> 0x3F80; -2.5 -> 0xC020; -0 -> 0x8000
    # 0x7F7F8000 as fp32 (3.3961e38) is halfway between bf16 max 0x7F7F and 0x7F80 -> even -> Inf
    vals = np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, 1 + 2 ** -9, -2.5, -0.0, 0.0], dtype=np.float32)
    vals = np.concatenate([vals, np.array([0x7F7F8000, 0x7F7F7FFF], dtype=np.uint32).view(np.float32)])
    got = multi.round_f32_to(vals, "bf16")
    assert [hex(v) for v in got] == ["0x3f80", "0x3f82", "0x3f80", "0xc020", "0x8000", "0x0",
                                     "0x7f80", "0x7f7f"]


def test_f16_path_matches_gemv_epilogue():
    S = np.array([[2307.0, 2305.0, -576.0, 1e6]])
    assert np.array_equal(multi.scale_sums(S, np.float32(1.0), "f16"), ref.epilogue(S, [1.0]))


@pytest.mark.parametrize("out", ["f16", "bf16"])
def test_smalln_against_float64_matmul(out):
    l, m, n, k = 2, 24, 5, 96
    ops = workloads.integer_coded(l, m, k, seed=4)
    B = workloads.integer_coded(l, n, k, seed=5)
    alpha = np.float32([1.5, 0.75])
    got = multi.gemm_smalln(ops["A"], ops["sfA"], B["A"], B["sfA"], alpha, l, m, n, k, out)
    S = np.einsum("lmk,lnk->lmn", decode(ops["A"], ops["sfA"]), decode(B["A"], B["sfA"]))
    want = multi.round_f32_to((alpha.astype(np.float64)[:, None, None] * S).astype(np.float32), out)
    assert np.array_equal(got, want)


def test_smalln_columns_are_gemvs():
    l, m, n, k = 3, 16, 4, 64
    ops = workloads.integer_coded(l, m, k, seed=6)
    B = workloads.integer_coded(l, n, k, seed=7)
    got = multi.gemm_smalln(ops["A"], ops["sfA"], B["A"], B["sfA"], None, l, m, n, k, "f16")
    for j in range(n):
        want = ref.gemv(ops["A"], ops["sfA"], np.ascontiguousarray(B["A"][:, j]),
                        np.ascontiguousarray(B["sfA"][:, j]), None, l, m, k)
        assert np.array_equal(got[:, :, j], want)


def test_expert_ranges_follow_cumulative_offsets():
    # counts [2, 0, 1, 3] -> cumulative offsets [2, 2, 3, 6]
    assert multi.expert_ranges([2, 2, 3, 6], 4) == [(0, 2), (2, 2), (2, 3), (3, 6)]


@pytest.mark.parametrize("out", ["f16", "bf16"])
def test_grouped_against_float64_matmul(out):
    E, n, k, T = 3, 16, 64, 5
    W = workloads.integer_coded(E, n, k, seed=8)
    X = workloads.integer_coded(1, T, k, seed=9)
    Xp, sfX = X["A"][0], X["sfA"][0]
    offsets = np.array([2, 2, 4], dtype=np.int32)           # token 4 belongs to no expert
    gs_x = np.float32([0.5, 3.0, 1.25])
    gs_w = np.float32([2.0, 1.0, 0.375])
    got = multi.grouped_gemv(Xp, sfX, W["A"], W["sfA"], offsets, gs_x, gs_w, T, E, n, k, out)
    Wd, Xd = decode(W["A"], W["sfA"]), decode(Xp, sfX)
    expert_of = [0, 0, 2, 2]
    for t, e in enumerate(expert_of):
        S = Wd[e] @ Xd[t]
        alpha = np.float32(gs_x[e] * gs_w[e])
        want = multi.round_f32_to((np.float64(alpha) * S).astype(np.float32), out)
        assert np.array_equal(got[t], want)
    assert np.all(got[4] == 0xFFFF)


def test_grouped_missing_scales_mean_one():
    E, n, k, T = 2, 8, 32, 3
    W = workloads.integer_coded(E, n, k, seed=10)
    X = workloads.integer_coded(1, T, k, seed=11)
    a = multi.grouped_gemv(X["A"][0], X["sfA"][0], W["A"], W["sfA"], [1, 3], None, None, T, E, n, k)
    b = multi.grouped_gemv(X["A"][0], X["sfA"][0], W["A"], W["sfA"], [1, 3], np.ones(2, np.float32),
                           np.ones(2, np.float32), T, E, n, k)
    assert np.array_equal(a, b)
