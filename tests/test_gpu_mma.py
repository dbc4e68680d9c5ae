"""GPU parity of the small-N GEMM and the grouped (MoE) GEMV: the HIP library,
called through its C ABI, against the CPU oracle (``oracle.multi``).

Integer-coded inputs must match bit for bit in both output formats (every fp32
partial sum is exact, whatever order the matrix cores add in); Gaussian
quantised inputs must agree within max(2 ulps of the output format, 1e-3
relative).
"""
import numpy as np
import pytest
import torch

import precision_decode_amd as pd
import workloads
from gpu_util import (assert_bits_equal, assert_within_tolerance, bits_to_f64,
                      grouped_special_ops, to_device)
from oracle import multi
from oracle import quantize as oq

pytestmark = [pytest.mark.gpu, pytest.mark.filterwarnings("ignore::RuntimeWarning")]

FMT = {pd.NVFP4_OUT_F16: "f16", pd.NVFP4_OUT_BF16: "bf16"}
FILL = 0xFFFF   # a NaN pattern in both formats: marks outputs the kernel must not touch


@pytest.fixture(scope="module", autouse=True)
def gpu_ready():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    pd.load()


# ---------------------------------------------------------------- small-N GEMM
def smalln_ops(l, m, n, k, seed=0):
    a = workloads.integer_coded(l, m, k, seed=seed, alpha="uniform")
    b = workloads.integer_coded(l, n, k, seed=seed + 1)
    return {"A": a["A"], "sfA": a["sfA"], "B": b["A"], "sfB": b["sfA"], "alpha": a["alpha"]}


def run_smalln(ops, l, m, n, k, out_type=pd.NVFP4_OUT_F16, tuning=None, use_alpha=True, dev=None):
    d = dev or to_device(ops)
    c = torch.full((l, m, n), -1, dtype=torch.int16, device="cuda")
    alpha = d["alpha"] if use_alpha else None
    if tuning is None:
        pd.nvfp4_gemm_smalln_launch(d["A"], d["sfA"], d["B"], d["sfB"], alpha, c, l, m, n, k, out_type)
    else:
        _, ws_bytes = pd.nvfp4_gemm_smalln_plan(l, m, n, k, aligned=True, tuning=tuning)
        ws = torch.empty(max(ws_bytes, 4), dtype=torch.uint8, device="cuda")
        pd.nvfp4_gemm_smalln_launch_tuned(d["A"], d["sfA"], d["B"], d["sfB"], alpha, c, l, m, n, k,
                                          out_type, tuning, ws, ws_bytes)
    torch.cuda.synchronize()
    return c.cpu().numpy().view(np.uint16)


def oracle_smalln(ops, l, m, n, k, out_type=pd.NVFP4_OUT_F16, use_alpha=True):
    return multi.gemm_smalln(ops["A"], ops["sfA"], ops["B"], ops["sfB"],
                             ops["alpha"] if use_alpha else None, l, m, n, k, FMT[out_type])


@pytest.mark.parametrize("name", list(workloads.SMALLN_CONFIGS))
@pytest.mark.parametrize("out_type", [pd.NVFP4_OUT_F16, pd.NVFP4_OUT_BF16])
def test_smalln_configs_bit_exact(name, out_type):
    cfg = workloads.SMALLN_CONFIGS[name]
    ops = workloads.smalln_operands(cfg)
    want = oracle_smalln(ops, cfg.l, cfg.m, cfg.n, cfg.k, out_type)
    got = run_smalln(ops, cfg.l, cfg.m, cfg.n, cfg.k, out_type)
    assert_bits_equal(got, want, name, FMT[out_type])


SMALLN_SHAPES = [
    (1, 1, 1, 32), (2, 80, 3, 256), (1, 17, 16, 2080), (3, 33, 5, 4096), (1, 100, 17, 1024),
    (2, 48, 2, 160), (1, 7, 40, 512), (1, 300, 16, 16384), (2, 31, 9, 320), (1, 64, 4, 64),
    # the defaults by vector count on weights that fill the GPU: one-vector VALU tiles,
    # vectors in registers up to 13, all in LDS from 14
    (1, 7168, 1, 16384), (2, 4100, 1, 2048), (1, 4096, 13, 2048), (1, 4096, 14, 2048),
]


@pytest.mark.parametrize("l,m,n,k", SMALLN_SHAPES)
def test_smalln_default_plan_shapes(l, m, n, k):
    ops = smalln_ops(l, m, n, k, seed=l + m + n + k)
    assert_bits_equal(run_smalln(ops, l, m, n, k), oracle_smalln(ops, l, m, n, k), f"{(l, m, n, k)}")


NUM_MMA_VARIANTS = 20


def valu_tiles(v):
    return pd.nvfp4_mma_variant_form(v) == pd.NVFP4_MMA_FORM_VALU_TILES


def test_mma_variant_count():
    assert pd.nvfp4_mma_num_variants() == NUM_MMA_VARIANTS


@pytest.mark.parametrize("variant", range(1, NUM_MMA_VARIANTS + 1))
@pytest.mark.parametrize("ksplit", [1, 3])
def test_smalln_every_variant(variant, ksplit):
    if ksplit > 1 and valu_tiles(variant):
        pytest.skip("VALU row tiles never split K")
    # ragged rows, k not a multiple of the 256-element window nor of the
    # 2048-element slice, 11 vectors: three passes of 4 for the VALU tiles
    l, m, n, k = 2, 75, 11, 2112
    ops = smalln_ops(l, m, n, k, seed=variant * 10 + ksplit)
    want = oracle_smalln(ops, l, m, n, k, pd.NVFP4_OUT_BF16)
    tuning = {"path": pd.NVFP4_GEMV_PATH_FAST, "variant": variant, "ksplit": ksplit}
    got = run_smalln(ops, l, m, n, k, pd.NVFP4_OUT_BF16, tuning=tuning)
    assert_bits_equal(got, want, f"variant {variant} ksplit {ksplit}", "bf16")


@pytest.mark.parametrize("l,m,n,k", [(1, 9, 4, 48), (2, 21, 3, 2064), (1, 5, 18, 80)])
def test_smalln_generic_path(l, m, n, k):
    ops = smalln_ops(l, m, n, k, seed=7)
    got = run_smalln(ops, l, m, n, k, tuning={"path": pd.NVFP4_GEMV_PATH_GENERIC})
    assert_bits_equal(got, oracle_smalln(ops, l, m, n, k), "generic")


def test_smalln_misaligned_pointers_take_generic_path():
    l, m, n, k = 1, 40, 6, 256
    ops = smalln_ops(l, m, n, k, seed=8)
    d = to_device(ops)
    big = torch.zeros(d["B"].numel() + 3, dtype=torch.uint8, device="cuda")
    big[3:] = d["B"].reshape(-1)
    d["B"] = big[3:]                       # 3 bytes past a 16-byte boundary
    assert pd.nvfp4_gemm_smalln_plan(l, m, n, k, aligned=False)[0].path == pd.NVFP4_GEMV_PATH_GENERIC
    got = run_smalln(ops, l, m, n, k, dev=d)
    assert_bits_equal(got, oracle_smalln(ops, l, m, n, k), "misaligned B")


def test_smalln_special_values_every_variant():
    """Every finite scale code (subnormal, negative, up to 448) on arbitrary
    bytes, plus NaN codes planted in one weight row and one vector.  Terms then
    span many binades, so the fp32 sums are not exact: the tolerance applies,
    and NaN positions must agree exactly."""
    l, m, n, k = 2, 40, 7, 512
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    a = workloads.random_bytes(l, m, k, seed=11, scale_codes=finite)
    b = workloads.random_bytes(l, n, k, seed=12, scale_codes=finite)
    ops = {"A": a["A"], "sfA": a["sfA"], "B": b["A"], "sfB": b["sfA"], "alpha": a["alpha"]}
    ops["sfA"][0, 3, 1] = 0x7F
    ops["sfB"][1, 2, 5] = 0xFF
    want = oracle_smalln(ops, l, m, n, k)
    nan = np.isnan(want.view(np.float16))
    assert nan[0, 3].all() and nan[1, :, 2].all() and nan.sum() == n + m
    for v in range(1, pd.nvfp4_mma_num_variants() + 1):
        got = run_smalln(ops, l, m, n, k, tuning={"variant": v})
        assert_within_tolerance(got, want, what=f"special values variant {v}")


def gaussian_smalln_ops(l, m, n, k, seed):
    """Gaussian bf16 draws quantised by the oracle, each batch's A and B a
    tensor of its own, alpha = gA * gB."""
    rawA = workloads.gaussian_bf16(l, m, k, seed=seed)["A"]
    rawB = workloads.gaussian_bf16(l, n, k, seed=seed + 1)["A"]
    ops = {"A": np.empty((l, m, k // 2), np.uint8), "sfA": np.empty((l, m, k // 16), np.uint8),
           "B": np.empty((l, n, k // 2), np.uint8), "sfB": np.empty((l, n, k // 16), np.uint8),
           "alpha": np.empty(l, np.float32)}
    for b in range(l):
        ops["A"][b], ops["sfA"][b], ga = oq.quantize_nvfp4(rawA[b])
        ops["B"][b], ops["sfB"][b], gb = oq.quantize_nvfp4(rawB[b])
        ops["alpha"][b] = np.float32(ga * gb)
    return ops


@pytest.mark.parametrize("ksplit", [1, 2])
def test_lds_staged_gaussian_within_tolerance(ksplit):
    """Gaussian data (inexact sums) through every LDS-staged variant: ragged
    rows, a K tail of one lane piece, waves whose K runs end mid-group, and
    rows per block below the tiles, against the oracle within tolerance."""
    l, m, n, k = 2, 203, 13, 4160
    ops = gaussian_smalln_ops(l, m, n, k, seed=90 + ksplit)
    dev = to_device(ops)
    want = oracle_smalln(ops, l, m, n, k)
    staged = [v for v in range(1, NUM_MMA_VARIANTS + 1)
              if pd.nvfp4_mma_variant_form(v) in (pd.NVFP4_MMA_FORM_LDS_STAGED,
                                                  pd.NVFP4_MMA_FORM_LDS_VECTOR_REGS)]
    assert staged
    for v in staged:
        for rpb in (0, 13):
            tun = {"variant": v, "ksplit": ksplit, "rows_per_block": rpb}
            got = run_smalln(ops, l, m, n, k, tuning=tun, dev=dev)
            assert_within_tolerance(got, want, what=f"staged variant {v} rpb {rpb} ks {ksplit}")


def test_lds_staged_scales_at_4_byte_alignment():
    """Scale rows that start 4 bytes past a 16-byte boundary (k a multiple of
    256): the LDS-staged variants then copy block scales 4 bytes at a time
    instead of 16, bit for bit the same results."""
    l, m, n, k = 2, 70, 16, 4096
    ops = smalln_ops(l, m, n, k, seed=123)
    want = oracle_smalln(ops, l, m, n, k)
    dev = to_device(ops)
    for key in ("sfA", "sfB"):
        t = dev[key]
        buf = torch.zeros(t.numel() + 16, dtype=torch.uint8, device="cuda")
        buf[4:4 + t.numel()].copy_(t.reshape(-1))
        dev[key] = buf[4:4 + t.numel()].view(t.shape)
        assert dev[key].data_ptr() % 16 == 4
    staged = [v for v in range(1, NUM_MMA_VARIANTS + 1)
              if pd.nvfp4_mma_variant_form(v) in (pd.NVFP4_MMA_FORM_LDS_STAGED,
                                                  pd.NVFP4_MMA_FORM_LDS_VECTOR_REGS)]
    for v in staged:
        for ks in (1, 2):
            got = run_smalln(ops, l, m, n, k, tuning={"variant": v, "ksplit": ks}, dev=dev)
            assert_bits_equal(got, want, f"variant {v} ks {ks}, 4-byte aligned scales")


@pytest.mark.parametrize("n", [1, 2])
def test_smalln_valu_tiles_gaussian_within_tolerance(n):
    """One or two vectors on a weight that fills the GPU: the default plan
    takes the VALU row tiles."""
    l, m, k = 1, 4096, 4096
    assert pd.nvfp4_mma_variant_form(pd.nvfp4_gemm_smalln_plan(l, m, n, k)[0].variant) == \
        pd.NVFP4_MMA_FORM_VALU_TILES
    ops = gaussian_smalln_ops(l, m, n, k, seed=60 + n)
    for out_type in (pd.NVFP4_OUT_F16, pd.NVFP4_OUT_BF16):
        want = oracle_smalln(ops, l, m, n, k, out_type)
        got = run_smalln(ops, l, m, n, k, out_type)
        assert_within_tolerance(got, want, what=f"gaussian VALU tiles n={n}", fmt=FMT[out_type])


def test_smalln_gaussian_within_tolerance():
    l, m, n, k = 4, 512, 8, 4096
    rawA = workloads.gaussian_bf16(l, m, k, seed=21)["A"]
    rawB = workloads.gaussian_bf16(l, n, k, seed=22)["A"]
    ops = {"A": np.empty((l, m, k // 2), np.uint8), "sfA": np.empty((l, m, k // 16), np.uint8),
           "B": np.empty((l, n, k // 2), np.uint8), "sfB": np.empty((l, n, k // 16), np.uint8),
           "alpha": np.empty(l, np.float32)}
    for b in range(l):
        ops["A"][b], ops["sfA"][b], ga = oq.quantize_nvfp4(rawA[b])
        ops["B"][b], ops["sfB"][b], gb = oq.quantize_nvfp4(rawB[b])
        ops["alpha"][b] = np.float32(ga * gb)
    for out_type in (pd.NVFP4_OUT_F16, pd.NVFP4_OUT_BF16):
        want = oracle_smalln(ops, l, m, n, k, out_type)
        got = run_smalln(ops, l, m, n, k, out_type)
        assert_within_tolerance(got, want, what="gaussian small-N", fmt=FMT[out_type])
        print(f"gaussian small-N {FMT[out_type]}: {float(np.mean(got == want)):.6f} bit-identical")


def test_smalln_zero_scales_give_positive_zero_and_alpha_null():
    l, m, n, k = 1, 32, 4, 256
    ops = smalln_ops(l, m, n, k, seed=13)
    ops["sfB"][:] = 0
    got = run_smalln(ops, l, m, n, k, use_alpha=False)
    assert np.all(got == 0)
    ops = smalln_ops(l, m, n, k, seed=14)
    got = run_smalln(ops, l, m, n, k, use_alpha=False)
    assert_bits_equal(got, oracle_smalln(ops, l, m, n, k, use_alpha=False), "alpha NULL")


def test_smalln_negative_zero_codes_give_positive_zero():
    l, m, n, k = 1, 16, 16, 128
    ops = smalln_ops(l, m, n, k, seed=15)
    ops["A"][:] = 0x88                     # every weight code is -0
    got = run_smalln(ops, l, m, n, k)
    assert np.all(got == 0x0000)


def test_smalln_run_to_run_determinism_with_split():
    l, m, n, k = 1, 200, 16, 8192
    rawA = workloads.gaussian_bf16(1, m, k, seed=31)["A"][0]
    rawB = workloads.gaussian_bf16(1, n, k, seed=32)["A"][0]
    A, sA, _ = oq.quantize_nvfp4(rawA)
    B, sB, _ = oq.quantize_nvfp4(rawB)
    ops = {"A": A[None], "sfA": sA[None], "B": B[None], "sfB": sB[None],
           "alpha": np.ones(1, np.float32)}
    d = to_device(ops)
    tuning = {"ksplit": 4}
    first = run_smalln(ops, l, m, n, k, tuning=tuning, dev=d)
    for _ in range(3):
        assert np.array_equal(run_smalln(ops, l, m, n, k, tuning=tuning, dev=d), first)


# ---------------------------------------------------------------- grouped (MoE) GEMV
def run_grouped(ops, tokens, experts, n, k, out_type=pd.NVFP4_OUT_BF16, tuning=None, scales=True):
    d = to_device(ops)
    c = torch.full((max(tokens, 1), n), FILL - 65536, dtype=torch.int16, device="cuda")
    gx, gw = (d["gs_x"], d["gs_w"]) if scales else (None, None)
    args = (d["X"], d["sfX"], d["W"], d["sfW"], d["offsets"], gx, gw, c, tokens, experts, n, k,
            out_type)
    if tuning is None:
        pd.nvfp4_grouped_gemv_launch(*args)
    else:
        pd.nvfp4_grouped_gemv_launch_tuned(*args, tuning)
    torch.cuda.synchronize()
    return c.cpu().numpy().view(np.uint16)[:tokens]


def oracle_grouped(ops, tokens, experts, n, k, out_type=pd.NVFP4_OUT_BF16, scales=True):
    return multi.grouped_gemv(ops["X"], ops["sfX"], ops["W"], ops["sfW"], ops["offsets"],
                              ops["gs_x"] if scales else None, ops["gs_w"] if scales else None,
                              tokens, experts, n, k, FMT[out_type], fill=FILL)


def grouped_ops(counts, n, k, seed=0):
    experts, tokens = len(counts), int(sum(counts))
    w = workloads.integer_coded(experts, n, k, seed=seed)
    x = workloads.integer_coded(1, max(tokens, 1), k, seed=seed + 1)
    rng = np.random.default_rng(seed + 2)
    return {"X": x["A"][0][:max(tokens, 1)], "sfX": x["sfA"][0][:max(tokens, 1)], "W": w["A"],
            "sfW": w["sfA"], "offsets": np.cumsum(counts).astype(np.int32),
            "gs_x": rng.uniform(0.5, 2, experts).astype(np.float32),
            "gs_w": rng.uniform(0.5, 2, experts).astype(np.float32)}


@pytest.mark.parametrize("name", list(workloads.MOE_CONFIGS))
@pytest.mark.parametrize("out_type", [pd.NVFP4_OUT_F16, pd.NVFP4_OUT_BF16])
def test_grouped_configs_bit_exact(name, out_type):
    cfg = workloads.MOE_CONFIGS[name]
    ops = workloads.moe_operands(cfg)
    want = oracle_grouped(ops, cfg.tokens, cfg.experts, cfg.n, cfg.k, out_type)
    got = run_grouped(ops, cfg.tokens, cfg.experts, cfg.n, cfg.k, out_type)
    assert_bits_equal(got, want, name, FMT[out_type])


@pytest.mark.parametrize("counts,n,k", [
    ([3, 0, 1, 5], 40, 256),          # an expert without tokens, ragged rows
    ([0, 0, 37], 17, 2112),           # more than two passes of 16 tokens
    ([1], 1, 32),
    ([16, 16], 33, 512),
    ([2, 1, 0, 0, 4, 9], 96, 1024),
])
@pytest.mark.parametrize("variant", range(0, NUM_MMA_VARIANTS + 1))
def test_grouped_shapes_every_variant(counts, n, k, variant):
    ops = grouped_ops(counts, n, k, seed=sum(counts) + n + variant)
    tokens, experts = int(sum(counts)), len(counts)
    want = oracle_grouped(ops, tokens, experts, n, k)
    got = run_grouped(ops, tokens, experts, n, k, tuning={"variant": variant})
    assert_bits_equal(got, want, f"{counts} n={n} k={k} v={variant}", "bf16")


def test_grouped_rows_past_the_last_offset_untouched():
    counts, n, k = [2, 3], 24, 256
    ops = grouped_ops(counts, n, k, seed=41)
    tokens = 9                                    # tokens 5..8 belong to no expert
    extra = workloads.integer_coded(1, tokens, k, seed=42)
    ops["X"], ops["sfX"] = extra["A"][0], extra["sfA"][0]
    got = run_grouped(ops, tokens, 2, n, k)
    want = oracle_grouped(ops, tokens, 2, n, k)
    assert np.all(got[5:] == FILL)
    assert_bits_equal(got[:5], want[:5], "covered rows", "bf16")


def test_grouped_generic_path_and_null_scales():
    counts, n, k = [4, 0, 3], 20, 208            # k % 32 == 16: generic kernel
    ops = grouped_ops(counts, n, k, seed=43)
    for scales in (True, False):
        want = oracle_grouped(ops, 7, 3, n, k, scales=scales)
        got = run_grouped(ops, 7, 3, n, k, scales=scales)
        assert_bits_equal(got, want, f"generic scales={scales}", "bf16")
    ops = grouped_ops(counts, n, 256, seed=44)
    got = run_grouped(ops, 7, 3, n, 256, tuning={"path": pd.NVFP4_GEMV_PATH_GENERIC})
    assert_bits_equal(got, oracle_grouped(ops, 7, 3, n, 256), "generic forced", "bf16")


def test_grouped_out_of_range_offsets_stay_in_bounds():
    """Offsets past the token count are clamped on the device: the call reads
    and writes only the arrays it was given."""
    counts, n, k = [3, 2], 16, 128
    ops = grouped_ops(counts, n, k, seed=45)
    ops["offsets"] = np.array([3, 1000], dtype=np.int32)
    got = run_grouped(ops, 5, 2, n, k)
    ops["offsets"] = np.array([3, 5], dtype=np.int32)
    assert_bits_equal(got, oracle_grouped(ops, 5, 2, n, k), "clamped offsets", "bf16")


def test_grouped_zero_tokens_is_a_no_op():
    ops = grouped_ops([0, 0], 16, 64, seed=46)
    got = run_grouped(ops, 0, 2, 16, 64)
    assert got.size == 0


@pytest.mark.parametrize("variant", range(1, NUM_MMA_VARIANTS + 1))
@pytest.mark.parametrize("rows_per_block,ksplit", [(1, 1), (3, 1), (7, 2), (14, 1), (16, 3), (32, 1)])
def test_smalln_rows_per_block(variant, rows_per_block, ksplit):
    r, _, _ = pd.nvfp4_mma_variant_info(variant)
    most = r if valu_tiles(variant) else 16 * r
    if rows_per_block > most:
        pytest.skip("more rows than the variant's tiles hold")
    if ksplit > 1 and valu_tiles(variant):
        pytest.skip("VALU row tiles never split K")
    l, m, n, k = 2, 45, 5, 1088
    ops = smalln_ops(l, m, n, k, seed=100 + variant * 7 + rows_per_block)
    tuning = {"variant": variant, "ksplit": ksplit, "rows_per_block": rows_per_block}
    got = run_smalln(ops, l, m, n, k, pd.NVFP4_OUT_BF16, tuning=tuning)
    assert_bits_equal(got, oracle_smalln(ops, l, m, n, k, pd.NVFP4_OUT_BF16),
                      f"v{variant} rpb {rows_per_block} ks {ksplit}", "bf16")


@pytest.mark.parametrize("variant,rows_per_block", [(1, 5), (3, 20), (4, 31), (2, 16), (7, 3),
                                                    (8, 5), (10, 1)])
def test_grouped_rows_per_block(variant, rows_per_block):
    counts, n, k = [3, 0, 18, 1], 70, 512
    ops = grouped_ops(counts, n, k, seed=200 + rows_per_block)
    want = oracle_grouped(ops, 22, 4, n, k)
    got = run_grouped(ops, 22, 4, n, k, tuning={"variant": variant, "rows_per_block": rows_per_block})
    assert_bits_equal(got, want, f"grouped v{variant} rpb {rows_per_block}", "bf16")


def test_grouped_special_values_every_variant():
    """Terms span many binades, so fp32 sums are not exact: the tolerance
    applies, and NaN positions (a row of an expert, a token) must agree."""
    counts, n, k = [3, 4, 0, 5], 24, 512
    ops = grouped_special_ops(counts, n, k, seed=81)
    tokens, experts = int(sum(counts)), len(counts)
    for out_type in (pd.NVFP4_OUT_F16, pd.NVFP4_OUT_BF16):
        want = oracle_grouped(ops, tokens, experts, n, k, out_type)
        nan = np.isnan(bits_to_f64(want, FMT[out_type]))
        assert nan[3:7, 3].all() and nan[tokens - 1].all()
        for v in range(0, pd.nvfp4_mma_num_variants() + 1):
            got = run_grouped(ops, tokens, experts, n, k, out_type, tuning={"variant": v})
            assert_within_tolerance(got, want, what=f"grouped special v{v}", fmt=FMT[out_type])


def test_grouped_gaussian_within_tolerance():
    experts, n, k = 6, 256, 2048
    counts = [3, 0, 1, 2, 5, 1]
    tokens = int(sum(counts))
    rawW = workloads.gaussian_bf16(experts, n, k, seed=91)["A"]
    rawX = workloads.gaussian_bf16(1, tokens, k, seed=92)["A"][0]
    W = np.empty((experts, n, k // 2), np.uint8)
    sW = np.empty((experts, n, k // 16), np.uint8)
    gw = np.empty(experts, np.float32)
    for e in range(experts):
        W[e], sW[e], gw[e] = oq.quantize_nvfp4(rawW[e])
    X, sX, gx = oq.quantize_nvfp4(rawX)          # the tokens as one tensor: one activation scale
    ops = {"X": X, "sfX": sX, "W": W, "sfW": sW, "offsets": np.cumsum(counts).astype(np.int32),
           "gs_x": np.full(experts, gx, np.float32), "gs_w": gw}
    for out_type in (pd.NVFP4_OUT_F16, pd.NVFP4_OUT_BF16):
        want = oracle_grouped(ops, tokens, experts, n, k, out_type)
        got = run_grouped(ops, tokens, experts, n, k, out_type)
        assert_within_tolerance(got, want, what="gaussian grouped", fmt=FMT[out_type])
