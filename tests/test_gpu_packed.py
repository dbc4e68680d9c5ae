"""GPU checks of the packed-weight calls: nvfp4_mma_pack_weight writes the
layout that include/nvfp4_mma.h defines (byte for byte, against a numpy
re-layout written from that definition), and the small-N GEMM and grouped GEMV
on packed weights match the CPU oracle on the row-major weights bit for bit
(integer-coded inputs), for every matrix-core variant, K splits, ragged rows
and K not a multiple of the 256-element window."""
import numpy as np
import pytest
import torch

import precision_decode_amd as pd
import workloads
from gpu_util import assert_bits_equal, assert_within_tolerance, grouped_special_ops, to_device
from oracle import multi
from oracle import quantize as oq

pytestmark = [pytest.mark.gpu, pytest.mark.filterwarnings("ignore::RuntimeWarning")]

FMT = {pd.NVFP4_OUT_F16: "f16", pd.NVFP4_OUT_BF16: "bf16"}
FILL = 0xFFFF


@pytest.fixture(scope="module", autouse=True)
def gpu_ready():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    pd.load()


def matrix_core_variants():
    return [v for v in range(1, pd.nvfp4_mma_num_variants() + 1)
            if pd.nvfp4_mma_variant_form(v) == pd.NVFP4_MMA_FORM_MATRIX_CORES]


def relayout(W, sW, groups, rows, k):
    """The packed layout of the header, from its definition: block
    (g, t, w) of 2048 code bytes and 256 scale bytes; lane l = i + 16 q holds
    code bytes 128 w + 32 q .. +31 of row 16 t + i (two 16-byte halves at 16 l
    and 1024 + 16 l) and scale bytes 16 w + 4 q .. +3 at 4 l."""
    tiles, wins = -(-rows // 16), -(-k // 256)
    Wz = np.zeros((groups, tiles * 16, wins * 128), np.uint8)
    Sz = np.zeros((groups, tiles * 16, wins * 16), np.uint8)
    Wz[:, :rows, :k // 2] = W.reshape(groups, rows, k // 2)
    Sz[:, :rows, :k // 16] = sW.reshape(groups, rows, k // 16)
    codes = np.zeros((groups, tiles, wins, 2, 64, 16), np.uint8)
    scales = np.zeros((groups, tiles, wins, 64, 4), np.uint8)
    for lane in range(64):
        i, q = lane % 16, lane // 16
        for w in range(wins):
            for h in range(2):
                b = 128 * w + 32 * q + 16 * h
                codes[:, :, w, h, lane, :] = Wz[:, i::16, b:b + 16]
            sb = 16 * w + 4 * q
            scales[:, :, w, lane, :] = Sz[:, i::16, sb:sb + 4]
    return codes.reshape(-1), scales.reshape(-1)


def pack(W, sW, groups, rows, k):
    cb, sb = pd.nvfp4_mma_packed_sizes(groups, rows, k)
    Wp = torch.full((cb,), 0xAB, dtype=torch.uint8, device="cuda")   # poisoned: every byte is written
    sWp = torch.full((sb,), 0xAB, dtype=torch.uint8, device="cuda")
    pd.nvfp4_mma_pack_weight(W, sW, groups, rows, k, Wp, sWp)
    torch.cuda.synchronize()
    return Wp, sWp


@pytest.mark.parametrize("groups,rows,k", [(1, 16, 256), (2, 75, 2112), (3, 33, 64), (1, 7168, 16384),
                                           (5, 20, 576)])
def test_pack_layout_matches_the_definition(groups, rows, k):
    ops = workloads.integer_coded(groups, rows, k, seed=groups + rows + k)
    d = to_device(ops)
    Wp, sWp = pack(d["A"], d["sfA"], groups, rows, k)
    want_c, want_s = relayout(ops["A"], ops["sfA"], groups, rows, k)
    assert Wp.numel() == want_c.size and sWp.numel() == want_s.size
    assert np.array_equal(Wp.cpu().numpy(), want_c)
    assert np.array_equal(sWp.cpu().numpy(), want_s)


# ---------------------------------------------------------------- small-N GEMM
def smalln_ops(l, m, n, k, seed=0):
    a = workloads.integer_coded(l, m, k, seed=seed, alpha="uniform")
    b = workloads.integer_coded(l, n, k, seed=seed + 1)
    return {"A": a["A"], "sfA": a["sfA"], "B": b["A"], "sfB": b["sfA"], "alpha": a["alpha"]}


def run_smalln_packed(ops, l, m, n, k, out_type=pd.NVFP4_OUT_F16, tuning=None):
    d = to_device(ops)
    Ap, sAp = pack(d["A"], d["sfA"], l, m, k)
    c = torch.full((l, m, n), -1, dtype=torch.int16, device="cuda")
    pd.nvfp4_gemm_smalln_launch_packed(Ap, sAp, d["B"], d["sfB"], d["alpha"], c, l, m, n, k, out_type,
                                       tuning)
    torch.cuda.synchronize()
    return c.cpu().numpy().view(np.uint16)


def oracle_smalln(ops, l, m, n, k, out_type=pd.NVFP4_OUT_F16):
    return multi.gemm_smalln(ops["A"], ops["sfA"], ops["B"], ops["sfB"], ops["alpha"], l, m, n, k,
                             FMT[out_type])


@pytest.mark.parametrize("ksplit", [0, 1, 3])
def test_smalln_packed_every_variant(ksplit):
    l, m, n, k = 2, 75, 11, 2112        # ragged rows, k = 8 windows + 64 elements
    ops = smalln_ops(l, m, n, k, seed=31 + ksplit)
    want = oracle_smalln(ops, l, m, n, k, pd.NVFP4_OUT_BF16)
    for v in matrix_core_variants():
        tuning = {"variant": v, "ksplit": ksplit}
        got = run_smalln_packed(ops, l, m, n, k, pd.NVFP4_OUT_BF16, tuning)
        assert_bits_equal(got, want, f"packed v{v} ks{ksplit}", "bf16")


@pytest.mark.parametrize("l,m,n,k", [(1, 7168, 16, 16384), (1, 7168, 4, 16384), (3, 40, 1, 64),
                                     (2, 130, 17, 1024)])
def test_smalln_packed_default_plan(l, m, n, k):
    ops = smalln_ops(l, m, n, k, seed=l + m + n + k)
    assert_bits_equal(run_smalln_packed(ops, l, m, n, k), oracle_smalln(ops, l, m, n, k),
                      f"packed {(l, m, n, k)}")


@pytest.mark.parametrize("rows_per_block", [16, 32])
def test_smalln_packed_rows_per_block(rows_per_block):
    l, m, n, k = 1, 100, 5, 1280
    ops = smalln_ops(l, m, n, k, seed=41)
    for v in matrix_core_variants():
        r, _, _ = pd.nvfp4_mma_variant_info(v)
        if rows_per_block > 16 * r:
            continue
        got = run_smalln_packed(ops, l, m, n, k, tuning={"variant": v, "rows_per_block": rows_per_block})
        assert_bits_equal(got, oracle_smalln(ops, l, m, n, k), f"packed v{v} rpb {rows_per_block}")


# ---------------------------------------------------------------- grouped GEMV
def grouped_ops(counts, n, k, seed=0):
    experts, tokens = len(counts), int(sum(counts))
    w = workloads.integer_coded(experts, n, k, seed=seed)
    x = workloads.integer_coded(1, max(tokens, 1), k, seed=seed + 1)
    rng = np.random.default_rng(seed + 2)
    return {"X": x["A"][0][:max(tokens, 1)], "sfX": x["sfA"][0][:max(tokens, 1)], "W": w["A"],
            "sfW": w["sfA"], "offsets": np.cumsum(counts).astype(np.int32),
            "gs_x": rng.uniform(0.5, 2, experts).astype(np.float32),
            "gs_w": rng.uniform(0.5, 2, experts).astype(np.float32)}


def run_grouped_packed(ops, tokens, experts, n, k, out_type=pd.NVFP4_OUT_BF16, tuning=None):
    d = to_device(ops)
    Wp, sWp = pack(d["W"], d["sfW"], experts, n, k)
    c = torch.full((max(tokens, 1), n), FILL - 65536, dtype=torch.int16, device="cuda")
    pd.nvfp4_grouped_gemv_launch_packed(d["X"], d["sfX"], Wp, sWp, d["offsets"], d["gs_x"], d["gs_w"],
                                        c, tokens, experts, n, k, out_type, tuning)
    torch.cuda.synchronize()
    return c.cpu().numpy().view(np.uint16)[:tokens]


def oracle_grouped(ops, tokens, experts, n, k, out_type=pd.NVFP4_OUT_BF16):
    return multi.grouped_gemv(ops["X"], ops["sfX"], ops["W"], ops["sfW"], ops["offsets"],
                              ops["gs_x"], ops["gs_w"], tokens, experts, n, k, FMT[out_type],
                              fill=FILL)


@pytest.mark.parametrize("counts,n,k", [
    ([3, 0, 1, 5], 40, 256),
    ([0, 0, 37], 17, 2112),
    ([16, 16], 33, 512),
    ([2, 1, 0, 0, 4, 9], 96, 1088),
])
def test_grouped_packed_every_variant(counts, n, k):
    ops = grouped_ops(counts, n, k, seed=sum(counts) + n)
    tokens, experts = int(sum(counts)), len(counts)
    want = oracle_grouped(ops, tokens, experts, n, k)
    for v in [0] + matrix_core_variants():
        got = run_grouped_packed(ops, tokens, experts, n, k, tuning={"variant": v})
        assert_bits_equal(got, want, f"packed {counts} n={n} k={k} v={v}", "bf16")


def test_grouped_packed_moe_decode():
    cfg = workloads.MOE_CONFIGS["moe_decode"]
    ops = workloads.moe_operands(cfg)
    for out_type in (pd.NVFP4_OUT_F16, pd.NVFP4_OUT_BF16):
        want = oracle_grouped(ops, cfg.tokens, cfg.experts, cfg.n, cfg.k, out_type)
        got = run_grouped_packed(ops, cfg.tokens, cfg.experts, cfg.n, cfg.k, out_type)
        assert_bits_equal(got, want, f"packed moe_decode {FMT[out_type]}", FMT[out_type])


@pytest.mark.parametrize("out_type", [pd.NVFP4_OUT_F16, pd.NVFP4_OUT_BF16])
def test_smalln_packed_gaussian_within_tolerance(out_type):
    """Gaussian bf16 draws quantised by the oracle (each batch's A and B a
    tensor of its own): the packed call agrees with the oracle within the
    tolerance, and with the row-major call bit for bit."""
    l, m, n, k = 2, 300, 16, 4096
    rawA = workloads.gaussian_bf16(l, m, k, seed=71)["A"]
    rawB = workloads.gaussian_bf16(l, n, k, seed=72)["A"]
    ops = {"A": np.empty((l, m, k // 2), np.uint8), "sfA": np.empty((l, m, k // 16), np.uint8),
           "B": np.empty((l, n, k // 2), np.uint8), "sfB": np.empty((l, n, k // 16), np.uint8),
           "alpha": np.empty(l, np.float32)}
    for b in range(l):
        ops["A"][b], ops["sfA"][b], ga = oq.quantize_nvfp4(rawA[b])
        ops["B"][b], ops["sfB"][b], gb = oq.quantize_nvfp4(rawB[b])
        ops["alpha"][b] = np.float32(ga * gb)
    want = oracle_smalln(ops, l, m, n, k, out_type)
    # the same matrix-core plan for both layouts: variant, K split and whole-tile row blocks
    tuning = {"variant": 3, "ksplit": 4, "rows_per_block": 32}
    got = run_smalln_packed(ops, l, m, n, k, out_type, tuning)
    assert_within_tolerance(got, want, what="gaussian packed small-N", fmt=FMT[out_type])
    d = to_device(ops)
    c = torch.full((l, m, n), -1, dtype=torch.int16, device="cuda")
    _, ws_bytes = pd.nvfp4_gemm_smalln_plan(l, m, n, k, tuning=tuning)
    ws = torch.empty(max(ws_bytes, 4), dtype=torch.uint8, device="cuda")
    pd.nvfp4_gemm_smalln_launch_tuned(d["A"], d["sfA"], d["B"], d["sfB"], d["alpha"], c, l, m, n, k,
                                      out_type, tuning, ws, ws_bytes)
    torch.cuda.synchronize()
    assert np.array_equal(got, c.cpu().numpy().view(np.uint16)), "packed and row-major differ"


def test_grouped_packed_special_values_and_clamped_offsets():
    """Every finite scale code and planted NaN scales through packed weights
    (tolerance; NaN positions agree), then offsets past the token count
    (clamped on the device) and a call with no tokens."""
    counts, n, k = [3, 4, 0, 5], 24, 512
    ops = grouped_special_ops(counts, n, k, seed=83)
    tokens, experts = int(sum(counts)), len(counts)
    for out_type in (pd.NVFP4_OUT_F16, pd.NVFP4_OUT_BF16):
        want = oracle_grouped(ops, tokens, experts, n, k, out_type)
        for v in [0] + matrix_core_variants():
            got = run_grouped_packed(ops, tokens, experts, n, k, out_type, tuning={"variant": v})
            assert_within_tolerance(got, want, what=f"packed grouped special v{v}", fmt=FMT[out_type])
    ops = grouped_ops([3, 2], 16, 128, seed=84)
    ops["offsets"] = np.array([3, 1000], dtype=np.int32)
    got = run_grouped_packed(ops, 5, 2, 16, 128)
    ops["offsets"] = np.array([3, 5], dtype=np.int32)
    assert_bits_equal(got, oracle_grouped(ops, 5, 2, 16, 128), "packed clamped offsets", "bf16")
    ops = grouped_ops([0, 0], 16, 64, seed=85)
    assert run_grouped_packed(ops, 0, 2, 16, 64).size == 0


def test_smalln_packed_split_determinism_and_two_streams():
    """Gaussian data with a K split: three packed calls give the same bits;
    then two streams run packed split-K calls on different operands
    concurrently, each taking its own library workspace."""
    l, m, n, k = 1, 200, 16, 8192
    plan = {"ksplit": 4}
    rawA = workloads.gaussian_bf16(1, m, k, seed=101)["A"][0]
    rawB = workloads.gaussian_bf16(1, n, k, seed=102)["A"][0]
    A, sA, _ = oq.quantize_nvfp4(rawA)
    B, sB, _ = oq.quantize_nvfp4(rawB)
    ops = {"A": A[None], "sfA": sA[None], "B": B[None], "sfB": sB[None],
           "alpha": np.ones(1, np.float32)}
    first = run_smalln_packed(ops, l, m, n, k, tuning=plan)
    for _ in range(2):
        assert np.array_equal(run_smalln_packed(ops, l, m, n, k, tuning=plan), first)

    o1 = smalln_ops(l, 448, n, 16384, seed=103)
    o2 = smalln_ops(l, 448, n, 16384, seed=104)
    w1, w2 = oracle_smalln(o1, l, 448, n, 16384), oracle_smalln(o2, l, 448, n, 16384)
    outs = []
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    packed = []
    for o in (o1, o2):
        d = to_device(o)
        Ap, sAp = pack(d["A"], d["sfA"], l, 448, 16384)
        packed.append((Ap, sAp, d))
        outs.append(torch.empty((l, 448, n), dtype=torch.int16, device="cuda"))
    torch.cuda.synchronize()
    for _ in range(3):
        for (Ap, sAp, d), c, s in zip(packed, outs, (s1, s2)):
            pd.nvfp4_gemm_smalln_launch_packed(Ap, sAp, d["B"], d["sfB"], d["alpha"], c, l, 448, n,
                                               16384, pd.NVFP4_OUT_F16, plan, stream=s)
    torch.cuda.synchronize()
    assert_bits_equal(outs[0].cpu().numpy().view(np.uint16), w1, "stream 1")
    assert_bits_equal(outs[1].cpu().numpy().view(np.uint16), w2, "stream 2")


def test_pack_weight_tensor_helper():
    """The tensor-level helper gives the same bytes as the C call, for a 3-D
    and a 2-D weight, and rejects a wrong scale shape."""
    ops = workloads.integer_coded(2, 40, 512, seed=111)
    d = to_device(ops)
    codes, scales = pd.pack_weight(d["A"], d["sfA"])
    want_c, want_s = relayout(ops["A"], ops["sfA"], 2, 40, 512)
    assert np.array_equal(codes.cpu().numpy(), want_c) and np.array_equal(scales.cpu().numpy(), want_s)
    c1, s1 = pd.pack_weight(d["A"][1], d["sfA"][1])
    w1c, w1s = relayout(ops["A"][1:], ops["sfA"][1:], 1, 40, 512)
    assert np.array_equal(c1.cpu().numpy(), w1c) and np.array_equal(s1.cpu().numpy(), w1s)
    with pytest.raises(ValueError):
        pd.pack_weight(d["A"], d["sfA"][:, :, :8])
