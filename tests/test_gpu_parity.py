"""GPU parity: the HIP library (called through its C ABI) against the CPU oracle.

Integer-coded inputs must match bit for bit (every fp32 partial sum is exact,
so the result does not depend on summation order); the Gaussian-quantised
workload must agree within max(2 fp16 ulp, 1e-3 relative).
"""
import numpy as np
import pytest
import torch

import precision_decode_amd as pd
import workloads
from golden_io import hand_examples
from gpu_util import assert_bits_equal, assert_within_tolerance, run_gpu, to_device
from oracle import quantize as oq
from oracle import reference as ref

pytestmark = [pytest.mark.gpu, pytest.mark.filterwarnings("ignore::RuntimeWarning")]


@pytest.fixture(scope="module", autouse=True)
def gpu_ready():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    pd.load()


def oracle_out(ops, l, m, k, use_alpha=True):
    return ref.gemv(ops["A"], ops["sfA"], ops["x"], ops["sfx"], ops["alpha"] if use_alpha else None,
                    l, m, k)


# ---------------------------------------------------------------- the five workloads
@pytest.mark.parametrize("name", ["tiny", "decode", "batched", "shortk"])
def test_integer_coded_configs_bit_exact(name):
    cfg = workloads.CONFIGS[name]
    ops = workloads.for_config(cfg)
    want = oracle_out(ops, cfg.l, cfg.m, cfg.k)
    got = run_gpu(to_device(ops), cfg.l, cfg.m, cfg.k)
    assert_bits_equal(got, want, name)


def test_gaussian_config_within_tolerance():
    cfg = workloads.CONFIGS["gaussian"]
    raw = workloads.gaussian_bf16(cfg.l, cfg.m, cfg.k, seed=cfg.seed)
    ops = oq.gaussian_operands(raw, cfg.l, cfg.m, cfg.k)
    want = oracle_out(ops, cfg.l, cfg.m, cfg.k)
    got = run_gpu(to_device(ops), cfg.l, cfg.m, cfg.k)
    assert_within_tolerance(got, want, what="gaussian")
    exact = float(np.mean(got == want))
    print(f"gaussian: {exact:.6f} of outputs bit-identical to the oracle")


# ---------------------------------------------------------------- hand examples
@pytest.mark.parametrize("ex", hand_examples(), ids=lambda e: e["name"])
def test_hand_examples_on_gpu(ex):
    ops = {n: ex[n] for n in ("A", "sfA", "x", "sfx", "alpha")}
    got = run_gpu(to_device(ops), 1, 1, ex["k"])
    assert int(got[0, 0]) == ex["c"], hex(int(got[0, 0]))


# ---------------------------------------------------------------- exhaustive decode
def test_every_e4m3_code_as_weight_scale():
    m, k = 256, 64
    ops = workloads.integer_coded(1, m, k, seed=1)
    ops["A"][:] = 0
    ops["A"][0, :, 0] = 0x02                      # element 0 = 1.0
    ops["sfA"][0, :, 0] = np.arange(256, dtype=np.uint8)
    ops["x"][:] = 0
    ops["x"][0, 0] = 0x02
    ops["sfx"][:] = 0x38
    want = oracle_out(ops, 1, m, k)
    assert_bits_equal(run_gpu(to_device(ops), 1, m, k), want, "sfA codes")


def test_every_e4m3_code_as_vector_scale():
    l, m, k = 256, 2, 64
    ops = workloads.integer_coded(l, m, k, seed=2)
    ops["A"][:] = 0
    ops["A"][:, :, 8] = 0x20                      # element 17 = 1.0 (block 1)
    ops["sfA"][:] = 0x38
    ops["x"][:] = 0
    ops["x"][:, 8] = 0x20
    ops["sfx"][:, 1] = np.arange(256, dtype=np.uint8)
    want = oracle_out(ops, l, m, k)
    assert_bits_equal(run_gpu(to_device(ops), l, m, k), want, "sfx codes")


@pytest.mark.parametrize("pos", [0, 5, 10, 15])
def test_every_byte_in_every_position(pos):
    """All 256 byte values of A against all 256 byte values of x, at byte
    positions that land in different 32-bit words and byte selects."""
    l, m, k = 256, 256, 64
    ops = workloads.integer_coded(l, m, k, seed=3)
    ops["A"][:] = 0
    ops["A"][:, :, pos] = np.arange(256, dtype=np.uint8)[None, :]
    ops["x"][:] = 0
    ops["x"][:, pos] = np.arange(256, dtype=np.uint8)
    ops["sfA"][:] = 0x38
    ops["sfx"][:] = 0x40
    want = oracle_out(ops, l, m, k)
    assert_bits_equal(run_gpu(to_device(ops), l, m, k), want, f"byte pos {pos}")


# ---------------------------------------------------------------- shapes and paths
EDGE_SHAPES = [
    (1, 1, 32), (1, 1, 16), (3, 5, 48), (2, 9, 2080), (1, 13, 4128), (37, 3, 64),
    (1, 1000, 256), (2, 7, 16416), (1, 3, 65536), (5, 129, 7168), (1, 4099, 1024),
    (2, 63, 2048), (1, 8, 14336),
]


@pytest.mark.parametrize("l,m,k", EDGE_SHAPES)
def test_edge_shapes_default_plan(l, m, k):
    ops = workloads.integer_coded(l, m, k, seed=l * 1000 + m + k, alpha="uniform")
    want = oracle_out(ops, l, m, k)
    assert_bits_equal(run_gpu(to_device(ops), l, m, k), want, f"{(l, m, k)}")


@pytest.mark.parametrize("l,m,k", [(1, 1, 32), (3, 5, 48), (2, 9, 2080), (5, 129, 7168)])
@pytest.mark.parametrize("ksplit", [1, 3])
def test_generic_kernel(l, m, k, ksplit):
    if ksplit > k // 16:
        pytest.skip("fewer 16-element blocks than splits")
    ops = workloads.integer_coded(l, m, k, seed=7, alpha="uniform")
    want = oracle_out(ops, l, m, k)
    tun = {"path": pd.NVFP4_GEMV_PATH_GENERIC, "ksplit": ksplit}
    assert_bits_equal(run_gpu(to_device(ops), l, m, k, tuning=tun), want, "generic")


NUM_VARIANTS = 33


def test_variant_count():
    assert pd.nvfp4_gemv_num_variants() == NUM_VARIANTS


@pytest.mark.parametrize("variant", range(1, NUM_VARIANTS + 1))
@pytest.mark.parametrize("ksplit", [1, 2, 5])
def test_every_variant_and_split(variant, ksplit):
    l, m, k = 2, 77, 10240
    ops = workloads.integer_coded(l, m, k, seed=variant * 10 + ksplit, alpha="uniform")
    want = oracle_out(ops, l, m, k)
    tun = {"path": pd.NVFP4_GEMV_PATH_FAST, "variant": variant, "ksplit": ksplit}
    assert_bits_equal(run_gpu(to_device(ops), l, m, k, tuning=tun), want, f"v{variant} ks{ksplit}")


@pytest.mark.parametrize("l,m,k", [(3, 100, 4096), (1, 1, 32), (5, 129, 7168), (2, 9, 2080),
                                   (37, 3, 64), (1, 3, 16384)])
def test_every_variant_on_ragged_shapes(l, m, k):
    ops = workloads.integer_coded(l, m, k, seed=l + m + k, alpha="uniform")
    want = oracle_out(ops, l, m, k)
    d = to_device(ops)
    for v in range(1, pd.nvfp4_gemv_num_variants() + 1):
        got = run_gpu(d, l, m, k, tuning={"path": pd.NVFP4_GEMV_PATH_FAST, "variant": v})
        assert_bits_equal(got, want, f"v{v} {(l, m, k)}")


def test_every_variant_gaussian_and_special_values():
    cfg = workloads.CONFIGS["gaussian"]
    raw = workloads.gaussian_bf16(2, cfg.m, cfg.k, seed=4)
    ops = oq.gaussian_operands(raw, 2, cfg.m, cfg.k)
    want = oracle_out(ops, 2, cfg.m, cfg.k)
    d = to_device(ops)
    sp = workloads.random_bytes(2, 70, 4096, seed=15)
    want_sp = oracle_out(sp, 2, 70, 4096)
    dsp = to_device(sp)
    for v in range(1, pd.nvfp4_gemv_num_variants() + 1):
        tun = {"path": pd.NVFP4_GEMV_PATH_FAST, "variant": v}
        assert_within_tolerance(run_gpu(d, 2, cfg.m, cfg.k, tuning=tun), want, what=f"v{v} gaussian")
        assert_bits_equal(run_gpu(dsp, 2, 70, 4096, tuning=tun), want_sp, f"v{v} all scale codes")


def test_misaligned_pointers_take_generic_path():
    l, m, k = 2, 33, 256
    ops = workloads.integer_coded(l, m, k, seed=8, alpha="uniform")
    want = oracle_out(ops, l, m, k)
    bufs, ptrs = [], {}
    for i, name in enumerate(("A", "sfA", "x", "sfx")):
        arr = ops[name].reshape(-1)
        off = 1 + 2 * i
        buf = torch.zeros(arr.size + 32, dtype=torch.uint8, device="cuda")
        buf[off:off + arr.size] = torch.from_numpy(arr).cuda()
        bufs.append(buf)
        ptrs[name] = buf.data_ptr() + off
    alpha = torch.from_numpy(ops["alpha"]).cuda()
    c = torch.full((l, m), -1, dtype=torch.int16, device="cuda")
    pd.nvfp4_gemv_launch(ptrs["A"], ptrs["sfA"], ptrs["x"], ptrs["sfx"], alpha, c, l, m, k)
    torch.cuda.synchronize()
    assert_bits_equal(c.cpu().numpy().view(np.uint16), want, "misaligned")


# ---------------------------------------------------------------- workspace and streams
def test_owned_and_caller_workspace_agree():
    l, m, k = 1, 896, 16384                          # one eighth of the decode weight: split K
    plan, ws_bytes = pd.nvfp4_gemv_plan(l, m, k)
    assert plan.ksplit > 1 and ws_bytes > 0
    ops = workloads.integer_coded(l, m, k, seed=9)
    want = oracle_out(ops, l, m, k)
    d = to_device(ops)
    assert_bits_equal(run_gpu(d, l, m, k, mode="launch"), want, "owned ws")
    assert_bits_equal(run_gpu(d, l, m, k, mode="ws"), want, "caller ws")


def test_two_streams_do_not_share_workspace():
    l, m, k = 1, 448, 16384
    o1 = workloads.integer_coded(l, m, k, seed=10)
    o2 = workloads.integer_coded(l, m, k, seed=11)
    w1, w2 = oracle_out(o1, l, m, k), oracle_out(o2, l, m, k)
    d1, d2 = to_device(o1), to_device(o2)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    c1 = torch.empty((l, m), dtype=torch.int16, device="cuda")
    c2 = torch.empty((l, m), dtype=torch.int16, device="cuda")
    torch.cuda.synchronize()
    for _ in range(3):
        pd.nvfp4_gemv_launch(d1["A"], d1["sfA"], d1["x"], d1["sfx"], d1["alpha"], c1, l, m, k, stream=s1)
        pd.nvfp4_gemv_launch(d2["A"], d2["sfA"], d2["x"], d2["sfx"], d2["alpha"], c2, l, m, k, stream=s2)
    torch.cuda.synchronize()
    assert_bits_equal(c1.cpu().numpy().view(np.uint16), w1, "stream 1")
    assert_bits_equal(c2.cpu().numpy().view(np.uint16), w2, "stream 2")


def test_run_to_run_determinism():
    cfg = workloads.CONFIGS["decode"]
    d = to_device(workloads.for_config(cfg))
    a = run_gpu(d, cfg.l, cfg.m, cfg.k)
    b = run_gpu(d, cfg.l, cfg.m, cfg.k)
    s = run_gpu(d, cfg.l, cfg.m, cfg.k, tuning={"ksplit": 4})
    assert np.array_equal(a, b) and np.array_equal(a, s)


# ---------------------------------------------------------------- special values
def test_alpha_null_means_one():
    l, m, k = 3, 50, 512
    ops = workloads.integer_coded(l, m, k, seed=12, alpha="uniform")
    want = oracle_out(ops, l, m, k, use_alpha=False)
    assert_bits_equal(run_gpu(to_device(ops), l, m, k, use_alpha=False), want, "alpha NULL")


def test_zero_scales_give_positive_zero():
    l, m, k = 2, 40, 2048
    ops = workloads.integer_coded(l, m, k, seed=13)
    ops["sfA"][:] = 0
    got = run_gpu(to_device(ops), l, m, k)
    assert (got == 0).all()


def test_nan_and_negative_scales_and_overflow():
    l, m, k = 2, 70, 4096
    ops = workloads.random_bytes(l, m, k, seed=14)     # scales from all 256 codes
    want = oracle_out(ops, l, m, k)
    assert np.isnan(want.view(np.float16)).any()
    assert_bits_equal(run_gpu(to_device(ops), l, m, k), want, "all scale codes")
    big = workloads.integer_coded(1, 16, 4096, seed=15)
    big["A"][:] = 0x77
    big["x"][:] = 0x77
    big["sfA"][:] = 0x7E
    big["sfx"][:] = 0x7E
    want = oracle_out(big, 1, 16, 4096)
    assert (want == 0x7C00).all()
    assert_bits_equal(run_gpu(to_device(big), 1, 16, 4096), want, "overflow")


@pytest.mark.parametrize("n", [64 << 20, (64 << 20) + 48, 300 << 20, 16, (16 << 10) + 16])
def test_hbm_read_probe_reads_every_byte_once(n):
    """16 KiB chunks, one per workgroup: exactly the group cap (4096 chunks),
    a ragged chunk past the cap (one group takes two), several chunks per
    group with a partial last round, a single 16-byte unit, and two chunks
    of which the second holds one unit."""
    data = torch.randint(0, 2 ** 31 - 1, (n // 4,), dtype=torch.int32, device="cuda")
    sink = torch.zeros(4096, dtype=torch.int32, device="cuda")
    print(f"probe over {n} bytes", flush=True)
    pd.nvfp4_hbm_read_probe(data, n, sink)
    torch.cuda.synchronize()
    want = np.bitwise_xor.reduce(data.cpu().numpy().view(np.uint32))
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    assert got == want


@pytest.mark.parametrize("rows,k", [(7168, 16384), (29, 2048), (15, 7168), (1, 32), (100, 4128)])
def test_hbm_read_probe_rows_reads_every_byte_once(rows, k):
    """Whole and ragged workgroups (14 rows each), rows shorter than one
    iteration, K not a multiple of the 4 KiB in flight."""
    print(f"row probe over {rows} x {k}", flush=True)
    g = torch.Generator().manual_seed(rows * 7 + k)
    a = torch.randint(0, 256, (rows * k // 2,), dtype=torch.uint8, generator=g)
    s = torch.randint(0, 256, (rows * k // 16,), dtype=torch.uint8, generator=g)
    groups = -(-rows // 14)
    sink = torch.zeros(groups, dtype=torch.int32, device="cuda")
    pd.nvfp4_hbm_read_probe_rows(a.cuda(), s.cuda(), rows, k, sink)
    torch.cuda.synchronize()

    # the probe XORs 16-byte code chunks and 2-byte scale pairs: fold both to 32 bits
    want = np.bitwise_xor.reduce(a.numpy().view(np.uint32))
    sv = s.numpy().view(np.uint16).astype(np.uint32)
    want ^= np.bitwise_xor.reduce(sv) if sv.size else np.uint32(0)
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    assert got == want
