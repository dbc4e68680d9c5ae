"""Host-side logic of bench.py (no GPU): argument defaults, the one-GPU rule,
the roofline fields and the lookup of recorded HBM traffic."""
import os

import pytest

import bench


def test_defaults_time_every_gemv_workload_batched_last():
    a = bench.parse_args([])
    assert a.gpus == 1 and a.path == "gemv" and a.config == "all" and a.launch == "graph"
    assert a.steps > 0 and a.warmup > 0 and a.single_launches > 0 and not a.trace_cold
    import workloads
    assert set(bench.GEMV_ORDER) == set(workloads.CONFIGS)
    assert bench.GEMV_ORDER[-1] == "batched"          # the line a parser of the last line reads


def test_metric_names_bandwidth_peak_fraction_and_latency():
    m = bench.METRIC
    assert "HBM GB/s" in m and "MI355X peak" in m and "NVFP4 batched GEMV" in m and "\u00b5s/call" in m


def test_plan_kernel_names_match_the_profiles():
    class FakePd:
        NVFP4_GEMV_PATH_FAST = 1
        info = {1: (2, 4, 7, 0), 11: (2, 2, 4, 1), 20: (2, 4, 4, 2), 29: (4, 1, 1, 3),
                25: (16, 1, 2, 3)}

        def nvfp4_gemv_variant_info(self, v):
            return self.info[v]

    class P:
        def __init__(self, v, path=1):
            self.variant, self.path = v, path

    pd = FakePd()
    assert bench.plan_kernel_name(pd, P(1)) == "gemv_fast<2, 4, 7>"
    assert bench.plan_kernel_name(pd, P(11)) == "gemv_fastp<2, 2, 4>"
    assert bench.plan_kernel_name(pd, P(20)) == "gemv_fastg<2, 4, 4>"
    assert bench.plan_kernel_name(pd, P(29)) == "gemv_tile<1, 4>"
    assert bench.plan_kernel_name(pd, P(25)) == "gemv_tile<2, 16>"
    assert bench.plan_kernel_name(pd, P(0, path=2)) == "gemv_generic"


def test_replicas_are_capped():
    class FakeT:
        def clone(self):
            return self

    reps_list, reps = bench.replicate(None, {"A": FakeT()}, 18832, 0)
    assert reps == bench.MAX_REPLICAS and len(reps_list) == reps
    _, reps = bench.replicate(None, {"A": FakeT()}, 66_083_840, 0)
    assert reps == 16 and reps * 66_083_840 >= 1_000_000_000


def test_more_than_one_gpu_exits_with_a_message(capsys):
    assert bench.main(["--gpus", "2"]) == 2
    assert "one GPU" in capsys.readouterr().err


def test_world_size_above_one_exits(monkeypatch):
    monkeypatch.setenv("WORLD_SIZE", "4")
    assert bench.main([]) == 2


def test_roofline_fields():
    r = bench.roofline(6000.0, 123.0, probe_read_gbs=5000.123)
    assert r["bound"] == "hbm" and r["peak"] == bench.HBM_PEAK_GBS and r["unit"] == "GB/s"
    assert r["frac"] == round(6000.0 / bench.HBM_PEAK_GBS, 4) and r["traffic"] == 123.0
    assert r["probe_read_gbs"] == 5000.12


def test_recorded_traffic_needs_the_current_source(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    assert bench.recorded_traffic("decode") is None                     # no file
    h = bench.kernel_source_hash("gemv")
    assert len(h) == 16 and h != bench.kernel_source_hash("mma_stream")
    f = tmp_path / "gemv_decode_hbm_counters.txt"
    f.write_text(f"kernel_source_sha256_16: {h}\nhbm_bytes_per_launch: 66291018\n")
    assert bench.recorded_traffic("decode") == 66291018.0
    f.write_text("kernel_source_sha256_16: 0000000000000000\nhbm_bytes_per_launch: 1\n")
    assert bench.recorded_traffic("decode") is None                     # stale kernel source


def test_committed_profiles_name_their_source_hash():
    for name in os.listdir(bench.PROFILES):
        if name.endswith("_hbm_counters.txt"):
            text = open(os.path.join(bench.PROFILES, name)).read()
            assert "kernel_source_sha256_16:" in text and "hbm_bytes_per_launch:" in text, name


def test_single_launch_percentiles_skip_when_zero():
    assert bench.single_launch_percentiles(None, None, None, 0) is None


@pytest.mark.parametrize("n", [1, 7, 50])
def test_single_launch_percentiles_order(n, monkeypatch):
    """The percentile picking on a fake clock: p10 <= p50 <= p90, all from the samples."""

    class FakeEvent:
        t = 0.0

        def __init__(self, enable_timing=True):
            self.at = None

        def record(self, stream):
            FakeEvent.t += 0.001 * (1 + (FakeEvent.t * 7919) % 3)
            self.at = FakeEvent.t

        def synchronize(self):
            pass

        def elapsed_time(self, other):
            return other.at - self.at

    class FakeTensor:
        def fill_(self, v):
            return self

    class FakeCuda:
        Event = FakeEvent

    class FakeTorch:
        cuda = FakeCuda
        uint8 = "u8"

        @staticmethod
        def empty(*a, **k):
            return FakeTensor()

    r = bench.single_launch_percentiles(FakeTorch, None, lambda i: None, n)
    assert r["launches"] == n and r["p10"] <= r["p50"] <= r["p90"]


def test_cpu_baseline_speedup():
    assert bench.with_speedup(None, 5000.0) is None
    cpu = {"value": 0.5, "unit": "GB/s", "cores": 16, "kind": "oracle", "sample": "s"}
    r = bench.with_speedup(cpu, 5000.0)
    assert r["gpu_speedup"] == 10000.0 and r["value"] == 0.5 and "gpu_speedup" not in cpu


def test_parity_summary_counts_ulps():
    import numpy as np
    want = np.array([0x3C00, 0x0000, 0x8001, 0xBC00], dtype=np.uint16)   # 1, +0, -tiny, -1
    got = np.array([0x3C00, 0x8000, 0x0001, 0xBC02], dtype=np.uint16)    # 1, -0, +tiny, -1 - 2 ulp
    r = bench.parity_summary(np, got, want)
    assert r == {"outputs": 4, "bit_identical": 1, "max_ulp": 2}
    assert bench.parity_summary(np, want, want)["bit_identical"] == 4


def test_mma_kernel_name_follows_the_plan_form():
    class Plan:
        def __init__(self, path, variant):
            self.path, self.variant = path, variant

    class FakePd:
        NVFP4_GEMV_PATH_FAST = 1
        NVFP4_MMA_FORM_VALU_TILES = 1
        NVFP4_MMA_FORM_LDS_STAGED = 2
        NVFP4_MMA_FORM_LDS_VECTOR_REGS = 3

        @staticmethod
        def nvfp4_mma_variant_form(v):
            return {3: 0, 7: 1, 11: 2, 18: 3}[v]

    assert bench.mma_kernel_name(FakePd, Plan(1, 3), False) == "mma_stream"
    assert bench.mma_kernel_name(FakePd, Plan(1, 7), False) == "vec_tile"
    assert bench.mma_kernel_name(FakePd, Plan(1, 11), False) == "mma_lds"
    assert bench.mma_kernel_name(FakePd, Plan(1, 18), False) == "mma_lds"
    assert bench.mma_kernel_name(FakePd, Plan(2, 0), False) == "mma_generic"
    assert bench.mma_kernel_name(FakePd, Plan(1, 3), True) == "mma_stream_packed"
    for name in ("mma_stream", "vec_tile", "mma_lds", "mma_generic", "mma_stream_packed"):
        assert name in bench.KERNEL_SOURCES


def test_graph_launch_bounds_the_steps():
    with pytest.raises(SystemExit):
        bench.parse_args(["--steps", str(bench.MAX_GRAPH_STEPS + 1)])
    assert bench.parse_args(["--steps", str(bench.MAX_GRAPH_STEPS + 1), "--launch", "stream"]).steps \
        == bench.MAX_GRAPH_STEPS + 1
    with pytest.raises(SystemExit):
        bench.parse_args(["--steps", "0"])
