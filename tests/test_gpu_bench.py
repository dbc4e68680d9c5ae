"""bench.py end to end on the GPU, on the tiny workload: one JSON line with
the contract's fields, parity with the oracle, and every timing consistent."""
import json

import pytest
import torch

import bench

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu_ready():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")


@pytest.mark.parametrize("launch", ["stream", "graph"])
def test_bench_line_on_the_tiny_workload(capsys, launch):
    assert bench.main(["--config", "tiny", "--steps", "7", "--warmup", "2", "--single-launches",
                       "3", "--launch", launch]) == 0
    lines = [l for l in capsys.readouterr().out.splitlines() if l.startswith("{")]
    assert len(lines) == 1
    d = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
                "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
                "roofline", "cpu_baseline", "parity", "timing_us"):
        assert key in d, key
    assert d["metric"] == bench.METRIC and d["unit"] == "GB/s" and d["n_gpus"] == 1
    assert d["steps"] == 7 and d["warmup"] == 2 and d["vs_baseline"] is None
    assert d["config"]["workload"].startswith("tiny") and d["config"]["bytes_per_step"] == 18832
    r = d["roofline"]
    assert r["bound"] == "hbm" and r["peak"] == bench.HBM_PEAK_GBS and r["kernel"].startswith("gemv_")
    assert abs(r["frac"] - d["value"] / bench.HBM_PEAK_GBS) < 1e-3
    t = d["timing_us"]
    headline = t["graph_replay"] if launch == "graph" else t["stream_launches"]
    assert abs(headline - d["ms_per_step"] * 1e3) < 1e-2
    # value is rounded to 0.01 GB/s
    assert d["value"] == pytest.approx(18832 / (d["ms_per_step"] * 1e-3) / 1e9, rel=1e-3, abs=0.01)
    assert d["parity"] == {"outputs": 128, "bit_identical": 128, "max_ulp": 0}
    assert d["cpu_baseline"]["kind"] == "oracle" and d["cpu_baseline"]["cores"] >= 1


@pytest.mark.parametrize("path_args", [
    ["--path", "quantize", "--act-config", "decode_x"],
    ["--path", "gemv_bf16x", "--config", "tiny"],
    ["--path", "smalln", "--smalln-config", "tiny_n3"],
    ["--path", "grouped", "--moe-config", "moe_tiny"],
], ids=["quantize", "bf16x", "smalln", "grouped"])
@pytest.mark.parametrize("launch", ["stream", "graph"])
def test_path_lines_time_stream_launches_or_one_graph_replay(capsys, path_args, launch):
    assert bench.main(path_args + ["--steps", "5", "--warmup", "2", "--launch", launch,
                                   "--no-cpu-baseline"]) == 0
    lines = [l for l in capsys.readouterr().out.splitlines() if l.startswith("{")]
    assert len(lines) == 1
    d = json.loads(lines[0])
    t = d["timing_us"]
    assert (t["graph_replay"] is None) == (launch == "stream")
    headline = t["graph_replay"] if launch == "graph" else t["stream_launches"]
    assert abs(headline - d["ms_per_step"] * 1e3) < 1e-2
    assert d["config"]["launch"] == bench.launch_label(bench.parse_args(["--launch", launch]))
    assert d["value"] == pytest.approx(d["config"]["bytes_per_step"] / (d["ms_per_step"] * 1e-3) / 1e9,
                                       rel=1e-3, abs=0.01)
