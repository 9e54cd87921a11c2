"""bench.py's one-line JSON contract, on a short run of the diamond-1000 workload."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_prints_one_json_line_with_the_contract_fields():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--workload", "3",
                        "--steps", "3", "--warmup", "1", "--no-cpu-baseline"],
                       capture_output=True, text=True, timeout=110)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.strip()]
    assert len(lines) == 1
    d = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
                "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
                "roofline", "cpu_baseline"):
        assert key in d, key
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 1
    assert d["unit"] == "atoms/s" and d["higher_is_better"] is True
    assert d["dtype"] == "f64" and d["data"] == "synthetic"
    assert d["config"]["workload"] == "diamond-1000" and d["config"]["n_atoms"] == 1000
    assert d["cpu_baseline"] is None  # --no-cpu-baseline
    # value is the whole step's throughput: atoms over the wall time per step
    assert d["value"] == pytest.approx(1000 / (d["ms_per_step"] * 1e-3), rel=1e-9)
    rf = d["roofline"]
    assert rf["bound"] == "mfma" and rf["unit"] == "TFLOP/s" and rf["peak"] == 78.6
    assert rf["frac"] == pytest.approx(rf["achieved"] / rf["peak"], rel=1e-9)
    assert 0.0 < rf["frac"] < 1.0


def test_bench_fp32_line_prices_the_fp32_matrix_cores():
    """On an fp32 workload the dominant kernel is the fp32 matrix-core kernel, priced against
    the fp32 MFMA peak; the timing block carries the median and trimmed mean of every call, and
    the opt-in split-pair leg is reported apart with its difference from the fp32 output."""
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--workload", "4",
                        "--steps", "4", "--warmup", "1", "--no-cpu-baseline", "--split16"],
                       capture_output=True, text=True, timeout=110)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.strip()]
    assert len(lines) == 1
    d = json.loads(lines[0])
    assert d["dtype"] == "f32" and d["config"]["workload"] == "fe-bcc-65536"
    assert d["config"]["attn_kernel"] == "fused_f32"
    rf = d["roofline"]
    assert rf["kernel"] == "fused_f32" and rf["peak"] == 157.3 and rf["unit"] == "TFLOP/s"
    assert 0.0 < rf["frac"] < 1.0
    t = d["timing"]
    for k in ("step_ms", "nl_build_ms", "edge_csr_ms", "block_attn_forward_ms"):
        for stat in ("mean", "median", "trimmed_mean_10"):
            assert t[k][stat] > 0.0, (k, stat)
    gs = d["gather_scatter"]
    assert gs["block_shape"] == [65536, 181, 64]
    for k in ("gather", "scatter"):
        assert gs[k]["achieved_gbs"] > 0.0 and 0.0 < gs[k]["frac"] < 1.0
    s16 = d["split16"]
    assert s16["kernel"] == "fused_f32_split16"
    assert 0.0 < s16["normwise_diff_vs_fp32_output"] < 2e-5
