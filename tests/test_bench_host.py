"""Host-only parts of bench.py: the per-device work balance it reports,
pinned by closed forms of the causal pair counts (no GPU needed)."""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import bench  # noqa: E402
import ring_inputs  # noqa: E402


def test_contiguous_ring_imbalance_closed_form():
    # device r of n holds rows [r c, (r+1) c): it sees r c^2 + c (c+1) / 2 pairs per head;
    # the last device over the mean is (n - 1 + (c+1)/(2c)) / ((n-1)/2 + (c+1)/(2c))
    wl = ring_inputs.WORKLOADS["contig1m_64dev"]
    n, c = wl.world, wl.local_len
    last = (n - 1) * c * c + c * (c + 1) // 2
    mean = sum(r * c * c + c * (c + 1) // 2 for r in range(n)) / n
    first = c * (c + 1) // 2
    lb = bench.load_balance(wl)
    assert lb["partition"] == "contiguous"
    assert lb["pairs_max"] == last and lb["pairs_min"] == first
    assert lb["max_over_mean"] == pytest.approx(last / mean, abs=1e-4)
    assert lb["max_over_mean"] == pytest.approx(1.9844, abs=1e-4)


@pytest.mark.parametrize("name", ["zigzag1m_64dev", "zigzag128k_8dev_gqa"])
def test_zigzag_ring_is_exactly_balanced(name):
    # every device sees L (L + 1) / 2 / n pairs per head: the zigzag split balances the causal triangle
    wl = ring_inputs.WORKLOADS[name]
    L = wl.total_len
    lb = bench.load_balance(wl)
    assert lb["pairs_max"] == lb["pairs_min"] == L * (L + 1) // 2 // wl.world
    assert lb["max_over_mean"] == 1.0 and lb["min_over_mean"] == 1.0


def test_cpu_baseline_reports_host_and_extrapolation():
    wl = ring_inputs.WORKLOADS["zigzag8k_8dev_d128"]
    rec = bench.cpu_baseline(wl, 0, share_flops=1.0e12, budget_s=0.2)
    assert rec["kind"] == "oracle" and rec["unit"] == "TFLOP/s" and rec["value"] > 0
    assert rec["os_cpu_count"] == os.cpu_count() and rec["cores"] >= 1
    assert "cpu_model" in rec and rec["blas_threads"] is not None
    assert rec["full_share_s_extrapolated"] == pytest.approx(1.0 / rec["value"], rel=1e-2)


def test_bench_line_keeps_the_contract():
    """The JSON line the benchmark prints: the contract's keys and types, the
    workload named in config (no model keys), the roofline and the CPU
    baseline objects (built here from fixed numbers, no GPU)."""
    import argparse
    import json
    import numpy as np
    wl = ring_inputs.WORKLOADS["zigzag128k_8dev_gqa"]
    args = argparse.Namespace(receive="auto", key_split_effective=1)
    roof_traffic = 763735326
    cpu = {"value": 0.05, "unit": "TFLOP/s", "cores": 16, "kind": "oracle", "sample": "rows x heads"}
    rec = bench.record(args, wl, 0, 20, 3, 1250.0, 14.07, True, 17.59e12, list(range(8)), 1.73, np.full(8, 1.73),
                       1272.75, bench.PEAK_BF16_TFLOPS, roof_traffic, None, None, None, None, bench.load_balance(wl),
                       cpu)
    line = json.loads(json.dumps(rec))
    for key, typ in (("metric", str), ("value", float), ("unit", str), ("n_gpus", int), ("steps", int),
                     ("warmup", int), ("ms_per_step", float), ("higher_is_better", bool), ("scaling", str),
                     ("dtype", str), ("data", str), ("config", dict)):
        assert isinstance(line[key], typ), key
    assert line["n_gpus"] == 1 and line["steps"] == 20 and line["warmup"] == 3
    assert line["higher_is_better"] is True and line["scaling"] == "weak" and line["vs_baseline"] is None
    assert line["dtype"] == "bf16" and line["unit"] == "TFLOP/s"
    assert line["config"]["workload"] == "zigzag128k_8dev_gqa" and "model" not in line["config"]
    roof = line["roofline"]
    assert roof["bound"] == "mfma" and roof["unit"] == "TFLOP/s" and roof["peak"] == 2500.0
    assert roof["frac"] == pytest.approx(1272.75 / 2500.0, abs=1e-4) and roof["traffic"] == roof_traffic
    assert line["cpu_baseline"]["kind"] == "oracle" and line["cpu_baseline"]["cores"] == 16


def test_bench_refuses_more_than_one_gpu():
    import json
    import subprocess
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in msg["error"]
