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
