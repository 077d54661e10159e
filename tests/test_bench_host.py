"""Host-side parts of bench.py, on the CPU: the refusal of multi-GPU runs, the spread
statistics, and that the committed HBM-traffic record still matches the decode kernel's
sources (bench.py reports `roofline.traffic` only from a record taken on the current
kernel; a source change without a new record would turn it into null)."""
from __future__ import annotations

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


@pytest.mark.parametrize("n", [2, 8])
def test_more_than_one_gpu_is_refused(n):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", str(n)],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""          # no JSON line for an unmeasured run


def test_percentiles_interpolate_linearly():
    xs = [5.0, 1.0, 4.0, 2.0, 3.0]         # unsorted on purpose
    st = bench.stats(xs)
    assert st["mean"] == 3.0
    assert st["p50"] == 3.0
    assert st["p10"] == pytest.approx(1.4)  # 10 % of the way from 1 to 2 on the 4-step axis
    assert st["p90"] == pytest.approx(4.6)
    assert bench.stats([7.0]) == dict(mean=7.0, p10=7.0, p50=7.0, p90=7.0)


def test_traffic_record_matches_the_current_decode_kernel():
    traffic = bench.measured_traffic()
    assert traffic is not None, ("profiles/ traffic record was taken on other kernel sources; "
                                 "retake FETCH_SIZE / WRITE_SIZE for the current decode kernel")
    # one decode launch of the benchmark reads at least its K/V and writes its output
    assert 0.95 * 492263765 <= traffic <= 1.10 * 492263765


def test_cpu_baseline_names_the_host_cpu_model():
    name = bench.cpu_model()
    assert isinstance(name, str) and name.strip()
    try:
        models = [l.split(":", 1)[1].strip() for l in open("/proc/cpuinfo")
                  if l.startswith("model name")]
    except OSError:
        models = []
    if models:
        assert name == models[0]
