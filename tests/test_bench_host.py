"""bench.py's host-side pieces (no GPU): the CPU baseline on a configuration
without double quantisation and on one with it, the multi-GPU refusal, and
the traffic lookup's key."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from synth import configs  # noqa: E402


@pytest.mark.parametrize("name", ["toy", "single"])
def test_cpu_baseline_runs_and_reports_its_host(name):
    cfg = configs.BY_NAME[name]
    n = sum(cfg.sizes)
    r = bench.cpu_baseline(cfg, 0.2, n, n)
    assert r["value"] > 0 and r["cores"] == 1 and r["kind"] == "oracle"
    assert r["cpu"]["compiler"].startswith("gcc") and r["cpu"]["cores_available"] >= 1
    assert os.sched_getaffinity(0) and len(os.sched_getaffinity(0)) == r["cpu"]["cores_available"]


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_traffic_is_read_only_for_matching_codec_sources():
    v = bench.read_traffic("14b", "nf4_dequantize")
    text = open(os.path.join(ROOT, "profiles", "traffic_14b.txt")).read()
    if f"codec_source_hash={bench.codec_source_hash()}" in text:
        assert v is not None and v > 3e10
    else:
        assert v is None
