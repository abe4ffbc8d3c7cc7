"""bench.py's host-side pieces (no GPU): the CPU baseline on a configuration
without double quantisation and on one with it, the multi-GPU refusal, and
the traffic and VALU-count lookups."""
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


def test_alu_roofline_from_matching_counters():
    """The VALU roofline entry uses the committed SQ_INSTS_VALU summary only
    when it was taken on the current codec sources; its peak is 256 CUs x 4
    SIMDs x 2.4 GHz / 4 cycles per wave64 instruction."""
    assert bench.VALU_PEAK_GIPS == pytest.approx(614.4)
    r = bench.alu_roofline("14b", "nf4_layer_error", 12687769600, 7.0)
    text = open(os.path.join(ROOT, "profiles", "counters_14b.txt")).read()
    if f"codec_source_hash={bench.codec_source_hash()}" in text:
        vpw = r["valu_per_weight"]
        assert 5 < vpw < 40
        assert r["achieved"] == pytest.approx(vpw * 12687769600 / 64 / 7e-3 / 1e9, rel=1e-3)
        assert r["frac"] == pytest.approx(r["achieved"] / 614.4, rel=1e-3)
    else:
        assert r is None
