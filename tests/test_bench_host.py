"""Host-side checks of bench.py's contract (no GPU): the one-GPU limit and the
rule that a recorded HBM-traffic figure is reported only for the kernel
sources it was measured on."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, env=dict(os.environ, WORLD_SIZE="1"))
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""  # no JSON line for a run that did not happen


@pytest.mark.parametrize("workload", ["b8_8k", "fp8_ragged", "b4_64k"])
def test_recorded_traffic_follows_the_kernel_sources(workload, monkeypatch):
    path = os.path.join(ROOT, "profiles", "prefix_kernel_%s_traffic.txt" % workload)
    fields = dict(line.split(":", 1) for line in open(path) if ":" in line and not line.startswith("#"))
    recorded = float(fields["hbm_bytes_per_launch"])
    assert recorded > 0
    if fields["kernel_sources_sha256"].strip() == bench.kernel_source_hash():
        assert bench.recorded_traffic(workload) == recorded
    # any other kernel source: no figure
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "0" * 64)
    assert bench.recorded_traffic(workload) is None


def test_no_traffic_for_a_workload_without_counters():
    assert bench.recorded_traffic("decode_b512") is None
