"""Host-side pieces of bench.py, on the CPU: the refusal of several GPUs, the
step statistics, and the committed profiles it reads (present, taken on the
current kernel sources, ignored once those sources change)."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402
from all_gather_gemm_agmm_amd import inputs as I  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "--gpus must be 1" in r.stderr
    assert r.stdout == ""


def test_percentiles_and_step_stats():
    xs = [5.0, 1.0, 4.0, 2.0, 3.0]
    assert bench.percentile(xs, 0.0) == 1.0 and bench.percentile(xs, 1.0) == 5.0
    assert bench.percentile(xs, 0.5) == 3.0
    assert bench.percentile([1.0, 2.0], 0.5) == 1.5
    assert bench.percentile([], 0.5) is None
    st = bench.step_stats([float(i) for i in range(11)])
    assert st == {"median": 5.0, "p10": 1.0, "p90": 9.0}


@pytest.mark.parametrize("wid,variant", [(5, "fused"), (4, "staged"), (4, "fused"), (3, "skinny")])
def test_committed_profiles_match_the_kernel_sources(wid, variant):
    """The traffic and kernel-trace summaries the bench line cites exist for
    its workloads and were taken on the current kernel sources."""
    w = I.WORKLOADS[wid]
    traffic = bench.traffic_from_profiles(w.name, variant)
    assert traffic is not None and traffic > 0
    with open(os.path.join(ROOT, "profiles", f"kernel_trace_{w.name}_{variant}.json")) as f:
        trace = json.load(f)
    assert trace["kernel_sha"] == bench.kernel_source_sha()
    # algorithmic bytes of one launch (read A and B, write C) bound the
    # measured HBM traffic from below, up to the counter calibration
    e = I.DTYPE_BYTES[w.dtype]
    algorithmic = e * (w.m * w.k + w.k * w.n_local + w.m * w.n_local)
    if variant == "staged":   # per chunk launch: half of A and C, all of B
        algorithmic = e * (w.m * w.k // 2 + w.k * w.n_local + w.m * w.n_local // 2)
    assert traffic > 0.9 * algorithmic


def test_profiles_are_ignored_after_a_kernel_change(monkeypatch):
    w = I.WORKLOADS[5]
    monkeypatch.setattr(bench, "kernel_source_sha", lambda: "0000000000000000")
    assert bench.traffic_from_profiles(w.name, "fused") is None


def test_variant_resolution():
    assert bench.resolve_variant(I.WORKLOADS[3], "auto") == "skinny"
    assert bench.resolve_variant(I.WORKLOADS[5], "auto") == "fused"
    assert bench.resolve_variant(I.WORKLOADS[1], "auto") == "fused"
