"""Host-side checks of bench.py (no GPU): the one-GPU contract and the
workload table that the committed profiles refer to."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_profiled_workloads_are_bench_workloads():
    sys.path.insert(0, ROOT)
    import bench
    with open(os.path.join(ROOT, "profiles", "traffic.json")) as f:
        prof = json.load(f)
    assert set(prof["workloads"]) <= set(bench.WORKLOADS)
    assert "moe_mxfp8_srelu" in prof["workloads"]   # the headline workload carries traffic
