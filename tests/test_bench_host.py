"""bench.py's host-side contract, on the CPU: it refuses runs on more than one
GPU with exit status 2, and its traffic lookup returns nothing for a workload
no committed counter summary covers."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], cwd=ROOT,
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and "--gpus 2" in r.stderr


def test_traffic_lookup_needs_a_matching_summary():
    sys.path.insert(0, ROOT)
    import bench
    assert bench.profiled_traffic("no_such_workload") is None
    # the hash ignores comments and blank lines, and is stable across calls
    assert bench.kernel_source_hash() == bench.kernel_source_hash()
    assert len(bench.kernel_source_hash(bench.BWD_KERNEL_SOURCES)) == 64
