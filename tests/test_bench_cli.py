"""bench.py command-line contract (CPU): it parses, and a multi-GPU request is
refused with a message and exit status 2 before any device work."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_refuses_several_gpus():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2, r.stderr
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in msg["error"]


def test_bench_kernel_work_accounting():
    sys.path.insert(0, ROOT)
    import bench
    work = bench.kernel_work()
    # every accounted kernel has a positive byte, multiply-add or product count
    for name, w in work.items():
        assert w.get("bytes", 0) > 0 or w.get("mads", 0) > 0 or w.get("products", 0) > 0, name
    # the measured-traffic table names only accounted kernels
    assert set(bench.MEASURED_TRAFFIC["bytes_per_launch"]) <= set(work)
