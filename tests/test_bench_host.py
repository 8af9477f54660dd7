"""bench.py's host-side contract (no GPU): more than one GPU is refused with
a message before anything touches a device, and the helpers that build the
record behave as stated."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr and r.stdout == ""


def test_traffic_table_is_keyed_by_kernel_source_hashes():
    h = bench.kernel_source_hash()
    assert len(h) == 64 and all(ch in "0123456789abcdef" for ch in h)
    assert all(os.path.isfile(os.path.join(ROOT, f)) for f in bench.KERNEL_SOURCES)
    for k, v in bench.TRAFFIC_BY_SOURCE.items():
        assert len(k) == 64 and all(ch in "0123456789abcdef" for ch in k)
        assert isinstance(v, int) and v > 0


def test_cpu_model_is_a_string_or_none():
    m = bench.cpu_model()
    assert m is None or (isinstance(m, str) and m)
