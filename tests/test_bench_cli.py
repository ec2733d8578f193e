"""bench.py's command line on the CPU: it measures one GPU only and says so
for more (before it touches torch or a GPU), and its defaults are the
headline run (the long-context workload, 20 timed steps after 5 warmup)."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("n", [2, 8])
def test_more_than_one_gpu_is_refused(n):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", str(n)], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and f"--gpus {n}" in r.stderr
    assert r.stdout == ""


def test_defaults(monkeypatch):
    sys.path.insert(0, ROOT)
    import bench
    monkeypatch.setattr(sys, "argv", ["bench.py"])
    a = bench.parse()
    assert (a.gpus, a.config, a.steps, a.warmup) == (1, 4, 20, 5)
