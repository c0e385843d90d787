"""Host-side checks of bench.py that need no GPU."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(HERE, "..", "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)

