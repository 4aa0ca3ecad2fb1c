"""Host-side checks of bench.py's contract that need no GPU: a request for
more than one GPU exits with a message instead of running."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stdout
    assert r.stdout.count("\n") <= 2   # a message, not a JSON result line
    assert '"metric"' not in r.stdout
