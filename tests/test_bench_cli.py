"""bench.py on more than one GPU: it refuses with a message and prints no
bench line (this path has no multi-GPU mode).  CPU only: the check happens
before anything touches a GPU."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert r.stdout.strip() == ""
    assert "one GPU" in r.stderr
