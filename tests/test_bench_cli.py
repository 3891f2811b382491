"""bench.py command line: the multi-GPU request is refused before any device work."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_refuses_more_than_one_gpu():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], cwd=ROOT,
                         stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True, timeout=300)
    assert res.returncode == 2
    assert "one GPU" in res.stderr and "--gpus 2" in res.stderr
    assert res.stdout == ""   # no JSON line is printed
