"""bench.py's command-line contract that needs no GPU: more than one GPU is refused with a
message and exit status 2, and the defaults are one GPU with a short run."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_defaults():
    a = bench.parse_args([])
    assert a.gpus == 1 and a.config == "C3" and 1 <= a.steps <= 100 and a.warmup >= 1
