"""bench.py's one-GPU contract, checked without a GPU: asked for several GPUs
it stops with a message and a non-zero status before touching a device."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_refuses_several_gpus():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
