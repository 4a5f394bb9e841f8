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


def test_bench_flop_convention_matches_the_oracle_counting():
    """bench.py counts FLOPs with its own copy of the metric's convention (it
    may not call the oracle outside its CPU-baseline leg); both must agree."""
    import importlib.util
    import random

    import oracle
    spec = importlib.util.spec_from_file_location("bench_module", os.path.join(ROOT, "bench.py"))
    bench = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(bench)
    rng = random.Random(5)
    for _ in range(200):
        pairs, hq, d = rng.randint(0, 10 ** 13), rng.choice([1, 8, 16, 32, 128]), rng.choice([64, 128])
        assert bench.forward_flops(pairs, hq, d) == oracle.forward_flops(pairs, hq, d)
        for per_pair in (8, 10):
            assert bench.backward_flops(pairs, hq, d, per_pair) == oracle.backward_flops(pairs, hq, d, per_pair)
