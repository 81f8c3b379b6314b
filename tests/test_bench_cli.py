"""bench.py's argument checks, which run before anything touches a GPU."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run_bench(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT,
                          capture_output=True, text=True, timeout=120)


def test_more_than_one_gpu_is_refused():
    r = run_bench("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU only" in r.stderr


def test_sweep_rows_out_of_range_are_refused():
    for bad in ("0", "16,5000", "a,b", ","):
        r = run_bench("--config", "sweep", "--sweep-rows", bad)
        assert r.returncode == 2, bad
        assert "--sweep-rows" in r.stderr
