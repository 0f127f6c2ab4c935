"""bench.py's command line on the host: the parts that run before any GPU work."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run_bench(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=120, cwd=ROOT)


def test_more_than_one_gpu_is_refused():
    r = run_bench("--gpus", "2", "--steps", "1", "--warmup", "0")
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""  # no JSON line


def test_zero_gpus_is_refused():
    r = run_bench("--gpus", "0")
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
