"""bench.py's command-line contract, checked without a GPU: one GPU only
(--gpus above 1 exits with a message saying so), and at least two scan
launches (the first is not timed)."""
import os
import subprocess
import sys

from conftest import ROOT

BENCH = os.path.join(ROOT, "bench.py")


def _run(*args):
    return subprocess.run([sys.executable, BENCH, *args], capture_output=True, text=True, timeout=120)


def test_more_than_one_gpu_is_refused():
    r = _run("--gpus", "2")
    assert r.returncode != 0
    assert "one GPU only" in r.stderr


def test_a_single_scan_launch_is_refused():
    r = _run("--scan-reps", "1")
    assert r.returncode != 0
    assert "--scan-reps must be at least 2" in r.stderr
