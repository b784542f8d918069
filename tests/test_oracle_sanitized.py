"""The oracle under AddressSanitizer and UndefinedBehaviorSanitizer (CPU).

oracle/sanitize_check.c drives every exported oracle function over its edge
cases (empty rows, fewer finite scores than k, equal scores, pools with missing
blocks, attention without keys, a wrapping replay ring); built here together
with oracle/csa2_oracle.c with gcc's -fsanitize=address,undefined, any
out-of-bounds access, leak or undefined operation aborts the run."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_oracle_under_sanitizers(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    exe = str(tmp_path / "oracle_sanitized")
    cmd = [gcc, "-std=c11", "-O1", "-g", "-ffp-contract=off", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
           os.path.join(ROOT, "oracle", "csa2_oracle.c"), os.path.join(ROOT, "oracle", "sanitize_check.c"),
           "-lm", "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0 and "asan" in (r.stderr or "").lower():
        pytest.skip("sanitizer runtime not available: " + r.stderr[-300:])
    assert r.returncode == 0, r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    env.pop("LD_PRELOAD", None)
    run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert run.returncode == 0, run.stdout + run.stderr
    assert "all checks passed" in run.stdout
