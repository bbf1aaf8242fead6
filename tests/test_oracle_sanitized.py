"""The oracle under AddressSanitizer and UndefinedBehaviorSanitizer: gcc
builds oracle/oracle.c with tests/oracle_sanitize_driver.c (host code
only), and the driver runs every entry point on small ragged cases (a
contraction and a causal reduce, dense against relational; uniform and
interval repartitions; attention, causal and over packed segments).  Any
out-of-bounds access, use of freed memory, leak or undefined behaviour in
the checker stops the run with a report."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_oracle_under_sanitizers(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no gcc")
    exe = str(tmp_path / "oracle_sanitize_driver")
    build = [gcc, "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
             "-fno-sanitize-recover=all", "-fopenmp", "-std=c11",
             os.path.join(ROOT, "oracle", "oracle.c"), os.path.join(ROOT, "tests", "oracle_sanitize_driver.c"),
             "-o", exe, "-lm"]
    r = subprocess.run(build, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1", UBSAN_OPTIONS="print_stacktrace=1", OMP_NUM_THREADS="2")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "0 failures" in r.stdout, r.stdout
