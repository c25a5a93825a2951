"""The fp64 oracle built with AddressSanitizer and UndefinedBehaviorSanitizer
(gcc, CPU only) and driven through every entry point on small inputs and edge
cases (tests/oracle_sanitize_main.c): no out-of-bounds access, leak or undefined
operation anywhere in the checker."""
import os
import shutil
import subprocess

import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(os.path.dirname(oracle.__file__), "saga_oracle.c")
MAIN = os.path.join(HERE, "oracle_sanitize_main.c")


def test_oracle_under_address_and_ub_sanitizers(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    exe = tmp_path / "oracle_asan"
    cmd = ["gcc", "-std=c99", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fopenmp",
           SRC, MAIN, "-o", str(exe), "-lm"]
    subprocess.run(cmd, check=True)
    env = dict(os.environ, OMP_NUM_THREADS="2",
               ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "oracle sanitizer run ok" in r.stdout
