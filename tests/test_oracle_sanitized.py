"""The CPU reference under AddressSanitizer and UndefinedBehaviorSanitizer.

oracle/oracle.c is compiled together with tests/oracle_sanitize_driver.c,
which calls every entry point on small inputs that take the skip, padding,
empty-range and empty-document paths.  Any out-of-bounds access, leak or
undefined behaviour aborts the run.
"""
from __future__ import annotations

import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc is not available")
def test_oracle_under_sanitizers(tmp_path):
    exe = tmp_path / "oracle_sanitized"
    cmd = ["gcc", "-std=c11", "-O1", "-g", "-fopenmp", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
           os.path.join(ROOT, "oracle", "oracle.c"), os.path.join(HERE, "oracle_sanitize_driver.c"),
           "-o", str(exe), "-lm"]
    build = subprocess.run(cmd, capture_output=True, text=True)
    if build.returncode != 0 and "asan" in build.stderr.lower():  # pragma: no cover
        pytest.skip("the sanitizer runtime is not installed: " + build.stderr[-300:])
    assert build.returncode == 0, build.stderr
    env = dict(os.environ, OMP_NUM_THREADS="4",
               ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    run = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=120)
    assert run.returncode == 0, run.stdout + run.stderr
    assert "oracle sanitized run ok" in run.stdout
