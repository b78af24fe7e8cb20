"""Host AddressSanitizer / UndefinedBehaviorSanitizer run of the C oracle:
tests/sanitize/oracle_driver.c calls every oracle entry point on edge
values, built together with oracle/pqo.c under -fsanitize=address,undefined
with no recovery, so any out-of-bounds access or undefined operation fails
this test.  CPU only."""
from __future__ import annotations

import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_asan")
    cmd = ["gcc", "-O1", "-g", "-std=c11", "-fno-fast-math", "-ffp-contract=off", "-fopenmp",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
           os.path.join(ROOT, "oracle", "pqo.c"), os.path.join(HERE, "sanitize", "oracle_driver.c"),
           "-o", exe, "-lm"]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    env = dict(os.environ, OMP_NUM_THREADS="4",
               ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "oracle driver done, inexact 0" in r.stdout
    assert "runtime error" not in r.stderr and "ERROR: AddressSanitizer" not in r.stderr
