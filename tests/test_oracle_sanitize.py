"""The CPU oracle under AddressSanitizer and UndefinedBehaviorSanitizer.

``oracle/sanitize_check.c`` calls every oracle entry point on small seeded
inputs (ragged and empty rows, partial blocks, float32 and bf16, refused
working-set rows, loaded slot tables); this test builds it together with
``oracle.c`` under ``-fsanitize=address,undefined`` with gcc and runs it.
Any sanitizer report or failed check fails the test.
"""
import os
import shutil
import subprocess
import tempfile

import pytest

ORACLE = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc is needed to build the sanitizer run")
def test_oracle_runs_clean_under_address_and_ub_sanitizers():
    with tempfile.TemporaryDirectory() as tmp:
        exe = os.path.join(tmp, "oracle_sanitize")
        cmd = ["gcc", "-std=c99", "-O1", "-g", "-fopenmp", "-fsanitize=address,undefined",
               "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-Wall", "-Wextra", "-Werror",
               "-Wno-unused-parameter", os.path.join(ORACLE, "oracle.c"), os.path.join(ORACLE, "sanitize_check.c"),
               "-o", exe, "-lm"]
        subprocess.run(cmd, check=True, capture_output=True, text=True)
        env = dict(os.environ, OMP_NUM_THREADS="4", ASAN_OPTIONS="detect_leaks=1:abort_on_error=0")
        r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
        assert r.returncode == 0, r.stdout + r.stderr
        assert "oracle sanitizer run ok" in r.stdout
        assert "Sanitizer" not in r.stderr and "runtime error" not in r.stderr, r.stderr
