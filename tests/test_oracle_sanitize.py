"""The CPU oracle built with AddressSanitizer and UndefinedBehaviorSanitizer.

tests/helpers/oracle_sanitize_driver.c calls every oracle entry point on small
seeded inputs and on the edge cases (V = 1, K = 0, L = 0, T = 0, the residual
fallback, degenerate schedules).  Built with gcc and both sanitizers (host code
only, nothing here runs on a GPU), any out-of-bounds access, leak or undefined
operation aborts the driver.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_under_asan_and_ubsan(tmp_path):
    exe = tmp_path / "oracle_sanitize"
    cmd = ["gcc", "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer", "-ffp-contract=off",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           os.path.join(ROOT, "tests", "helpers", "oracle_sanitize_driver.c"),
           os.path.join(ROOT, "oracle", "dspark_oracle.c"), "-lm", "-o", str(exe)]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    env.pop("LD_PRELOAD", None)
    res = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=300)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "ok" in res.stdout
