"""The C oracle built with AddressSanitizer and UndefinedBehaviorSanitizer.

tests/oracle_sanitize_driver.c includes oracle/kvq_oracle.c and calls every
function it exports on small seeded inputs (a zero block, equal-magnitude
blocks, row lists, split-and-merge, the dense form, the INT2 codec).  Any
out-of-bounds access, leak or undefined operation in the oracle makes the
sanitized run fail.  Host code only: gcc, no GPU.
"""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not found")
def test_oracle_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_sanitized")
    cmd = ["gcc", "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer", "-fopenmp", "-ffp-contract=off",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-o", exe, os.path.join(HERE, "oracle_sanitize_driver.c"), "-lm"]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr
    env = dict(os.environ, OMP_NUM_THREADS="2",
               ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, f"rc={r.returncode}\n{r.stdout}\n{r.stderr[-4000:]}"
    assert "ok" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr
