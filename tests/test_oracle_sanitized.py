"""The CPU oracle under AddressSanitizer and UndefinedBehaviorSanitizer: a
standalone C driver (oracle/sanitize_check.c) is compiled with gcc together
with oracle/moe_oracle.c, -fsanitize=address,undefined and no recovery, and
run.  It calls every oracle function on small seeded inputs and degenerate
shapes and checks properties the definitions fix; any invalid memory access
or undefined operation aborts the run."""
from __future__ import annotations

import os
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_under_asan_and_ubsan():
    with tempfile.TemporaryDirectory() as tmp:
        exe = os.path.join(tmp, "oracle_sanitized")
        cmd = ["gcc", "-std=c11", "-O1", "-g", "-fopenmp", "-fno-omit-frame-pointer",
               "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-Wall", "-Wextra",
               "-o", exe, os.path.join(ROOT, "oracle", "moe_oracle.c"),
               os.path.join(ROOT, "oracle", "sanitize_check.c"), "-lm"]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr
        env = dict(os.environ, OMP_NUM_THREADS="4",
                   ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:halt_on_error=1",
                   UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
        r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
        assert r.returncode == 0, r.stdout + r.stderr
        assert "every check passed" in r.stdout
