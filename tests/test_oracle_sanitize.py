"""The C oracle built with AddressSanitizer and UndefinedBehaviorSanitizer
(gcc, host code) and driven on small and degenerate shapes by
tests/oracle_sanitize.c: no out-of-bounds access, no undefined behaviour, and
the program's own value checks hold."""
import os
import shutil
import subprocess
import tempfile

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_under_address_and_ub_sanitizers():
    with tempfile.TemporaryDirectory() as tmp:
        exe = os.path.join(tmp, "oracle_sanitize")
        build = subprocess.run(
            ["gcc", "-O1", "-g", "-std=c11", "-fno-omit-frame-pointer",
             "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
             os.path.join(HERE, "oracle_sanitize.c"), os.path.join(ROOT, "oracle", "aaren_oracle.c"),
             "-o", exe, "-lm"],
            capture_output=True, text=True)
        assert build.returncode == 0, build.stderr
        env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
                   UBSAN_OPTIONS="print_stacktrace=1")
        run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
        assert run.returncode == 0, run.stdout + run.stderr
        assert "ERROR: AddressSanitizer" not in run.stderr
        assert "runtime error" not in run.stderr
        assert "all calls and checks passed" in run.stdout
