"""The fp64 oracle built with the address and undefined-behaviour sanitizers (gcc), driven through
every one of its functions by oracle/sanitize_check.c: any out-of-bounds access, use after free,
leak or undefined operation ends the run with a report, and the driver's own invariant checks
(kept indices in range and ascending, s = S_trig + S_norm, constant heads, 0 <= R <= 1, ...) must
hold.  CPU only."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc is needed to build the oracle")
def test_oracle_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_sanitized")
    build = subprocess.run(
        ["gcc", "-O1", "-g", "-std=c99", "-fopenmp", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
         "-fno-omit-frame-pointer", os.path.join(ROOT, "oracle", "sanitize_check.c"),
         os.path.join(ROOT, "oracle", "tria_oracle.c"), "-lm", "-o", exe],
        capture_output=True, text=True)
    assert build.returncode == 0, build.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1", UBSAN_OPTIONS="print_stacktrace=1", OMP_NUM_THREADS="2")
    run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert run.returncode == 0, run.stdout + run.stderr
    assert "runtime error" not in run.stderr and "ERROR: AddressSanitizer" not in run.stderr, run.stderr
    assert "all checks passed" in run.stdout
