"""The fp64 oracle under AddressSanitizer and UndefinedBehaviorSanitizer.

The oracle produces every expected value the parity tests compare with; an
out-of-bounds read or undefined behaviour in it would change those values
without failing anything.  This test builds the oracle's C source together
with a small driver (oracle_sanitize_driver.c: every oracle function on eight
seeded problems, ragged and single-block shapes included) with both
sanitizers, on the host only, and requires a clean run.
"""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


def test_oracle_clean_under_sanitizers(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not found")
    exe = tmp_path / "oracle_sanitized"
    cmd = [gcc, "-O1", "-g", "-fopenmp", "-fsanitize=address,undefined", "-fno-omit-frame-pointer",
           "-fno-sanitize-recover=undefined", "-o", str(exe),
           os.path.join(HERE, "oracle_sanitize_driver.c"), os.path.join(ROOT, "oracle", "llsa_oracle.c"), "-lm"]
    build = subprocess.run(cmd, capture_output=True, text=True)
    if build.returncode != 0 and ("asan" in build.stderr or "ubsan" in build.stderr):
        pytest.skip("sanitizer runtime not available: " + build.stderr[-200:])
    assert build.returncode == 0, build.stderr
    env = dict(os.environ, OMP_NUM_THREADS="4", ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    run = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=300)
    out = run.stdout + run.stderr
    assert run.returncode == 0, out[-3000:]
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-3000:]
    assert run.stdout.strip().endswith("done"), out[-3000:]
    assert run.stdout.count("transpose out of range 0") == 8, run.stdout
