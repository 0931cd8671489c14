"""The C oracle built with AddressSanitizer and UndefinedBehaviorSanitizer
(gcc, host code only, serial build) and run on a small case through
tests/sanitize/oracle_sanitize_main.c: any out-of-bounds access, use of freed
memory, leak or undefined arithmetic aborts the run."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_c_oracle_under_address_and_ub_sanitizers(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    exe = str(tmp_path / "oracle_san")
    build = subprocess.run(
        ["gcc", "-O1", "-g", "-std=c99", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
         "-fno-sanitize-recover=all", "-static-libasan", "-o", exe,
         os.path.join(ROOT, "tests", "sanitize", "oracle_sanitize_main.c"),
         os.path.join(ROOT, "oracle", "cpu", "oracle_cpu.c"), "-lm"],
        capture_output=True, text=True, timeout=300)
    if build.returncode != 0:
        pytest.skip(f"sanitizer build unavailable: {build.stderr.strip()[:200]}")
    run = subprocess.run([exe], capture_output=True, text=True, timeout=300,
                         env=dict(os.environ, ASAN_OPTIONS="detect_leaks=1"))
    assert run.returncode == 0, run.stderr[-2000:]
    assert "rc 0" in run.stdout
    assert "runtime error" not in run.stderr and "AddressSanitizer" not in run.stderr
