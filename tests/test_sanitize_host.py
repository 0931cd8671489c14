"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU:

* the C oracle (gcc, serial build) on a small case through
  tests/sanitize/oracle_sanitize_main.c;
* the C ABI's host layer (replayssm_api.hip compiled for the host only, the
  kernel launchers replaced by stubs that abort if reached) through
  tests/sanitize/abi_sanitize_main.c: size queries over many shapes, handle
  creation and destruction, and every rejection path.

Any out-of-bounds access, use of freed memory, leak or undefined arithmetic
aborts the run."""
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


def test_abi_host_layer_under_address_and_ub_sanitizers(tmp_path):
    hipcc, clang = "/opt/rocm/bin/hipcc", "/opt/rocm/llvm/bin/clang"
    if not (os.path.exists(hipcc) and os.path.exists(clang)):
        pytest.skip("ROCm compilers not available")
    inc = ["-I" + os.path.join(ROOT, "include"), "-I" + os.path.join(ROOT, "ssm_layer_decode_amd", "csrc")]
    host = ["-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-Xarch_host", "-fsanitize=address",
            "-Xarch_host", "-fsanitize=undefined", "-Xarch_host", "-fno-sanitize-recover=all",
            "--offload-host-only", *inc]
    objs = {"api": os.path.join(ROOT, "ssm_layer_decode_amd", "csrc", "replayssm_api.hip"),
            "probes": os.path.join(ROOT, "ssm_layer_decode_amd", "csrc", "probe_api.hip"),
            "stubs": os.path.join(ROOT, "tests", "sanitize", "launch_stubs.hip")}
    steps = [[hipcc, *host, "-c", src, "-o", str(tmp_path / f"{name}.o")] for name, src in objs.items()]
    steps.append([clang, "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                  "-fno-sanitize-recover=all", *inc, "-c",
                  os.path.join(ROOT, "tests", "sanitize", "abi_sanitize_main.c"), "-o", str(tmp_path / "main.o")])
    exe = str(tmp_path / "abi_san")
    steps.append([clang + "++", "-fsanitize=address,undefined", "-static-libsan", str(tmp_path / "main.o"),
                  str(tmp_path / "api.o"), str(tmp_path / "probes.o"), str(tmp_path / "stubs.o"),
                  "-L/opt/rocm/lib", "-lamdhip64",
                  "-Wl,-rpath,/opt/rocm/lib", "-o", exe])
    for cmd in steps:
        r = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
        if r.returncode != 0:
            pytest.skip(f"sanitizer build unavailable: {r.stderr.strip()[:200]}")
    run = subprocess.run([exe], capture_output=True, text=True, timeout=300,
                         env=dict(os.environ, ASAN_OPTIONS="detect_leaks=1"))
    assert run.returncode == 0, run.stdout[-2000:] + run.stderr[-2000:]
    assert "fails 0" in run.stdout
    assert "runtime error" not in run.stderr and "AddressSanitizer" not in run.stderr
