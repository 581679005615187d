"""The C ABI's argument checks under AddressSanitizer and
UndefinedBehaviorSanitizer (host code only, no GPU).

tests/abi_sanitize_main.cpp compiles the ABI source as plain C++ with g++ and
stand-ins for the kernel launchers, then drives every entry point with null,
misaligned, negative, oversized and empty arguments and with valid ones: each
must return the documented status and reach the expected launcher (or none),
and no check may overflow, read out of bounds or leak."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir("/opt/rocm/include"),
                    reason="g++ or the HIP headers not available")
def test_abi_checks_under_sanitizers(tmp_path):
    exe = str(tmp_path / "abi_sanitize")
    cmd = ["g++", "-x", "c++", "-std=c++17", "-O1", "-g", "-Wall", "-Wextra", "-Werror",
           "-Wno-unused-parameter", "-Wno-unused-function", "-D__HIP_PLATFORM_AMD__",
           "-isystem", "/opt/rocm/include",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
           os.path.join(ROOT, "tests", "abi_sanitize_main.cpp"), "-o", exe]
    build = subprocess.run(cmd, capture_output=True, text=True)
    if build.returncode != 0 and "sanitize" in build.stderr and "cannot find" in build.stderr:
        pytest.skip("sanitizer runtime not installed")
    assert build.returncode == 0, build.stderr
    env = dict(os.environ, QBLK_LOG="1", ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert run.returncode == 0, run.stdout + run.stderr
    assert "clean" in run.stdout
    # the log line was written, and cut to its buffer
    lines = [ln for ln in run.stderr.splitlines() if ln.startswith("qblk: gemv x")]
    assert len(lines) == 1 and len(lines[0]) < 520
