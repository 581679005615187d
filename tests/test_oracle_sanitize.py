"""The C oracle under AddressSanitizer and UndefinedBehaviorSanitizer (host
code only): oracle/sanitize_main.c drives every entry point on small seeded
inputs at exact buffer sizes; any out-of-bounds access, leak, or undefined
operation (signed overflow, bad shift, misaligned access) fails the build's
run."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ORACLE = os.path.join(ROOT, "oracle")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_sanitize")
    cmd = ["gcc", "-std=c11", "-O1", "-g", "-ffp-contract=off", "-fno-fast-math",
           "-fexcess-precision=standard", "-fno-strict-aliasing", "-Wall", "-Wextra", "-Werror",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
           os.path.join(ORACLE, "sanitize_main.c"), os.path.join(ORACLE, "qblk_oracle.c"),
           "-I", ORACLE, "-o", exe, "-lm"]
    build = subprocess.run(cmd, capture_output=True, text=True)
    if build.returncode != 0 and "sanitize" in build.stderr and "cannot find" in build.stderr:
        pytest.skip("sanitizer runtime not installed")
    assert build.returncode == 0, build.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert run.returncode == 0, run.stdout + run.stderr
    assert "clean" in run.stdout
