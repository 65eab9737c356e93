"""The oracle's C code under AddressSanitizer and UndefinedBehaviorSanitizer
(host build with gcc): every entry point on small inputs that reach its
edge cases (out-of-range page ids, empty rows, ties, appends at negative
positions and past the page table) runs without a report."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_sanitized")
    src = os.path.join(HERE, "sanitize", "oracle_sanitized_main.c")
    build = subprocess.run(["gcc", "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer",
                            "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                            "-o", exe, src, "-lm"], capture_output=True, text=True)
    assert build.returncode == 0, build.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert run.returncode == 0, run.stdout + run.stderr
    assert "oracle sanitized run: ok" in run.stdout
