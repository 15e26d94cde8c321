"""The plain-C oracle under AddressSanitizer and UndefinedBehaviorSanitizer (host code
only, gcc): a small driver calls every oracle entry point, including the multi-word
CRT paths, and cross-checks a few results.  Any out-of-bounds access, overflow of a
signed type or misaligned access aborts the run."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_oracle_under_sanitizers(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no gcc")
    exe = tmp_path / "oracle_sanitize"
    cmd = [gcc, "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-pthread",
           os.path.join(ROOT, "tests", "native", "oracle_sanitize.c"), os.path.join(ROOT, "oracle", "ntt_oracle.c"),
           "-o", str(exe)]
    build = subprocess.run(cmd, capture_output=True, text=True)
    if build.returncode != 0 and "sanitize" in build.stderr:
        pytest.skip("sanitizer runtime not available: " + build.stderr[-300:])
    assert build.returncode == 0, build.stderr
    # verify_asan_link_order=0: the environment may preload other libraries first
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300, env=env)
    assert run.returncode == 0, run.stdout + run.stderr
    assert "oracle sanitized run ok" in run.stdout
