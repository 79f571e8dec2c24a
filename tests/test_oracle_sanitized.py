"""The C++ oracle under AddressSanitizer and UndefinedBehaviorSanitizer.

tests/sanitize/oracle_driver.cpp calls every exported oracle routine on
small seeded inputs of each storage type and on the edge cases (empty
sequence, context inside the window, dense fallback, k >= C, exact ties,
shuffled table, a block-completing append, the threaded step). It is built
with g++ for the host only, so any out-of-bounds access, use of freed
memory, signed overflow or other undefined behaviour aborts the run."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_oracle_is_clean_under_asan_and_ubsan(tmp_path):
    exe = tmp_path / "oracle_driver"
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fopenmp",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           os.path.join(ROOT, "oracle", "kvsp_oracle.cpp"),
           os.path.join(ROOT, "tests", "sanitize", "oracle_driver.cpp"), "-o", str(exe)]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1", OMP_NUM_THREADS="3")
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "driver ok" in r.stdout
