"""The C++ oracle under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

oracle/qmoe_oracle.cpp is compiled with g++ together with a driver
(tests/oracle_sanitize_main.cpp) that calls every entry point on small
inputs of every codec and variant; any out-of-bounds access, leak, signed
overflow, misaligned or invalid conversion aborts the run.  Host code only:
nothing here touches a GPU.
"""
import os
import shutil
import subprocess
import tempfile

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not found")
def test_cpp_oracle_clean_under_asan_and_ubsan():
    with tempfile.TemporaryDirectory() as d:
        exe = os.path.join(d, "oracle_sanitized")
        cmd = ["g++", "-O1", "-g", "-std=c++17", "-Wall", "-Wextra", "-Werror", "-ffp-contract=off",
               "-fno-omit-frame-pointer", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
               os.path.join(ROOT, "oracle", "qmoe_oracle.cpp"), os.path.join(HERE, "oracle_sanitize_main.cpp"),
               "-o", exe]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr
        env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
                   UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
        r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
        assert r.returncode == 0, r.stdout + r.stderr
        assert "oracle sanitizer run ok" in r.stdout
