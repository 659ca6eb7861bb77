"""The host code under AddressSanitizer and UndefinedBehaviorSanitizer:
tests/sanitize_driver.cpp, built with gcc/g++ together with the oracle's C
(oracle/ltref.c) and the library's host packer (lt_pack.cpp), runs round
trips, table builds, generated streams and damaged blocks; any
out-of-bounds access or undefined behaviour fails the run."""
import os
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]


@pytest.mark.skipif(shutil.which("g++") is None or shutil.which("gcc") is None, reason="needs gcc and g++")
def test_host_code_under_sanitizers():
    with tempfile.TemporaryDirectory() as d:
        oracle_o = os.path.join(d, "ltref.o")
        exe = os.path.join(d, "sanitize_driver")
        subprocess.run(["gcc", "-std=c11", *SAN, "-c", os.path.join(ROOT, "oracle", "ltref.c"), "-o", oracle_o],
                       check=True, capture_output=True, text=True)
        subprocess.run(["g++", "-std=c++17", *SAN, "-pthread", "-I" + os.path.join(ROOT, "include"),
                        os.path.join(ROOT, "tests", "sanitize_driver.cpp"),
                        os.path.join(ROOT, "weight_dequantization_amd", "csrc", "lt_pack.cpp"), oracle_o,
                        "-o", exe], check=True, capture_output=True, text=True)
        env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
                   UBSAN_OPTIONS="print_stacktrace=1")
        env.pop("LD_PRELOAD", None)
        r = subprocess.run([exe], capture_output=True, text=True, timeout=600, env=env)
        assert r.returncode == 0 and r.stdout.strip() == "ok", (r.stdout[-2000:], r.stderr[-4000:])
