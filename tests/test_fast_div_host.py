"""The launch-time divisors of the kernels' block-index decode (CPU only).

mha::fast_div (csrc/mha_host.h) gives a multiplier and a shift with which
the kernels divide by a launch constant: (n + mulhi(n, mul)) >> shift.  A
plain C++ driver (tests/c_abi/fast_div_check.cpp), built against the
host-only translation unit, compares that expression with n / d over every
divisor up to 4096, divisors around each power of two up to 2^31, random
divisors, and indices near 0, near 2^31 - 1, around multiples of d and at
random.
"""
import os
import subprocess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
INCLUDE = os.path.join(ROOT, "include")
CSRC = os.path.join(ROOT, "transformer_head_scaled_fwd_amd", "csrc")


def test_fast_div_matches_division(tmp_path):
    exe = tmp_path / "fast_div_check"
    subprocess.run(["g++", "-O2", "-std=c++17", "-Wall", "-Wextra", "-Werror", "-I", INCLUDE,
                    "-I", CSRC, os.path.join(ROOT, "tests", "c_abi", "fast_div_check.cpp"),
                    os.path.join(CSRC, "mha_host.cpp"), "-o", str(exe)], check=True)
    res = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300)
    assert res.returncode == 0, res.stdout + res.stderr
    assert ", 0 failed" in res.stdout, res.stdout
