"""The host code under address and undefined-behaviour sanitizers (CPU only).

Two builds, neither of which involves a GPU:

* the host-only half of the library (include/libmha.h's argument checks,
  workspace sizes, plans and kernel names, csrc/mha_host.cpp) linked with a
  plain C driver (tests/c_abi/host_checks.c) that calls every host-side
  entry point, extreme sizes included, and checks each status;
* the oracle (oracle/mha_oracle.c) compiled with the same sanitizers, with
  the oracle's pin tests run against it in a child process that preloads
  the sanitizer runtimes.

Any overflow, out-of-bounds access or undefined conversion aborts the
program (-fno-sanitize-recover=all), so both tests fail on the first one.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
INCLUDE = os.path.join(ROOT, "include")
CSRC = os.path.join(ROOT, "transformer_head_scaled_fwd_amd", "csrc")
SAN = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
       "-fno-sanitize-recover=all"]


def _runtime(name):
    out = subprocess.run(["gcc", "-print-file-name=" + name], capture_output=True,
                         text=True).stdout.strip()
    return out if os.path.isabs(out) and os.path.exists(out) else None


def test_host_checks_under_asan_ubsan(tmp_path):
    drv = tmp_path / "host_checks.o"
    host = tmp_path / "mha_host.o"
    exe = tmp_path / "host_checks"
    subprocess.run(["gcc"] + SAN + ["-std=c11", "-Wall", "-Wextra", "-Werror", "-I", INCLUDE,
                                    "-c", os.path.join(ROOT, "tests", "c_abi", "host_checks.c"),
                                    "-o", str(drv)], check=True)
    subprocess.run(["g++"] + SAN + ["-std=c++17", "-Wall", "-Wextra", "-Werror", "-I", INCLUDE,
                                    "-I", CSRC, "-c", os.path.join(CSRC, "mha_host.cpp"),
                                    "-o", str(host)], check=True)
    subprocess.run(["g++"] + SAN + [str(drv), str(host), "-o", str(exe)], check=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    res = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=120)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "host checks:" in res.stdout and "failed" not in res.stdout
    assert "runtime error" not in res.stderr, res.stderr


def test_oracle_pins_under_asan_ubsan(tmp_path):
    if os.environ.get("LD_PRELOAD"):
        pytest.skip("another library is preloaded here; the sanitizer runtime must come first")
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if not asan or not ubsan:
        pytest.skip("gcc's sanitizer runtimes are not installed")
    import oracle
    lib = oracle.build_sanitized(str(tmp_path / "liboracle_san.so"))
    env = dict(os.environ, LD_PRELOAD=asan + " " + ubsan, MHA_ORACLE_LIB=lib,
               ASAN_OPTIONS="detect_leaks=0", UBSAN_OPTIONS="print_stacktrace=1",
               OMP_NUM_THREADS=os.environ.get("OMP_NUM_THREADS", "4"))
    pins = [os.path.join(ROOT, "tests", f) for f in
            ("test_oracle_pins.py", "test_oracle_ex_pins.py", "test_oracle_mha_pins.py")]
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                          "-m", "not gpu"] + pins,
                         capture_output=True, text=True, env=env, cwd=ROOT, timeout=600)
    tail = (res.stdout + res.stderr)[-3000:]
    assert res.returncode == 0, tail
    assert "passed" in res.stdout and "failed" not in res.stdout, tail
    assert "runtime error" not in res.stderr and "AddressSanitizer" not in res.stderr, tail
