"""A plain C program drives libmha through include/libmha.h alone: device
memory from hipMalloc, the pages' 4-token worked example, no Python or
torch on the call path ("序列建模架构的演进与变革（二）" §4.3 for the example;
its exact output is pinned in tests/golden/worked_example_4token.json)."""
import os
import subprocess

import pytest

import transformer_head_scaled_fwd_amd as mha

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "c_abi", "worked_example.c")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build(out):
    lib_dir = os.path.dirname(mha.LIB_PATH)
    cmd = ["gcc", "-std=c11", "-Wall", "-Wextra", "-Werror", SRC,
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROCM, "include"),
           "-D__HIP_PLATFORM_AMD__", "-L", lib_dir, "-lmha", "-Wl,-rpath," + lib_dir,
           "-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-Wl,-rpath," + os.path.join(ROCM, "lib"),
           "-lm", "-o", out]
    return subprocess.run(cmd, capture_output=True, text=True)


def test_c_program_builds_against_header_and_library(tmp_path):
    mha.load()  # the library must exist
    res = build(str(tmp_path / "worked_example"))
    assert res.returncode == 0, res.stderr


@pytest.mark.gpu
def test_c_program_runs_the_worked_example(gpu, tmp_path):
    exe = str(tmp_path / "worked_example")
    res = build(exe)
    assert res.returncode == 0, res.stderr
    run = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    print(run.stdout, run.stderr, flush=True)
    assert run.returncode == 0, run.stdout + run.stderr
    assert "worked_example: ok" in run.stdout
