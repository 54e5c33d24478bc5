"""Build libmha.so (the HIP kernels and the C ABI) in-tree for gfx950.

    python -m transformer_head_scaled_fwd_amd.build

hipcc cross-compiles for gfx950 without a GPU present.  The packed-fp32
target feature is switched off for all device code.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libmha.so")

SOURCES = ["mha_abi.hip", "mha_fwd_kernel.hip", "mha_weights_kernel.hip",
           "mha_decode_kernel.hip", "mha_proj_kernel.hip"]
# Host-only C++ (argument checks, plans): built with g++, no HIP header.
HOST_SOURCES = ["mha_host.cpp"]
GXX_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra"]
OBJDIR = os.path.join(PKG, "_build")

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def compile_command(src: str, obj: str):
    return ([hipcc()] + [f for f in HIPCC_FLAGS if f != "-shared"]
            + ["-I", INCLUDE, "-I", CSRC, "-c", os.path.join(CSRC, src), "-o", obj])


def host_compile_command(src: str, obj: str, extra=()):
    return (["g++"] + GXX_FLAGS + list(extra)
            + ["-I", INCLUDE, "-I", CSRC, "-c", os.path.join(CSRC, src), "-o", obj])


def link_command(objs, out: str = LIB):
    return [hipcc(), "--offload-arch=gfx950", "-fPIC", "-shared"] + list(objs) + ["-o", out]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the gfx target feature; that warning
    # is expected, anything else is shown.
    noise = "is not a recognized feature for this target"
    msgs = [l for l in (res.stdout + res.stderr).splitlines() if noise not in l]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if msgs and verbose:
        print("\n".join(msgs), file=sys.stderr)


def build(verbose: bool = False) -> str:
    """Compile every HIP source (in parallel) and link libmha.so; returns its path."""
    os.makedirs(OBJDIR, exist_ok=True)
    tag = "%d" % os.getpid()
    objs = [os.path.join(OBJDIR, s.replace(".hip", ".%s.o" % tag)) for s in SOURCES]
    hobjs = [os.path.join(OBJDIR, s.replace(".cpp", ".%s.o" % tag)) for s in HOST_SOURCES]
    cmds = [compile_command(s, o) for s, o in zip(SOURCES, objs)]
    cmds += [host_compile_command(s, o) for s, o in zip(HOST_SOURCES, hobjs)]
    objs = objs + hobjs
    try:
        with ThreadPoolExecutor(max_workers=len(cmds)) as ex:
            list(ex.map(lambda c: _run(c, verbose), cmds))
        tmp = LIB + ".tmp" + tag
        _run(link_command(objs, tmp), verbose)
    finally:
        for o in objs:
            if os.path.exists(o):
                os.remove(o)
    check_stubs(tmp)
    os.replace(tmp, LIB)
    return LIB


def check_stubs(path: str) -> None:
    """Fail if a kernel's host launch stub is missing from the library.

    clang drops the stub of a kernel whose body is invalid for the host
    pass (for example a device-only builtin inside a lambda) without an
    error; the library would then fail to load at run time."""
    res = subprocess.run(["nm", "-u", path], capture_output=True, text=True)
    missing = [l.split()[-1] for l in res.stdout.splitlines() if "__device_stub__" in l]
    if missing:
        os.remove(path)
        raise RuntimeError("kernel launch stubs missing from the build: " + ", ".join(missing))


if __name__ == "__main__":
    print(build(verbose=True))
