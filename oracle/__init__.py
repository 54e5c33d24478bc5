"""CPU fp64 oracle for multi-head scaled dot-product attention.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
cpu_baseline leg are the only callers.  The library path never imports this
package, and this package imports nothing from the library path.

The arithmetic lives in ``mha_oracle.c`` (plain C, fp64, an explicit score
row per query, mask, max-subtracted softmax, weighted sum); this module only
widens inputs to float64, builds the shared object with gcc when it is
missing or stale, and marshals arguments through ctypes.  ``brute`` holds a
50-digit mpmath evaluation for tiny inputs.

Inputs may be numpy arrays or torch CPU tensors of any float dtype; widening
bf16 or fp32 to fp64 is exact, so the oracle sees the very bits a GPU run
receives.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mha_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

# gcc line for the oracle: plain -O2, no fast-math, no FP contraction.
GCC_CMD = ["gcc", "-O2", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared",
           "-std=c11", "-Wall", "-Wextra", _SRC, "-o", _LIB, "-lm"]

_lib = None


def build(force: bool = False) -> str:
    """Compile liboracle.so if it is missing, older than its source, or force."""
    stale = (not os.path.exists(_LIB)
             or os.path.getmtime(_LIB) < os.path.getmtime(_SRC))
    if force or stale:
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = GCC_CMD[:-3] + ["-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(_LIB)
        dp = ctypes.POINTER(ctypes.c_double)
        ip = ctypes.POINTER(ctypes.c_int32)
        lp = ctypes.POINTER(ctypes.c_int64)
        i64 = ctypes.c_int64
        lib.mha_oracle_f64.argtypes = [dp, dp, dp, ip, ctypes.c_int, ctypes.c_double,
                                       i64, i64, i64, i64, i64, i64, dp, dp, dp]
        lib.mha_oracle_f64.restype = ctypes.c_int
        lib.mha_oracle_rows_f64.argtypes = [dp, dp, dp, ip, ctypes.c_int, ctypes.c_double,
                                            i64, i64, i64, i64, i64, i64, lp, i64, dp]
        lib.mha_oracle_rows_f64.restype = ctypes.c_int
        lib.mha_oracle_threads.argtypes = []
        lib.mha_oracle_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def to_f64(x) -> np.ndarray:
    """Widen a numpy array or a torch CPU tensor to a contiguous float64 array."""
    if type(x).__module__.split(".")[0] == "torch":
        import torch
        x = x.detach().to("cpu", torch.float64).contiguous().numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a: np.ndarray, ctype):
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def _lens(key_lens, B):
    if key_lens is None:
        return None
    if type(key_lens).__module__.split(".")[0] == "torch":
        key_lens = key_lens.detach().cpu().numpy()
    kl = np.ascontiguousarray(np.asarray(key_lens, dtype=np.int32))
    if kl.shape != (B,):
        raise ValueError("key_lens must have shape (B,)")
    return kl


def _default_scale(dk: int) -> float:
    # The fp32 value a caller of the GPU library passes, widened to fp64.
    return float(np.float32(1.0 / np.sqrt(dk)))


def attention(q, k, v, key_lens=None, causal=False, scale=None,
              return_weights=False):
    """O = softmax(scale * Q K^T + mask) V for every (b, head, row).

    q [B,H,n,dk], k [B,H,m,dk], v [B,H,m,dv].  Returns O [B,H,n,dv] in fp64,
    and with return_weights also the masked scores S and weights A
    [B,H,n,m].
    """
    Q, K, V = to_f64(q), to_f64(k), to_f64(v)
    B, H, n, dk = Q.shape
    m, dv = K.shape[2], V.shape[3]
    if K.shape != (B, H, m, dk) or V.shape != (B, H, m, dv):
        raise ValueError("shape mismatch")
    kl = _lens(key_lens, B)
    sc = _default_scale(dk) if scale is None else float(scale)
    O = np.zeros((B, H, n, dv), np.float64)
    S = A = None
    if return_weights:
        S = np.zeros((B, H, n, m), np.float64)
        A = np.zeros((B, H, n, m), np.float64)
    lib = _load()
    rc = lib.mha_oracle_f64(_ptr(Q, ctypes.c_double), _ptr(K, ctypes.c_double),
                            _ptr(V, ctypes.c_double),
                            None if kl is None else _ptr(kl, ctypes.c_int32),
                            int(bool(causal)), sc, B, H, n, m, dk, dv,
                            _ptr(O, ctypes.c_double),
                            None if S is None else _ptr(S, ctypes.c_double),
                            None if A is None else _ptr(A, ctypes.c_double))
    if rc != 0:
        raise ValueError("oracle rejected the arguments")
    return (O, S, A) if return_weights else O


def attention_rows(q, k, v, rows, key_lens=None, causal=False, scale=None):
    """The same definition for selected rows only.

    rows: int array [R, 3] of (b, head, i).  Returns [R, dv] fp64.
    """
    Q, K, V = to_f64(q), to_f64(k), to_f64(v)
    B, H, n, dk = Q.shape
    m, dv = K.shape[2], V.shape[3]
    idx = np.ascontiguousarray(np.asarray(rows, dtype=np.int64).reshape(-1, 3))
    kl = _lens(key_lens, B)
    sc = _default_scale(dk) if scale is None else float(scale)
    out = np.zeros((idx.shape[0], dv), np.float64)
    lib = _load()
    rc = lib.mha_oracle_rows_f64(_ptr(Q, ctypes.c_double), _ptr(K, ctypes.c_double),
                                 _ptr(V, ctypes.c_double),
                                 None if kl is None else _ptr(kl, ctypes.c_int32),
                                 int(bool(causal)), sc, B, H, n, m, dk, dv,
                                 _ptr(idx, ctypes.c_int64), idx.shape[0],
                                 _ptr(out, ctypes.c_double))
    if rc != 0:
        raise ValueError("oracle rejected the arguments")
    return out


def threads() -> int:
    """OpenMP threads the oracle runs on in this process."""
    return int(_load().mha_oracle_threads())


def library_path() -> str:
    return _LIB


__all__ = ["attention", "attention_rows", "threads", "build", "to_f64",
           "library_path"]
