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

# Sanitizer build of the same source (address and undefined-behaviour
# checks), for running the pins under the sanitizers on the host.
SAN_FLAGS = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
             "-fno-sanitize-recover=all"]

_lib = None


def build_sanitized(out: str) -> str:
    """Compile the oracle with SAN_FLAGS into `out` (a shared object that
    needs the sanitizer runtimes preloaded into the process that loads it)."""
    cmd = [c for c in GCC_CMD[:-3] if c != "-O2"] + SAN_FLAGS + ["-o", out, "-lm"]
    subprocess.run(cmd, check=True)
    return out


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
        # MHA_ORACLE_LIB names another build of this source (the sanitizer
        # build); otherwise the default build, compiled when stale.
        path = os.environ.get("MHA_ORACLE_LIB") or build()
        lib = ctypes.CDLL(path)
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
        lib.mha_oracle_ex_f64.argtypes = [dp, dp, dp, ip, ctypes.c_int, dp, ctypes.c_double,
                                          i64, i64, i64, i64, i64, i64, i64, dp, dp, dp, dp]
        lib.mha_oracle_ex_f64.restype = ctypes.c_int
        lib.mha_oracle_ex_rows_f64.argtypes = [dp, dp, dp, ip, ctypes.c_int, dp,
                                               ctypes.c_double, i64, i64, i64, i64, i64, i64,
                                               i64, lp, i64, dp, dp]
        lib.mha_oracle_ex_rows_f64.restype = ctypes.c_int
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


_MODES = {False: 0, None: 0, "none": 0, True: 1, "top_left": 1, "bottom_right": 2}


def _mode(causal) -> int:
    if causal not in _MODES:
        raise ValueError("causal must be False, True, 'top_left' or 'bottom_right'")
    return _MODES[causal]


def _slopes(alibi_slopes, H):
    if alibi_slopes is None:
        return None
    sl = to_f64(alibi_slopes).reshape(-1)
    if sl.shape != (H,):
        raise ValueError("alibi_slopes must have H entries")
    return np.ascontiguousarray(sl)


def _ex_shapes(Q, K, V):
    B, H, n, dk = Q.shape
    Bk, Hkv, m, dk2 = K.shape
    dv = V.shape[3]
    if (Bk, dk2) != (B, dk) or V.shape != (B, Hkv, m, dv):
        raise ValueError("shape mismatch")
    return B, H, Hkv, n, m, dk, dv


def attention_ex(q, k, v, key_lens=None, causal=False, alibi_slopes=None,
                 scale=None, return_lse=False, return_weights=False):
    """The extended definition: grouped K/V heads, ALiBi, causal alignment.

    q [B,H,n,dk]; k [B,Hkv,m,dk] and v [B,Hkv,m,dv] with H % Hkv == 0 (query
    head t reads K/V head t // (H // Hkv)).  causal: False, True or
    'top_left' (key j visible when j <= i), or 'bottom_right' (when
    j <= i + L_b - n).  alibi_slopes: H values or None; the scaled score of
    (i, j) gets -slope * |p_i - j|, p_i = i (+ L_b - n for bottom_right).
    Returns O [B,H,n,dv] in fp64, then LSE [B,H,n] (natural log, -inf for a
    row with no valid key) if return_lse, then S and A [B,H,n,m] if
    return_weights.
    """
    Q, K, V = to_f64(q), to_f64(k), to_f64(v)
    B, H, Hkv, n, m, dk, dv = _ex_shapes(Q, K, V)
    kl = _lens(key_lens, B)
    sl = _slopes(alibi_slopes, H)
    sc = _default_scale(dk) if scale is None else float(scale)
    O = np.zeros((B, H, n, dv), np.float64)
    LSE = np.zeros((B, H, n), np.float64) if return_lse else None
    S = A = None
    if return_weights:
        S = np.zeros((B, H, n, m), np.float64)
        A = np.zeros((B, H, n, m), np.float64)
    d = ctypes.c_double
    rc = _load().mha_oracle_ex_f64(
        _ptr(Q, d), _ptr(K, d), _ptr(V, d),
        None if kl is None else _ptr(kl, ctypes.c_int32), _mode(causal),
        None if sl is None else _ptr(sl, d), sc, B, H, Hkv, n, m, dk, dv, _ptr(O, d),
        None if LSE is None else _ptr(LSE, d), None if S is None else _ptr(S, d),
        None if A is None else _ptr(A, d))
    if rc != 0:
        raise ValueError("oracle rejected the arguments")
    out = (O,)
    if return_lse:
        out += (LSE,)
    if return_weights:
        out += (S, A)
    return out if len(out) > 1 else O


def attention_ex_rows(q, k, v, rows, key_lens=None, causal=False,
                      alibi_slopes=None, scale=None):
    """attention_ex for selected rows: rows int [R, 3] of (b, head, i).
    Returns (O_rows [R, dv], LSE_rows [R]) in fp64."""
    Q, K, V = to_f64(q), to_f64(k), to_f64(v)
    B, H, Hkv, n, m, dk, dv = _ex_shapes(Q, K, V)
    idx = np.ascontiguousarray(np.asarray(rows, dtype=np.int64).reshape(-1, 3))
    kl = _lens(key_lens, B)
    sl = _slopes(alibi_slopes, H)
    sc = _default_scale(dk) if scale is None else float(scale)
    out = np.zeros((idx.shape[0], dv), np.float64)
    lse = np.zeros((idx.shape[0],), np.float64)
    d = ctypes.c_double
    rc = _load().mha_oracle_ex_rows_f64(
        _ptr(Q, d), _ptr(K, d), _ptr(V, d),
        None if kl is None else _ptr(kl, ctypes.c_int32), _mode(causal),
        None if sl is None else _ptr(sl, d), sc, B, H, Hkv, n, m, dk, dv,
        _ptr(idx, ctypes.c_int64), idx.shape[0], _ptr(out, d), _ptr(lse, d))
    if rc != 0:
        raise ValueError("oracle rejected the arguments")
    return out, lse


def multihead(xq, xk, xv, Wq, bq, Wk, bk, Wv, bv, Wo, bo, H, key_lens=None,
              causal=False, scale=None, return_weights=False):
    """The multi-head formula ("Transformer: 详解" §4.2, "第2章：完整的
    Transformer 架构" §2.2; the projections carry a bias as the
    nn.Linear layers of "序列建模架构的演进与变革（二）" §4.9 do):

      head_t = Attention(xq W_t^Q + b_t^Q, xk W_t^K + b_t^K, xv W_t^V + b_t^V)
      Y      = Concat(head_1, ..., head_H) W^O + b^O

    The weights come in nn.Linear's [out, in] layout, [d_model, d_model];
    head t's projection W_t^Q is the transpose of rows t d_k .. (t+1) d_k of
    Wq (and likewise for K and V), and the product of the concatenation with
    W^O is the sum over heads of head_t times the transpose of columns
    t d_k .. (t+1) d_k of Wo.  b* are [d_model] or None; d_k = d_model / H.
    All fp64 with library matmuls, no rounding of intermediates.  Returns Y
    [B, n, d_model], and with return_weights also A [B, H, n, m].
    """
    Xq, Xk, Xv = to_f64(xq), to_f64(xk), to_f64(xv)
    B, n, dm = Xq.shape
    m = Xk.shape[1]
    if dm % H:
        raise ValueError("d_model must be a multiple of H")
    dk = dm // H
    W = {name: to_f64(w) for name, w in (("q", Wq), ("k", Wk), ("v", Wv), ("o", Wo))}
    bias = {name: (None if b is None else to_f64(b))
            for name, b in (("q", bq), ("k", bk), ("v", bv), ("o", bo))}

    def head_projection(x, name, t):
        """x W_t + b_t for head t: [B, L, d_model] -> [B, L, d_k]."""
        rows = slice(t * dk, (t + 1) * dk)
        y = np.matmul(x, W[name][rows].T)
        return y if bias[name] is None else y + bias[name][rows]

    Q = np.stack([head_projection(Xq, "q", t) for t in range(H)], axis=1)  # [B, H, n, dk]
    K = np.stack([head_projection(Xk, "k", t) for t in range(H)], axis=1)
    V = np.stack([head_projection(Xv, "v", t) for t in range(H)], axis=1)
    res = attention_ex(Q, K, V, key_lens=key_lens, causal=causal, scale=scale,
                       return_weights=return_weights)
    O = res[0] if return_weights else res
    Y = np.zeros((B, n, dm)) if bias["o"] is None else np.broadcast_to(bias["o"], (B, n, dm)).copy()
    for t in range(H):
        Y += np.matmul(O[:, t], W["o"][:, t * dk:(t + 1) * dk].T)
    return (Y, res[2]) if return_weights else Y


def threads() -> int:
    """OpenMP threads the oracle runs on in this process."""
    return int(_load().mha_oracle_threads())


def library_path() -> str:
    return os.environ.get("MHA_ORACLE_LIB") or _LIB


__all__ = ["attention", "attention_rows", "attention_ex", "attention_ex_rows", "multihead",
           "threads", "build", "to_f64", "library_path"]
