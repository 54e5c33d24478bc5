"""50-digit evaluation of scaled dot-product attention for tiny inputs.

TEST INFRASTRUCTURE ONLY.  Pure-Python loops over mpmath numbers, meant for
n, m <= 8 and d <= 8.  It evaluates the textbook formula directly, with no
subtraction of the row maximum ("序列建模架构的演进与变革（二）" §4.3,
steps 2-5): scores q.k times scale, masked keys dropped (a masked score of
-inf contributes exp(-inf) = 0; "Transformer: 详解" §3.4 and §5.3), weights
exp(s)/sum exp(s), output sum of weight times value row.  A row without any
valid key returns zeros (the reading the oracle also adopts).
"""
from __future__ import annotations

import mpmath


def _exps(q, K, valid, scale, bias):
    sc = mpmath.mpf(scale)
    e = []
    for j in range(len(K)):
        if not valid[j]:
            e.append(mpmath.mpf(0))
            continue
        dot = mpmath.fsum(mpmath.mpf(a) * mpmath.mpf(b) for a, b in zip(q, K[j]))
        s = sc * dot + (mpmath.mpf(bias[j]) if bias is not None else 0)
        e.append(mpmath.exp(s))
    return e


def attention_row(q, K, V, valid, scale, dps=50, bias=None):
    """One query row.  q: list[d_k]; K: list[m][d_k]; V: list[m][d_v];
    valid: list[bool] of length m; bias: None or list[m] added to the scaled
    scores (ALiBi).  Returns (weights list[m], out list[d_v]) as mpmath
    numbers."""
    with mpmath.workdps(dps):
        m = len(K)
        dv = len(V[0]) if m else 0
        e = _exps(q, K, valid, scale, bias)
        z = mpmath.fsum(e)
        if z == 0:
            return [mpmath.mpf(0)] * m, [mpmath.mpf(0)] * dv
        w = [x / z for x in e]
        out = [mpmath.fsum(w[j] * mpmath.mpf(V[j][c]) for j in range(m))
               for c in range(dv)]
        return w, out


def row_logsumexp(q, K, valid, scale, dps=50, bias=None):
    """log(sum_j exp(s_j)) over the valid keys of one row, as a float, or
    None when no key is valid."""
    with mpmath.workdps(dps):
        z = mpmath.fsum(_exps(q, K, valid, scale, bias))
        return None if z == 0 else float(mpmath.log(z))


def attention(Q, K, V, key_lens=None, causal=False, scale=1.0, dps=50):
    """Nested lists Q[B][H][n][dk], K[B][H][m][dk], V[B][H][m][dv].
    Returns (O[B][H][n][dv], A[B][H][n][m]) as nested lists of floats."""
    O, A = [], []
    for b in range(len(Q)):
        L = len(K[b][0]) if key_lens is None else max(0, min(int(key_lens[b]), len(K[b][0])))
        Ob, Ab = [], []
        for t in range(len(Q[b])):
            m = len(K[b][t])
            Ot, At = [], []
            for i, q in enumerate(Q[b][t]):
                valid = [(j < L) and (not causal or j <= i) for j in range(m)]
                w, o = attention_row(q, K[b][t], V[b][t], valid, scale, dps)
                Ot.append([float(x) for x in o])
                At.append([float(x) for x in w])
            Ob.append(Ot)
            Ab.append(At)
        O.append(Ob)
        A.append(Ab)
    return O, A
