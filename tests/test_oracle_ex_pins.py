"""Pins of the extended oracle: grouped K/V heads, ALiBi, causal alignment,
log-sum-exp and weights.

As for the core pins, each test checks the oracle against something other
than itself: torch's float64 scaled_dot_product_attention (its own GQA head
mapping and its own bottom-right causal bias), scipy's logsumexp, numbers the
pages print, closed forms, and the 50-digit brute force.  CPU only.
"""
import math

import numpy as np
import pytest
import scipy.special
import torch
import torch.nn.functional as F
from torch.nn.attention.bias import causal_lower_right

import oracle
from oracle import brute
from conftest import load_golden


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _sdpa(q, k, v, mask=None, scale=None, enable_gqa=False):
    return F.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v),
        attn_mask=mask, scale=scale, enable_gqa=enable_gqa).numpy()


# --- grouped / multi-query heads --------------------------------------------------

@pytest.mark.parametrize("Hkv", [1, 2, 3, 6])
def test_gqa_matches_torch_head_mapping(Hkv):
    # torch's enable_gqa maps query head t to K/V head t // (H // Hkv).
    B, H, n, m, d = 2, 6, 5, 7, 8
    q, k, v = _rand((B, H, n, d), 1), _rand((B, Hkv, m, d), 2), _rand((B, Hkv, m, d), 3)
    sc = 0.3
    O = oracle.attention_ex(q, k, v, scale=sc)
    ref = _sdpa(q, k, v, scale=sc, enable_gqa=True)
    np.testing.assert_allclose(O, ref, rtol=0, atol=1e-12)


def test_gqa_with_equal_heads_is_the_core_operation():
    B, H, n, d = 2, 4, 9, 8
    q, k, v = _rand((B, H, n, d), 4), _rand((B, H, n, d), 5), _rand((B, H, n, d), 6)
    lens = np.array([9, 4], np.int32)
    O = oracle.attention_ex(q, k, v, key_lens=lens, causal=True, scale=0.4)
    ref = oracle.attention(q, k, v, key_lens=lens, causal=True, scale=0.4)
    np.testing.assert_array_equal(O, ref)


def test_gqa_rejects_indivisible_heads():
    q, k = _rand((1, 6, 3, 4), 0), _rand((1, 4, 3, 4), 1)
    with pytest.raises(ValueError):
        oracle.attention_ex(q, k, k)


# --- bottom-right causal alignment --------------------------------------------------

@pytest.mark.parametrize("n,L", [(1, 9), (3, 9), (4, 4), (5, 3), (2, 0)])
def test_bottom_right_matches_torch_lower_right_bias(n, L):
    # Per sequence: the first L cached keys, queries aligned to their end.
    B, H, m, d = 1, 2, 9, 4
    q, k, v = _rand((B, H, n, d), 7), _rand((B, H, m, d), 8), _rand((B, H, m, d), 9)
    lens = np.array([L], np.int32)
    O = oracle.attention_ex(q, k, v, key_lens=lens, causal="bottom_right", scale=0.5)
    for i in range(n):
        if i + L - n < 0:  # no visible key: the zero-row reading
            np.testing.assert_array_equal(O[0, :, i], 0.0)
    if L == 0:
        return
    ref = _sdpa(q, k[:, :, :L], v[:, :, :L], mask=causal_lower_right(n, L), scale=0.5)
    rows = [i for i in range(n) if i + L - n >= 0]
    np.testing.assert_allclose(O[0, :, rows], ref[0, :, rows], rtol=0, atol=1e-12)


def test_one_decode_query_sees_the_whole_prefix():
    # n = 1, bottom-right: the new token sees every filled key, which is the
    # plain padded (non-causal) attention over key_lens.
    B, H, m, d = 3, 2, 11, 4
    q, k, v = _rand((B, H, 1, d), 10), _rand((B, H, m, d), 11), _rand((B, H, m, d), 12)
    lens = np.array([11, 6, 1], np.int32)
    O = oracle.attention_ex(q, k, v, key_lens=lens, causal="bottom_right", scale=0.25)
    for b in range(B):
        L = lens[b]
        ref = _sdpa(q[b:b + 1], k[b:b + 1, :, :L], v[b:b + 1, :, :L], scale=0.25)
        np.testing.assert_allclose(O[b:b + 1], ref, rtol=0, atol=1e-12)


def test_square_full_length_alignments_agree():
    q, k, v = _rand((1, 2, 6, 4), 13), _rand((1, 2, 6, 4), 14), _rand((1, 2, 6, 4), 15)
    a = oracle.attention_ex(q, k, v, causal="top_left", scale=0.5)
    b = oracle.attention_ex(q, k, v, causal="bottom_right", scale=0.5)
    ref = F.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v), is_causal=True,
        scale=0.5).numpy()
    np.testing.assert_array_equal(a, b)
    np.testing.assert_allclose(a, ref, rtol=0, atol=1e-12)


# --- ALiBi ---------------------------------------------------------------------------

def _alibi_mask(n, m, L, slopes, mode):
    """Float mask: -slope * |p_i - j| where visible, -inf elsewhere."""
    H = len(slopes)
    out = np.full((H, n, m), -np.inf)
    for i in range(n):
        p = i + L - n if mode == "bottom_right" else i
        for j in range(m):
            vis = j < L and (mode is False or j <= p)
            if vis:
                out[:, i, j] = -np.asarray(slopes) * abs(p - j)
    return out


@pytest.mark.parametrize("mode", [False, "top_left", "bottom_right"])
def test_alibi_matches_sdpa_with_float_bias(mode):
    B, H, n, m, d = 2, 3, 6, 6, 4
    q, k, v = _rand((B, H, n, d), 16), _rand((B, H, m, d), 17), _rand((B, H, m, d), 18)
    lens = np.array([6, 4], np.int32)
    slopes = [0.5, 0.125, 1.0 / 64]
    O = oracle.attention_ex(q, k, v, key_lens=lens, causal=mode, alibi_slopes=slopes,
                            scale=0.5)
    for b in range(B):
        mask = torch.from_numpy(_alibi_mask(n, m, lens[b], slopes, mode))[None]
        ref = _sdpa(q[b:b + 1], k[b:b + 1], v[b:b + 1], mask=mask, scale=0.5)
        ok = np.isfinite(ref[0, 0, :, 0])
        np.testing.assert_allclose(O[b][:, ok], ref[0][:, ok], rtol=0, atol=1e-12)


@pytest.mark.parametrize("slope", [0.0, 0.3, 2.0])
def test_alibi_zero_query_closed_form(slope):
    # Q = 0 leaves only the bias: a_ij = r^|i-j| / sum_k r^|i-k| with
    # r = e^{-slope}.  With V = I the output row is that weight row.  The
    # sum is two geometric series: (1 - r^{i+1})/(1 - r) + r (1 - r^{m-1-i})/(1 - r).
    n = m = 7
    q = np.zeros((1, 1, n, m))
    k = _rand((1, 1, m, m), 19)
    v = np.eye(m)[None, None]
    O = oracle.attention_ex(q, k, v, alibi_slopes=[slope], scale=1.0)
    r = math.exp(-slope)
    for i in range(n):
        if slope == 0.0:
            z = m
        else:
            z = (1 - r ** (i + 1)) / (1 - r) + r * (1 - r ** (m - 1 - i)) / (1 - r)
        want = [r ** abs(i - j) / z for j in range(m)]
        np.testing.assert_allclose(O[0, 0, i], want, rtol=0, atol=1e-14)


def test_alibi_zero_slopes_is_the_core_operation():
    q, k, v = _rand((2, 2, 5, 4), 20), _rand((2, 2, 5, 4), 21), _rand((2, 2, 5, 4), 22)
    a = oracle.attention_ex(q, k, v, causal=True, alibi_slopes=[0.0, 0.0], scale=0.5)
    b = oracle.attention(q, k, v, causal=True, scale=0.5)
    np.testing.assert_array_equal(a, b)


# --- log-sum-exp and weights ---------------------------------------------------------

def test_lse_worked_example_printed_sum():
    # The page's hand-worked example prints the sum of the exponentiated
    # scaled scores (rounded intermediates); lse is its logarithm.
    g = load_golden("worked_example_4token.json")
    q = np.asarray(g["q"])[None, None, None]
    K = np.asarray(g["K"])[None, None]
    V = np.asarray(g["V"])[None, None]
    _, lse = oracle.attention_ex(q, K, V, scale=1 / math.sqrt(g["d_k"]), return_lse=True)
    assert abs(math.exp(lse[0, 0, 0]) - g["printed_exp_sum"]) < 0.02
    r2 = math.sqrt(2.0)
    assert abs(lse[0, 0, 0] - math.log(2 * math.exp(1 / r2) + 1 + math.exp(0.7 / r2))) < 1e-14


@pytest.mark.parametrize("mode", [False, "top_left", "bottom_right"])
def test_lse_matches_scipy_logsumexp(mode):
    B, H, Hkv, n, m, d = 2, 4, 2, 5, 8, 6
    q, k, v = _rand((B, H, n, d), 23), _rand((B, Hkv, m, d), 24), _rand((B, Hkv, m, d), 25)
    lens = np.array([8, 3], np.int32)
    slopes = [0.25, 0.0, 0.5, 0.125]
    sc = 0.4
    O, lse, S, A = oracle.attention_ex(q, k, v, key_lens=lens, causal=mode,
                                       alibi_slopes=slopes, scale=sc, return_lse=True,
                                       return_weights=True)
    for b in range(B):
        for t in range(H):
            raw = torch.from_numpy(q[b, t]) @ torch.from_numpy(k[b, t // 2]).T
            bias = _alibi_mask(n, m, lens[b], [slopes[t]], mode)[0]
            s = sc * raw.numpy() + bias
            want = scipy.special.logsumexp(s, axis=1)
            np.testing.assert_allclose(lse[b, t], want, rtol=0, atol=1e-12)
            w = torch.softmax(torch.from_numpy(s), dim=1).numpy()
            ok = np.isfinite(want)
            np.testing.assert_allclose(A[b, t][ok], w[ok], rtol=0, atol=1e-14)
            assert np.all(A[b, t][~ok] == 0)


def test_lse_of_row_without_keys_is_minus_inf():
    q, k = _rand((1, 1, 3, 4), 26), _rand((1, 1, 5, 4), 27)
    _, lse = oracle.attention_ex(q, k, k, key_lens=np.array([0], np.int32), return_lse=True)
    assert np.all(np.isneginf(lse))
    _, lse2 = oracle.attention_ex(q, k, k, key_lens=np.array([1], np.int32),
                                  causal="bottom_right", return_lse=True)
    # rows 0 and 1 sit before the first key; row 2 sees key 0 only
    assert np.isneginf(lse2[0, 0, 0]) and np.isneginf(lse2[0, 0, 1])
    assert np.isfinite(lse2[0, 0, 2])


# --- 50-digit brute force on tiny inputs ----------------------------------------------

@pytest.mark.parametrize("mode", [False, "top_left", "bottom_right"])
def test_extended_brute_force_tiny(mode):
    B, H, Hkv, n, m, d = 2, 2, 1, 3, 4, 3
    q, k, v = _rand((B, H, n, d), 28), _rand((B, Hkv, m, d), 29), _rand((B, Hkv, m, d), 30)
    slopes = [0.75, 0.0625]
    for L in range(m + 1):
        lens = np.array([L, m], np.int32)
        O, lse = oracle.attention_ex(q, k, v, key_lens=lens, causal=mode,
                                     alibi_slopes=slopes, scale=0.6, return_lse=True)
        for b in range(B):
            Lb = int(lens[b])
            for t in range(H):
                for i in range(n):
                    p = i + Lb - n if mode == "bottom_right" else i
                    valid = [j < Lb and (mode is False or j <= p) for j in range(m)]
                    bias = [-slopes[t] * abs(p - j) for j in range(m)]
                    w, o = brute.attention_row(q[b, t, i].tolist(), k[b, 0].tolist(),
                                               v[b, 0].tolist(), valid, 0.6, bias=bias)
                    np.testing.assert_allclose(O[b, t, i], [float(x) for x in o],
                                               rtol=0, atol=1e-13)
                    z = brute.row_logsumexp(q[b, t, i].tolist(), k[b, 0].tolist(), valid,
                                            0.6, bias=bias)
                    if z is None:
                        assert np.isneginf(lse[b, t, i])
                    else:
                        assert abs(lse[b, t, i] - z) < 1e-13


def test_rows_entry_point_matches_full_evaluation():
    B, H, Hkv, n, m, d = 2, 4, 1, 6, 9, 5
    q, k, v = _rand((B, H, n, d), 31), _rand((B, Hkv, m, d), 32), _rand((B, Hkv, m, d), 33)
    lens = np.array([9, 5], np.int32)
    slopes = [0.1, 0.2, 0.3, 0.4]
    O, lse = oracle.attention_ex(q, k, v, key_lens=lens, causal="bottom_right",
                                 alibi_slopes=slopes, scale=0.3, return_lse=True)
    rows = [(b, t, i) for b in range(B) for t in range(H) for i in range(n)]
    Or, lr = oracle.attention_ex_rows(q, k, v, rows, key_lens=lens, causal="bottom_right",
                                      alibi_slopes=slopes, scale=0.3)
    np.testing.assert_array_equal(Or, O.reshape(-1, d))
    np.testing.assert_array_equal(lr, lse.reshape(-1))
