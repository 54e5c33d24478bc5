"""Pins of the CPU fp64 oracle to facts the pages and the mathematics fix.

Each test checks the oracle against something other than itself: numbers the
pages print for a worked example, closed forms, stated invariants, a library
special case, or a 50-digit brute force on tiny inputs.  They run on the CPU.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import brute
from conftest import load_golden
from transformer_head_scaled_fwd_amd import inputs


def _single(q, K, V, scale, causal=False, key_lens=None):
    """Wrap one head's matrices as [1,1,n,d] and call the oracle."""
    q = np.asarray(q, np.float64)
    if q.ndim == 1:
        q = q[None, :]
    K = np.asarray(K, np.float64)
    V = np.asarray(V, np.float64)
    O, S, A = oracle.attention(q[None, None], K[None, None], V[None, None],
                               key_lens=key_lens, causal=causal, scale=scale,
                               return_weights=True)
    return O[0, 0], S[0, 0], A[0, 0]


# --- P-1: the hand-worked 4-token example --------------------------------------

def test_worked_example_4token_printed_values():
    g = load_golden("worked_example_4token.json")
    scale = 1.0 / math.sqrt(g["d_k"])
    O, S, A = _single(g["q"], g["K"], g["V"], scale)
    tol = g["printed_tolerance"]
    np.testing.assert_allclose(S[0] / scale, g["printed_raw_scores"], atol=1e-15)
    np.testing.assert_allclose(S[0], g["printed_scaled_scores"], atol=tol)
    np.testing.assert_allclose(A[0], g["printed_weights"], atol=tol)
    np.testing.assert_allclose(O[0], g["printed_output"], atol=tol)


def test_worked_example_4token_closed_form():
    # With a = e^{1/sqrt2}, c = e^{0.7/sqrt2}: weights (a, 1, c, a) / (2a+1+c);
    # O = (2a + c, a + 3 + 2c) / (2a + 1 + c).
    g = load_golden("worked_example_4token.json")
    r2 = math.sqrt(2.0)
    a, c = math.exp(1.0 / r2), math.exp(0.7 / r2)
    Z = 2 * a + 1 + c
    O, _, A = _single(g["q"], g["K"], g["V"], 1.0 / r2)
    np.testing.assert_allclose(A[0], [a / Z, 1 / Z, c / Z, a / Z], rtol=0, atol=1e-14)
    np.testing.assert_allclose(O[0], [(2 * a + c) / Z, (a + 3 + 2 * c) / Z],
                               rtol=0, atol=1e-14)
    # the values quoted with six decimals in the design notes
    np.testing.assert_allclose(O[0], [0.850672, 1.240767], atol=5e-7)


# --- P-2: the 3x3 causal softmax ----------------------------------------------

def test_causal_3x3_example():
    g = load_golden("causal_softmax_3x3.json")
    Sg = np.array(g["scaled_scores"])
    I3 = np.eye(3)
    # Q = the printed scores, K = I, scale 1  =>  S = Q;  V = I  =>  O = A.
    O, S, A = _single(Sg, I3, I3, 1.0, causal=True)
    assert np.isneginf(S[0, 1]) and np.isneginf(S[0, 2]) and np.isneginf(S[1, 2])
    np.testing.assert_array_equal(O, A)
    printed = np.array(g["printed_softmax"])
    for r in g["rows_that_follow_from_the_printed_scores"]:
        np.testing.assert_allclose(A[r], printed[r], atol=g["printed_tolerance"])
    e = np.exp(Sg[2])
    np.testing.assert_allclose(A[2], e / e.sum(), atol=1e-15)
    np.testing.assert_allclose(A[2], [0.2399, 0.2522, 0.5079], atol=1e-4)
    # the misprinted row really is off by more than its printed precision
    assert np.abs(A[2] - printed[2]).max() > 0.02


# --- P-9: saturation ------------------------------------------------------------

def test_saturation_example():
    g = load_golden("saturation_8_minus3.json")
    s = g["scores"]
    # one query [1], keys [8] and [-3], scale 1 -> scores [8, -3]; V = I.
    O, S, A = _single([[1.0]], [[s[0]], [s[1]]], np.eye(2), 1.0)
    np.testing.assert_allclose(np.exp(S[0]), g["printed_exp"], rtol=0.01)
    np.testing.assert_allclose(A[0], g["printed_softmax"], atol=g["printed_tolerance"])
    t = math.exp(-11.0)
    np.testing.assert_allclose(A[0], [1.0 / (1.0 + t), t / (1.0 + t)], rtol=1e-13, atol=0)
    np.testing.assert_allclose(A[0], [0.9999833, 1.67e-5], rtol=1e-3)


def test_large_scores_stay_finite():
    # Scores of 1000 overflow fp64 exp() unless the row maximum is
    # subtracted first; the real-valued weights are 1, e^-500 and e^-2000
    # (the last below the fp64 range, so 0).
    q = [[1000.0]]
    K = [[1.0], [0.5], [-1.0]]
    O, S, A = _single(q, K, np.eye(3), 1.0)
    assert np.all(np.isfinite(A))
    np.testing.assert_allclose(A[0], [1.0, math.exp(-500.0), 0.0], rtol=1e-14, atol=0)


# --- P-3: weights sum to one, masked weights are exactly zero -------------------

@pytest.mark.parametrize("causal", [False, True])
def test_rows_sum_to_one_and_masked_are_zero(causal):
    B, H, n, d = 3, 2, 37, 16
    q, k, v, kl = inputs.draw(B, H, n, n, d, d, "f32", seed=11, lens=(0, n))
    kl[0] = 0           # one sequence with no valid key at all
    kl[1] = n
    O, S, A = oracle.attention(q, k, v, key_lens=kl, causal=causal,
                               return_weights=True)
    for b in range(B):
        L = int(kl[b])
        for i in range(n):
            valid = np.array([(j < L) and (not causal or j <= i) for j in range(n)])
            row = A[b, :, i, :]
            assert np.all(row[:, ~valid] == 0.0)
            assert np.all(np.isneginf(S[b, :, i, ~valid]))
            if valid.any():
                np.testing.assert_allclose(row.sum(-1), 1.0, atol=1e-14, rtol=0)
                assert np.all(row[:, valid] > 0.0)
            else:
                assert np.all(row == 0.0) and np.all(O[b, :, i] == 0.0)


# --- P-4: permutation equivariance / invariance ---------------------------------

def test_self_attention_permutation_equivariant():
    B, H, n, d = 2, 3, 29, 8
    q, k, v, _ = inputs.draw(B, H, n, n, d, d, "f32", seed=21)
    P = np.random.Generator(np.random.PCG64(5)).permutation(n)
    O = oracle.attention(q, k, v)
    Op = oracle.attention(q[:, :, P], k[:, :, P], v[:, :, P])
    np.testing.assert_allclose(Op, O[:, :, P], atol=1e-12, rtol=0)


def test_permuting_keys_and_values_jointly_leaves_output_unchanged():
    B, H, n, m, d = 2, 2, 7, 41, 8
    q, k, v, _ = inputs.draw(B, H, n, m, d, d, "f32", seed=22)
    P = np.random.Generator(np.random.PCG64(6)).permutation(m)
    O = oracle.attention(q, k, v)
    Op = oracle.attention(q, k[:, :, P], v[:, :, P])
    np.testing.assert_allclose(Op, O, atol=1e-12, rtol=0)
    # permuting keys alone (without values) does change it
    Ok = oracle.attention(q, k[:, :, P], v)
    assert np.abs(Ok - O).max() > 1e-3


# --- P-5: causal row 0 returns v_0 ----------------------------------------------

def test_causal_row0_is_v0():
    B, H, n, d = 2, 4, 33, 64
    q, k, v, _ = inputs.draw(B, H, n, n, d, d, "bf16", seed=23)
    O = oracle.attention(q, k, v, causal=True)
    np.testing.assert_array_equal(O[:, :, 0, :], oracle.to_f64(v)[:, :, 0, :])


# --- P-6: Q = 0 gives the mean of the valid value rows --------------------------

@pytest.mark.parametrize("causal", [False, True])
def test_zero_query_gives_mean_of_valid_values(causal):
    B, H, n, d = 3, 2, 45, 16
    _, k, v, kl = inputs.draw(B, H, n, n, d, d, "f32", seed=24, lens=(1, n))
    q = np.zeros((B, H, n, d))
    O = oracle.attention(q, k, v, key_lens=kl, causal=causal)
    V = oracle.to_f64(v)
    for b in range(B):
        for i in range(n):
            cnt = min(i + 1, int(kl[b])) if causal else int(kl[b])
            np.testing.assert_allclose(O[b, :, i], V[b, :, :cnt].mean(axis=1),
                                       atol=1e-13, rtol=0)


# --- P-7: 50-digit brute force on tiny inputs -----------------------------------

@pytest.mark.parametrize("causal", [False, True])
def test_brute_force_tiny(causal):
    rng = np.random.Generator(np.random.PCG64(77))
    for trial in range(4):
        n = int(rng.integers(1, 7))
        m = n if causal else int(rng.integers(1, 7))
        dk, dv = int(rng.integers(1, 5)), int(rng.integers(1, 5))
        scale = float(rng.uniform(0.2, 2.0))
        q = rng.standard_normal((1, 1, n, dk))
        k = rng.standard_normal((1, 1, m, dk))
        v = rng.standard_normal((1, 1, m, dv))
        for L in range(0, m + 1):
            kl = np.array([L], np.int32)
            O, _, A = oracle.attention(q, k, v, key_lens=kl, causal=causal,
                                       scale=scale, return_weights=True)
            Ob, Ab = brute.attention(q.tolist(), k.tolist(), v.tolist(),
                                     key_lens=[L], causal=causal, scale=scale)
            np.testing.assert_allclose(O, np.array(Ob), atol=1e-13, rtol=0)
            np.testing.assert_allclose(A, np.array(Ab), atol=1e-13, rtol=0)


# --- P-8: a library special case: torch SDPA in float64 -------------------------

@pytest.mark.parametrize("causal,n,m", [(False, 19, 19), (True, 23, 23), (False, 11, 30)])
def test_matches_torch_sdpa_float64(causal, n, m):
    B, H, d = 3, 2, 16
    q, k, v, kl = inputs.draw(B, H, n, m, d, d, "bf16", seed=25, lens=(1, m))
    scale = float(np.float32(1 / np.sqrt(d)))
    O = oracle.attention(q, k, v, key_lens=kl, causal=causal, scale=scale)
    j = torch.arange(m)
    i = torch.arange(n)
    keep = (j[None, None, :] < torch.as_tensor(kl)[:, None, None])
    if causal:
        keep = keep & (j[None, :] <= i[:, None])[None]
    keep = keep[:, None]                                     # [B,1,n,m]
    ref = torch.nn.functional.scaled_dot_product_attention(
        q.double(), k.double(), v.double(), attn_mask=keep, scale=scale)
    has_valid = keep.any(-1, keepdim=True).expand(B, H, n, 1)[..., 0].numpy()
    np.testing.assert_allclose(O[has_valid], ref.numpy()[has_valid], atol=1e-12, rtol=0)


# --- P-10: padding has no effect on any query -----------------------------------

@pytest.mark.parametrize("causal", [False, True])
def test_padding_content_has_no_effect(causal):
    B, H, n, d = 3, 2, 40, 16
    q, k, v, kl = inputs.draw(B, H, n, n, d, d, "bf16", seed=26, lens=(1, n))
    O = oracle.attention(q, k, v, key_lens=kl, causal=causal)
    k2, v2 = k.clone(), v.clone()
    g = torch.Generator().manual_seed(3)
    for b in range(B):
        L = int(kl[b])
        shape = k2[b, :, L:].shape
        k2[b, :, L:] = (torch.randint(0, 2, shape, generator=g) * 2 - 1).to(k2.dtype) * 1e4
        v2[b, :, L:] = (torch.randint(0, 2, shape, generator=g) * 2 - 1).to(v2.dtype) * 1e4
    O2 = oracle.attention(q, k2, v2, key_lens=kl, causal=causal)
    np.testing.assert_array_equal(O, O2)


# --- edge cases of the definition -------------------------------------------------

def test_key_lens_are_clamped():
    B, H, n, d = 3, 1, 6, 4
    q, k, v, _ = inputs.draw(B, H, n, n, d, d, "f32", seed=27)
    O1 = oracle.attention(q, k, v, key_lens=np.array([-5, 100, 0], np.int32))
    O2 = oracle.attention(q, k, v, key_lens=np.array([0, n, 0], np.int32))
    np.testing.assert_array_equal(O1, O2)
    assert np.all(O1[0] == 0) and np.all(O1[2] == 0)


def test_sampled_rows_equal_full_oracle():
    B, H, n, m, d = 2, 3, 50, 50, 8
    q, k, v, kl = inputs.draw(B, H, n, m, d, d, "bf16", seed=28, lens=(5, m))
    for causal in (False, True):
        O = oracle.attention(q, k, v, key_lens=kl, causal=causal)
        rows = np.array([[b, t, i] for b in range(B) for t in range(H) for i in (0, 7, n - 1)])
        Or = oracle.attention_rows(q, k, v, rows, key_lens=kl, causal=causal)
        np.testing.assert_array_equal(Or, O[rows[:, 0], rows[:, 1], rows[:, 2]])


def test_causal_requires_square():
    q, k, v, _ = inputs.draw(1, 1, 4, 5, 4, 4, "f32", seed=29)
    with pytest.raises(ValueError):
        oracle.attention(q, k, v, causal=True)


# --- P-11: the generator's statistics --------------------------------------------

@pytest.mark.parametrize("name,expected", [
    ("encoder_pad_n128", 1.0), ("decoder_causal_n512", 1.0), ("cross_n256_m1024", 1.0),
    ("causal_n16384_d128", 0.0625),
])
def test_generator_score_variance(name, expected):
    # For iid zero-mean q and k components of variance s^2, q.k has variance
    # d_k s^4 ("序列建模架构的演进与变革（二）" §4.4: d_k for unit variance),
    # so the score scaled by 1/sqrt(d_k) has variance s^4: 1 for N(0, 1)
    # inputs, and 0.5^4 = 0.0625 for the long workload's N(0, 1) * 0.5.
    # Every matched pair q_i . k_i of every head is one sample (32768 to
    # 262144 of them: the sample variance is within about 1% of the truth,
    # so the 5% band is at least five standard errors wide).
    w = inputs.WORKLOADS[name]
    q, k, v, kl = inputs.make(w)
    r = min(w.n, w.m)
    qs = q[:, :, :r].double().reshape(-1, w.d)
    ks = k[:, :, :r].double().reshape(-1, w.d)
    s = (qs * ks).sum(-1) * w.scale
    assert abs(float(s.var()) / expected - 1.0) < 0.05, float(s.var())
    assert abs(float(s.mean())) < 0.05 * expected ** 0.5
    if w.lens is not None:
        lo, hi = w.lens
        assert kl.min() >= lo and kl.max() <= hi and kl.dtype == np.int32


def test_generator_is_deterministic_and_rounds_to_nearest_even():
    a = inputs.draw(2, 2, 8, 8, 8, 8, "bf16", seed=9, lens=(1, 8))
    b = inputs.draw(2, 2, 8, 8, 8, 8, "bf16", seed=9, lens=(1, 8))
    for x, y in zip(a[:3], b[:3]):
        assert torch.equal(x, y)
    np.testing.assert_array_equal(a[3], b[3])
    rng = np.random.Generator(np.random.PCG64(9))
    q32 = rng.standard_normal((2, 2, 8, 8)).astype(np.float32)
    # round-to-nearest-even on the upper 16 bits, done on the integer bits
    u = q32.view(np.uint32).astype(np.uint64)
    rne = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    got = a[0].view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(got, rne)
