"""Pins of the multi-head oracle (projections, head split, core, concat,
output projection) against torch's float64 multi_head_attention_forward, a
library implementation that shares no code with the oracle, and against a
closed form.  CPU only."""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle


def _weights(dm, seed, bias=True):
    rng = np.random.default_rng(seed)
    bound = 1.0 / np.sqrt(dm)   # nn.Linear's default init range
    W = [rng.uniform(-bound, bound, (dm, dm)) for _ in range(4)]
    b = [rng.uniform(-bound, bound, dm) if bias else None for _ in range(4)]
    return W, b


def _torch_mha(xq, xk, xv, W, b, H, key_lens=None, causal=False):
    B, n, dm = xq.shape
    m = xk.shape[1]
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a))  # noqa: E731
    kpm = None
    if key_lens is not None:
        kpm = torch.arange(m)[None, :] >= torch.as_tensor(key_lens)[:, None]
    am = None
    if causal:
        am = torch.triu(torch.ones(n, m, dtype=torch.bool), diagonal=1)
    in_b = None if b[0] is None else t(np.concatenate(b[:3]))
    y, w = F.multi_head_attention_forward(
        t(xq).transpose(0, 1), t(xk).transpose(0, 1), t(xv).transpose(0, 1), dm, H,
        t(np.concatenate(W[:3])), in_b, None, None, False, 0.0, t(W[3]),
        None if b[3] is None else t(b[3]), training=False, key_padding_mask=kpm,
        need_weights=True, attn_mask=am, average_attn_weights=False)
    return y.transpose(0, 1).numpy(), w.numpy()


@pytest.mark.parametrize("B,n,m,dm,H,causal,lens,bias", [
    (2, 5, 5, 16, 2, False, None, True),
    (2, 6, 6, 24, 3, True, None, True),
    (3, 4, 7, 16, 4, False, [7, 3, 5], True),
    (2, 6, 6, 32, 2, True, [6, 4], False),
])
def test_multihead_matches_torch(B, n, m, dm, H, causal, lens, bias):
    rng = np.random.default_rng(B * 100 + n + m + dm)
    xq = rng.standard_normal((B, n, dm))
    xk = rng.standard_normal((B, m, dm))
    xv = rng.standard_normal((B, m, dm))
    W, b = _weights(dm, dm + H, bias)
    kl = None if lens is None else np.array(lens, np.int32)
    Y, A = oracle.multihead(xq, xk, xv, W[0], b[0], W[1], b[1], W[2], b[2], W[3], b[3], H,
                            key_lens=kl, causal=causal, scale=1.0 / np.sqrt(dm // H),
                            return_weights=True)
    Yt, At = _torch_mha(xq, xk, xv, W, b, H, kl, causal)
    np.testing.assert_allclose(Y, Yt, rtol=0, atol=1e-12)
    np.testing.assert_allclose(A, At, rtol=0, atol=1e-12)


def test_multihead_self_attention_uses_one_input():
    # Encoder self-attention: query = key = value = x.
    rng = np.random.default_rng(5)
    x = rng.standard_normal((2, 6, 16))
    W, b = _weights(16, 9)
    Y = oracle.multihead(x, x, x, W[0], b[0], W[1], b[1], W[2], b[2], W[3], b[3], 4,
                         scale=0.5)
    Yt, _ = _torch_mha(x, x, x, W, b, 4)
    np.testing.assert_allclose(Y, Yt, rtol=0, atol=1e-12)


def test_multihead_zero_query_projection_is_mean_pooling():
    # W_Q = 0, b_Q = 0: every score is 0, the weights are uniform over the
    # L_b valid keys, so each head outputs the mean of its value rows and
    # Y = (mean_j xv_j Wv^T + bv) Wo^T + bo for every query row.
    rng = np.random.default_rng(6)
    B, n, m, dm, H = 2, 3, 5, 8, 2
    xq, xk, xv = (rng.standard_normal((B, L, dm)) for L in (n, m, m))
    W, b = _weights(dm, 10)
    lens = np.array([5, 2], np.int32)
    Y = oracle.multihead(xq, xk, xv, np.zeros((dm, dm)), None, W[1], b[1], W[2], b[2],
                         W[3], b[3], H, key_lens=lens, scale=0.7)
    for bb in range(B):
        mean_x = xv[bb, :lens[bb]].mean(axis=0)
        want = (mean_x @ W[2].T + b[2]) @ W[3].T + b[3]
        for i in range(n):
            np.testing.assert_allclose(Y[bb, i], want, rtol=0, atol=1e-13)


MHA_MUTANTS = {
    # heads taken as every H-th feature instead of contiguous blocks of d_k
    "heads_interleaved": ("rows = slice(t * dk, (t + 1) * dk)", "rows = slice(t, dm, H)"),
    # the projection uses columns of the [out, in] weight (its transpose)
    "projection_transposed": ("np.matmul(x, W[name][rows].T)", "np.matmul(x, W[name][:, rows])"),
    "key_projection_on_values": ('K = np.stack([head_projection(Xk, "k", t)',
                                 'K = np.stack([head_projection(Xv, "k", t)'),
    # head t meets rows, not columns, of the output weight
    "output_projection_transposed": ('W["o"][:, t * dk:(t + 1) * dk].T',
                                     'W["o"][t * dk:(t + 1) * dk, :]'),
    "output_bias_dropped": ('Y = np.zeros((B, n, dm)) if bias["o"] is None else',
                            'Y = np.zeros((B, n, dm)) if True else'),
}


@pytest.mark.parametrize("name", sorted(MHA_MUTANTS))
def test_mha_pins_catch_planted_mistake(monkeypatch, name):
    import inspect
    old, new = MHA_MUTANTS[name]
    src = inspect.getsource(oracle.multihead)
    assert old in src
    ns = dict(oracle.__dict__)
    exec(compile(src.replace(old, new), "<mutant>", "exec"), ns)
    monkeypatch.setattr(oracle, "multihead", ns["multihead"])
    caught = 0
    for case in [(3, 4, 7, 16, 4, False, [7, 3, 5], True), (2, 6, 6, 24, 3, True, None, True)]:
        try:
            test_multihead_matches_torch(*case)
        except (AssertionError, ValueError):
            caught += 1
    assert caught > 0, name
