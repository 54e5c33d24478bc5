"""GPU parity of the forward kernel's two-key-group workgroups.

For bf16 inputs the forward kernel splits the key axis between two groups
of waves when the grid is small (at most 256 workgroups of 128 query rows,
i.e. B * H * ceil(n / 128) <= 256) and the key axis is long (m >= 1024).
Each group walks every other 64-key block and the two partial softmax sums
(running max, row sum, unnormalised output) are merged before the store.
Every shape below satisfies that rule, so each test runs the merge.

Bars as for the core operation: max-abs 1.5e-2 on O (bf16 inputs, fp32
accumulation), 3e-3 on the log-sum-exp; bitwise where the method makes the
result exact.
"""
import numpy as np
import pytest
import torch

import oracle
import transformer_head_scaled_fwd_amd as mha
from transformer_head_scaled_fwd_amd import inputs

pytestmark = pytest.mark.gpu

TOL_O = 1.5e-2
TOL_LSE = 3e-3
DEV = "cuda:0"


def _say(msg):
    print(msg, flush=True)


def splits(B, H, n, m):
    return B * H * -(-n // 128) <= 256 and m >= 1024


def maxerr(got, ref, what):
    g = oracle.to_f64(got)
    both_inf = np.isneginf(g) & np.isneginf(ref)
    with np.errstate(invalid="ignore"):
        err = np.where(both_inf, 0.0, np.abs(g - ref))
    mx = float(err.max()) if err.size else 0.0
    _say("%s max_abs_err=%.3e at %s" % (what, mx, np.unravel_index(np.argmax(err), err.shape)))
    return mx


CASES = [
    # B, H, Hkv, n, m, d, causal, alibi, lens
    (2, 2, 2, 300, 1100, 64, False, False, (0, 1100)),       # one empty sequence, ragged tails
    (1, 2, 2, 1100, 1100, 64, "top_left", False, None),      # causal, diagonal in both groups
    (1, 2, 1, 1030, 1030, 128, "top_left", True, None),      # MQA + ALiBi, d = 128
    (2, 4, 2, 200, 1300, 128, "bottom_right", True, (700, 1300)),
    (3, 2, 2, 70, 1024, 64, False, True, (1, 1024)),         # ragged, the last of one key
    (1, 3, 3, 129, 1088, 64, False, False, (1025, 1088)),    # length past a stage boundary
    (2, 2, 1, 5, 4000, 128, "bottom_right", False, (64, 4000)),
    # B * H_kv a multiple of 8 with grouped heads: each K/V head's workgroups
    # are pinned to one XCD as well
    (8, 8, 2, 100, 1100, 64, False, False, (500, 1100)),
    (8, 4, 1, 64, 1024, 128, "bottom_right", True, (900, 1024)),
]


@pytest.mark.parametrize("B,H,Hkv,n,m,d,causal,alibi,lens", CASES)
def test_key_split_parity(gpu, B, H, Hkv, n, m, d, causal, alibi, lens):
    assert splits(B, H, n, m)
    _say("key split: B=%d H=%d Hkv=%d n=%d m=%d d=%d causal=%s alibi=%s lens=%s"
         % (B, H, Hkv, n, m, d, causal, alibi, lens))
    q, _, _, _ = inputs.draw(B, H, n, 1, d, d, "bf16", seed=700 + n + m)
    _, k, v, kl = inputs.draw(B, Hkv, 1, m, d, d, "bf16", seed=701 + n + m, lens=lens)
    if kl is not None and lens[0] == 0:
        kl[0] = 0
    if kl is not None and lens[0] == 1:
        kl[-1] = 1
    sl = inputs.alibi_slopes(H) if alibi else None
    dl = lambda t: None if t is None else torch.as_tensor(t).to(DEV)  # noqa: E731
    o, lse = mha.forward_ex(q.to(DEV), k.to(DEV), v.to(DEV), key_lens=dl(kl), causal=causal,
                            alibi_slopes=dl(sl), return_lse=True)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention_ex(q, k, v, key_lens=kl, causal=causal, alibi_slopes=sl,
                                         scale=mha.default_scale(d), return_lse=True)
    assert torch.isfinite(o.float()).all()
    assert maxerr(o.cpu(), o_ref, "O") <= TOL_O
    assert np.array_equal(np.isneginf(oracle.to_f64(lse.cpu())), np.isneginf(lse_ref))
    assert maxerr(lse.cpu(), lse_ref, "lse") <= TOL_LSE
    if kl is not None and lens[0] == 0:
        assert torch.count_nonzero(o[0]) == 0


@pytest.mark.parametrize("d", [64, 128])
def test_key_split_causal_row0_is_v0_bitwise(gpu, d):
    # Row 0 sees key 0 only: key group 1 contributes nothing (weight 0) and
    # key group 0's single weight is exactly 1.
    B, H, n = 1, 2, 1024
    assert splits(B, H, n, n)
    q, k, v, _ = inputs.draw(B, H, n, n, d, d, "bf16", seed=71)
    o = mha.forward(q.to(DEV), k.to(DEV), v.to(DEV), causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o[:, :, 0].cpu(), v[:, :, 0])


@pytest.mark.parametrize("causal", [False, True])
def test_key_split_padding_is_never_read(gpu, causal):
    B, H, n, d = 2, 2, 1200, 64
    assert splits(B, H, n, n)
    q, k, v, kl = inputs.draw(B, H, n, n, d, d, "bf16", seed=72, lens=(600, n))
    kd = torch.as_tensor(kl).to(DEV)
    o1 = mha.forward(q.to(DEV), k.to(DEV), v.to(DEV), key_lens=kd, causal=causal)
    k2, v2 = k.clone(), v.clone()
    for b in range(B):
        L = int(kl[b])
        k2[b, :, L:] = float("nan")
        v2[b, :, L:] = float("inf")
    o2 = mha.forward(q.to(DEV), k2.to(DEV), v2.to(DEV), key_lens=kd, causal=causal)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)


def test_key_split_zero_query_is_mean_of_valid_values(gpu):
    # All valid scores equal: each row is the mean of the valid value rows,
    # however the keys are divided between the two groups.
    B, H, n, d = 3, 2, 100, 128
    m = 1500
    assert splits(B, H, n, m)
    _, k, v, kl = inputs.draw(B, H, 1, m, d, d, "bf16", seed=73, lens=(1, m))
    q = torch.zeros(B, H, n, d, dtype=torch.bfloat16)
    o = mha.forward(q.to(DEV), k.to(DEV), v.to(DEV), key_lens=torch.as_tensor(kl).to(DEV))
    torch.cuda.synchronize()
    V = oracle.to_f64(v)
    ref = np.stack([np.broadcast_to(V[b, :, :int(kl[b])].mean(axis=1)[:, None, :], (H, n, d))
                    for b in range(B)])
    assert maxerr(o.cpu(), ref, "Q=0 mean") <= TOL_O


def test_key_split_deterministic(gpu):
    B, H, n, m, d = 2, 4, 256, 2048, 64
    assert splits(B, H, n, m)
    q, k, v, kl = inputs.draw(B, H, n, m, d, d, "bf16", seed=74, lens=(1000, m))
    qd, kd, vd, ld = q.to(DEV), k.to(DEV), v.to(DEV), torch.as_tensor(kl).to(DEV)
    outs = [mha.forward(qd, kd, vd, key_lens=ld) for _ in range(3)]
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[1], outs[2])
