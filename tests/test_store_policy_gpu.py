"""The cache policy of result stores changes no bit of a result.

Launches whose results fit the L2s write them through to memory; larger
ones keep the default policy.  The same batch entry computed in a small
launch (written through) and in a large one (default) must agree bit for
bit: every workgroup's arithmetic is the same in both, only the stores'
cache policy and the grid differ.  Checked for the forward pass (O and the
log-sum-exp), the weights pass (A) and the multi-head layer (projections
and core).
"""
import pytest
import torch

import transformer_head_scaled_fwd_amd as mha
from transformer_head_scaled_fwd_amd import inputs

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
MIB = 1 << 20


def _say(msg):
    print(msg, flush=True)


def _batch(B, H, n, m, d, seed):
    q, k, v, _ = inputs.draw(B, H, n, m, d, d, "bf16", seed=seed)
    return q.to(DEV), k.to(DEV), v.to(DEV)


@pytest.mark.parametrize("causal,H,n,B", [(False, 32, 2048, 4), ("top_left", 16, 4096, 4)])
def test_forward_same_bits_streamed_or_not(gpu, causal, H, n, B):
    # 16 MiB of O per batch entry: one entry is written through, four
    # (64 MiB) keep the default policy.  Both sizes take the same workgroup
    # shape.
    d = 128
    q, k, v = _batch(B, H, n, n, d, seed=81)
    assert 1 * H * n * d * 2 <= 48 * MIB < B * H * n * d * 2
    lib = mha.load()
    mode = mha.mask_mode(causal)
    assert lib.mha_forward_kernel_name(1, H, H, n, n, d, mha.MHA_BF16, mode, 0) == \
        lib.mha_forward_kernel_name(B, H, H, n, n, d, mha.MHA_BF16, mode, 0)
    o4, l4 = mha.forward_ex(q, k, v, causal=causal, return_lse=True)  # B entries
    o1, l1 = mha.forward_ex(q[:1].contiguous(), k[:1].contiguous(), v[:1].contiguous(),
                            causal=causal, return_lse=True)
    torch.cuda.synchronize()
    _say("forward causal=%s: max |diff| %.3g" % (causal, (o4[:1].float() - o1.float()).abs().max()))
    assert torch.equal(o4[:1], o1)
    assert torch.equal(l4[:1], l1)


def test_weights_same_bits_streamed_or_not(gpu):
    # 16 MiB of A per batch entry: one entry streamed, four not.
    H, n, d = 8, 1024, 64
    q, k, v = _batch(4, H, n, n, d, seed=82)
    kl = torch.tensor([700, 1024, 300, 900], dtype=torch.int32, device=DEV)
    assert 1 * H * n * n * 2 <= 48 * MIB < 4 * H * n * n * 2
    _, lse4 = mha.forward_ex(q, k, v, key_lens=kl, causal="top_left", return_lse=True)
    a4 = mha.attention_weights(q, k, lse4, key_lens=kl, causal="top_left")
    q1, k1 = q[:1].contiguous(), k[:1].contiguous()
    _, lse1 = mha.forward_ex(q1, k1, v[:1].contiguous(), key_lens=kl[:1].contiguous(),
                             causal="top_left", return_lse=True)
    a1 = mha.attention_weights(q1, k1, lse1, key_lens=kl[:1].contiguous(), causal="top_left")
    torch.cuda.synchronize()
    assert torch.equal(lse4[:1], lse1)
    assert torch.equal(a4[:1], a1)


def test_layer_same_bits_streamed_or_not(gpu):
    # The Q/K/V projections write 3 MiB per batch entry: one entry streams
    # them, 17 (51 MiB) do not.  (n = 512 keeps the core on the same
    # workgroup shape for both batch sizes.)
    B, n, dm, H = 17, 512, 1024, 16
    g = torch.Generator().manual_seed(83)
    x = (torch.randn(B, n, dm, generator=g)).to(torch.bfloat16).to(DEV)
    ws = [(torch.rand(dm, dm, generator=g) * 2 - 1).mul(dm ** -0.5).to(torch.bfloat16).to(DEV)
          for _ in range(4)]
    bs = [(torch.rand(dm, generator=g) * 2 - 1).mul(dm ** -0.5).to(torch.bfloat16).to(DEV)
          for _ in range(4)]
    assert 1 * n * 3 * dm * 2 <= 48 * MIB < B * n * 3 * dm * 2
    args = (ws[0], bs[0], ws[1], bs[1], ws[2], bs[2], ws[3], bs[3], H)
    y5 = mha.multihead_forward(x, x, x, *args, causal=True)
    x1 = x[:1].contiguous()
    y1 = mha.multihead_forward(x1, x1, x1, *args, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(y5[:1], y1)
