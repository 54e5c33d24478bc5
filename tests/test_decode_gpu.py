"""GPU parity of mha_decode (few new queries against a key/value cache).

The decode pass must give the result of the extended oracle with
bottom-right causal alignment and key_lens = cache_lens: query i is the
token at position i + L_b - n of a cache filled to L_b rows.  Tolerances are
those of the forward pass (O: 1e-5 fp32, 1.5e-2 bf16; lse: 2e-5 fp32,
3e-3 bf16, see test_parity_ex_gpu.py for their derivation).
"""
import numpy as np
import pytest
import torch

import oracle
import transformer_head_scaled_fwd_amd as mha
from transformer_head_scaled_fwd_amd import inputs
from test_parity_ex_gpu import TOL_LSE, TOL_O, draw, far_inputs, maxerr

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _say(msg):
    print(msg, flush=True)


def run_decode(q, k, v, kl, sl, scale=None, workspace=None):
    dl = lambda t: None if t is None else torch.as_tensor(t).to(DEV)  # noqa: E731
    o, lse = mha.decode(q.to(DEV), k.to(DEV), v.to(DEV), cache_lens=dl(kl),
                        alibi_slopes=dl(sl), scale=scale, return_lse=True,
                        workspace=workspace)
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu()


CASES = [
    # B, H, Hkv, n, m, d, dtype, alibi, lens
    (4, 32, 8, 1, 4096, 128, "bf16", False, (1000, 4096)),   # split over workgroups
    (2, 8, 1, 3, 2000, 64, "bf16", True, (1, 2000)),         # MQA, 24 rows, ragged cache
    (1, 16, 2, 5, 1500, 128, "bf16", False, None),           # 40 rows: two row sets
    (3, 4, 4, 1, 300, 64, "bf16", True, (0, 300)),           # an empty cache
    (2, 4, 2, 6, 100, 64, "bf16", False, (3, 100)),          # more queries than keys
    (64, 16, 16, 1, 256, 64, "bf16", False, (100, 256)),     # no split: direct store
    (2, 8, 2, 2, 1000, 128, "f32", True, (500, 1000)),
    (2, 4, 4, 1, 700, 64, "f32", False, None),
    # one sequence, MQA, a long cache: 128 splits per row, merged by four
    # waves per row; and a ragged pair with 40 splits and ALiBi
    (1, 32, 1, 1, 32768, 128, "bf16", False, None),
    (2, 8, 1, 1, 20000, 64, "bf16", True, (9000, 20000)),
]


@pytest.mark.parametrize("B,H,Hkv,n,m,d,dt,alibi,lens", CASES)
def test_decode_parity(gpu, B, H, Hkv, n, m, d, dt, alibi, lens):
    _say("decode B=%d H=%d Hkv=%d n=%d m=%d d=%d %s alibi=%s lens=%s"
         % (B, H, Hkv, n, m, d, dt, alibi, lens))
    q, k, v, kl = draw(B, H, Hkv, n, m, d, dt, seed=1300 + n + m + d + H, lens=lens)
    if kl is not None and lens[0] == 0:
        kl[0] = 0
    sl = inputs.alibi_slopes(H) if alibi else None
    o, lse = run_decode(q, k, v, kl, sl)
    o_ref, lse_ref = oracle.attention_ex(q, k, v, key_lens=kl, causal="bottom_right",
                                         alibi_slopes=sl, scale=mha.default_scale(d),
                                         return_lse=True)
    assert torch.isfinite(o.float()).all()
    assert maxerr(o, o_ref, "O") <= TOL_O[dt]
    assert np.array_equal(np.isneginf(oracle.to_f64(lse)), np.isneginf(lse_ref))
    assert maxerr(lse, lse_ref, "lse") <= TOL_LSE[dt]


def test_decode_ignores_workspace_contents_and_padding(gpu):
    # The workspace carries nothing between calls, and cache rows past L_b
    # are never read: NaN in either changes no bit of the result.
    B, H, Hkv, n, m, d = 4, 32, 8, 2, 3000, 128
    q, k, v, kl = draw(B, H, Hkv, n, m, d, "bf16", seed=1401, lens=(700, 3000))
    need = mha.decode_workspace_size(B, H, Hkv, n, m, d, mha.MHA_BF16)
    assert need > 0
    ws = torch.zeros(need, dtype=torch.uint8, device=DEV)
    o1, l1 = run_decode(q, k, v, kl, None, workspace=ws)
    ws.view(torch.float32).fill_(float("nan"))
    k2, v2 = k.clone(), v.clone()
    for b in range(B):
        k2[b, :, kl[b]:] = float("nan")
        v2[b, :, kl[b]:] = float("nan")
    o2, l2 = run_decode(q, k2, v2, kl, None, workspace=ws)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    o3, l3 = run_decode(q, k, v, kl, None, workspace=ws)
    assert torch.equal(o1, o3) and torch.equal(l1, l3)   # run to run


def test_decode_workspace_reused_across_sizes(gpu):
    # One workspace, filled with NaN first, serves calls of different sizes
    # in turn, and every result matches the oracle.
    cases = [(1, 32, 32, 1, 8192, 128, None), (2, 8, 1, 4, 5000, 64, (1000, 5000)),
             (1, 32, 32, 1, 8192, 128, None), (3, 16, 4, 1, 2100, 128, (64, 2100))]
    need = max(mha.decode_workspace_size(B, H, Hkv, n, m, d, mha.MHA_BF16)
               for B, H, Hkv, n, m, d, _ in cases)
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    ws.view(torch.float32).fill_(float("nan"))
    for i, (B, H, Hkv, n, m, d, lens) in enumerate(cases):
        q, k, v, kl = draw(B, H, Hkv, n, m, d, "bf16", seed=1410 + i, lens=lens)
        assert mha.decode_workspace_size(B, H, Hkv, n, m, d, mha.MHA_BF16) > 0
        o, lse = run_decode(q, k, v, kl, None, workspace=ws)
        o_ref, lse_ref = oracle.attention_ex(q, k, v, key_lens=kl, causal="bottom_right",
                                             return_lse=True)
        assert maxerr(o, o_ref, "O") <= TOL_O["bf16"]


def test_decode_matches_forward_ex(gpu):
    # The same operation through the prefill-shaped kernel.
    B, H, Hkv, n, m, d = 2, 16, 4, 3, 1200, 64
    q, k, v, kl = draw(B, H, Hkv, n, m, d, "bf16", seed=1402, lens=(400, 1200))
    o_dec, _ = run_decode(q, k, v, kl, None)
    o_fwd = mha.forward_ex(q.to(DEV), k.to(DEV), v.to(DEV), key_lens=torch.as_tensor(kl).to(DEV),
                           causal="bottom_right")
    torch.cuda.synchronize()
    assert (o_dec.float() - o_fwd.cpu().float()).abs().max().item() <= 2 * TOL_O["bf16"]


@pytest.mark.parametrize("name", ["decode_gqa_m16384", "decode_mha_m8192"])
def test_decode_workload_every_row(gpu, name):
    # The benchmarked decode workloads at full size, in the launch
    # configuration bench.py times; every output row against the oracle.
    w = inputs.EXT_WORKLOADS[name]
    _say("decode workload %s" % name)
    q, k, v, kl, sl = inputs.draw_ex(w)
    o, lse = run_decode(q, k, v, kl, sl, scale=w.scale)
    rows = np.array([[b, t, i] for b in range(w.B) for t in range(w.H) for i in range(w.n)],
                    np.int64)
    ref, lref = oracle.attention_ex_rows(q, k, v, rows, key_lens=kl, causal="bottom_right",
                                         alibi_slopes=sl, scale=w.scale)
    assert maxerr(o.reshape(-1, w.d), ref, "O") <= TOL_O[w.dtype]
    assert maxerr(lse.reshape(-1), lref, "lse") <= TOL_LSE[w.dtype]


def test_decode_at_the_per_head_limit(gpu):
    # A cache head of 2^23 - 1 rows of d = 128 bf16, just under the 2 GiB the
    # kernels' 32-bit offsets allow, filled to L rows; NaN past L.  With
    # Q = 0 every visible score is equal, so the output is the mean of the
    # valid value rows ("序列建模架构的演进与变革（二）" §4.3: the weights sum
    # to 1), whatever the split of the key axis.
    m, d = (1 << 23) - 1, 128
    L = m - 5
    _say("decode at the limit: m=%d (filled %d) d=%d bf16" % (m, L, d))
    k = inputs.device_normal((1, 1, m, d), seed=44)
    v = inputs.device_normal((1, 1, m, d), seed=45)
    k[0, 0, L:] = float("nan")
    v[0, 0, L:] = float("nan")
    q = torch.zeros((1, 1, 1, d), dtype=torch.bfloat16, device=DEV)
    o = mha.decode(q, k, v, cache_lens=torch.tensor([L], dtype=torch.int32, device=DEV))
    torch.cuda.synchronize()
    vh = v[0, 0, :L].cpu()
    total = np.zeros(d)
    for c0 in range(0, L, 1 << 20):
        total += oracle.to_f64(vh[c0:c0 + (1 << 20)]).sum(axis=0)
    ref = (total / L).reshape(1, 1, 1, d)
    assert maxerr(o.cpu(), ref, "O") <= TOL_O["bf16"]
    del k, v, o
    torch.cuda.empty_cache()


def test_decode_binding_rejects_host_workspace(gpu):
    q, k, v, kl = draw(4, 32, 8, 1, 4096, 128, "bf16", seed=12, lens=(1000, 4096))
    host_ws = torch.empty(1 << 22, dtype=torch.uint8)
    with pytest.raises(ValueError):
        mha.decode(q.to(DEV), k.to(DEV), v.to(DEV), cache_lens=torch.as_tensor(kl).to(DEV),
                   workspace=host_ws)


# Decode without ALiBi takes every block on the weights-first path, the first
# included: a row with no running max yet must take the exact path at its
# first block with a valid key, even when its weights against 0 all
# underflow to 0 (scores far below 0, see far_inputs).  A wave holds 32 query
# rows of one K/V head; rows past the head's group * n are padding lanes with
# q = 0, whose first block always takes the exact path for the whole wave,
# so the cases that matter fill all 32 rows (group * n = 32).  fp32 compares
# O only, as in the forward test.
@pytest.mark.parametrize("B,H,Hkv,n,m,d,dt,alibi,lens", [
    (1, 32, 1, 1, 700, 64, "bf16", False, None),             # MQA, one full row set
    (2, 8, 1, 4, 5000, 128, "bf16", False, (2000, 5000)),    # full row set, split
    (1, 16, 1, 3, 900, 64, "bf16", False, (1, 900)),         # a full set and a partial one
    (1, 32, 1, 1, 300, 64, "f32", False, (1, 300)),
    (2, 8, 2, 1, 700, 64, "bf16", False, None),              # padding lanes in every wave
    (2, 8, 2, 2, 900, 128, "bf16", True, (400, 900)),        # ALiBi: exact every block
])
def test_decode_far_scores(gpu, B, H, Hkv, n, m, d, dt, alibi, lens):
    _say("decode far scores B=%d H=%d Hkv=%d n=%d m=%d d=%d %s alibi=%s lens=%s"
         % (B, H, Hkv, n, m, d, dt, alibi, lens))
    q, k, v = far_inputs(B, H, Hkv, n, m, d, dt, seed=83)
    kl = None
    if lens is not None:
        kl = np.linspace(lens[0], lens[1], B).astype(np.int32)
    sl = inputs.alibi_slopes(H) if alibi else None
    o, lse = run_decode(q, k, v, kl, sl)
    o_ref, lse_ref = oracle.attention_ex(q, k, v, key_lens=kl, causal="bottom_right",
                                         alibi_slopes=sl, return_lse=True)
    assert maxerr(o, o_ref, "O") <= TOL_O[dt]
    assert np.array_equal(np.isneginf(oracle.to_f64(lse)), np.isneginf(lse_ref))
    if dt == "bf16":
        assert maxerr(lse, lse_ref, "lse") <= TOL_LSE[dt]
