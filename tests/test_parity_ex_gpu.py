"""GPU parity of the extended entry points against the CPU oracle.

mha_forward_ex (grouped K/V heads, ALiBi, top-left and bottom-right causal
alignment, log-sum-exp output) and mha_attention_weights, called through the
C ABI via the binding, on seeded inputs the oracle also receives.

Tolerances (max-abs over every compared element):
  O       1e-5 (fp32), 1.5e-2 (bf16): as for the core operation.
  lse     2e-5 (fp32); 3e-3 (bf16): the kernel's row sum adds the weights
          after rounding them to bf16 (relative error <= 2^-9 each), so
          |d ln l| <= 2^-9 ~ 1.95e-3, plus fp32 rounding of the scores.
  A       2e-5 (fp32); 5e-3 (bf16): A <= 1 is stored in bf16 (half an ulp
          <= 2^-9 ~ 1.95e-3) and carries the lse error above (<= 3e-3 * A).
Masked weights must be exactly 0.
"""
import numpy as np
import pytest
import torch

import oracle
import transformer_head_scaled_fwd_amd as mha
from transformer_head_scaled_fwd_amd import inputs

pytestmark = pytest.mark.gpu

TOL_O = {"f32": 1e-5, "bf16": 1.5e-2}
TOL_LSE = {"f32": 2e-5, "bf16": 3e-3}
TOL_A = {"f32": 2e-5, "bf16": 5e-3}
DEV = "cuda:0"


def _say(msg):
    print(msg, flush=True)


slopes = inputs.alibi_slopes


def draw(B, H, Hkv, n, m, d, dt, seed, lens=None):
    """Q with H heads, K/V with Hkv heads, from the shared generator."""
    q, _, _, kl = inputs.draw(B, H, n, 1, d, d, dt, seed=seed, lens=None)
    _, k, v, kl = inputs.draw(B, Hkv, 1, m, d, d, dt, seed=seed + 7919, lens=lens)
    return q, k, v, kl


def gpu_ex(q, k, v, kl, causal, sl, scale=None, weights=False):
    dl = lambda t: None if t is None else torch.as_tensor(t).to(DEV)  # noqa: E731
    res = mha.forward_ex(q.to(DEV), k.to(DEV), v.to(DEV), key_lens=dl(kl), causal=causal,
                         alibi_slopes=dl(sl), scale=scale, return_lse=True,
                         need_weights=weights)
    torch.cuda.synchronize()
    return [r.cpu() for r in res]


def maxerr(got, ref, what):
    g = oracle.to_f64(got)
    both_inf = np.isneginf(g) & np.isneginf(ref)
    with np.errstate(invalid="ignore"):  # -inf - -inf: both rows have no valid key
        err = np.where(both_inf, 0.0, np.abs(g - ref))
    mx = float(err.max()) if err.size else 0.0
    where = np.unravel_index(np.argmax(err), err.shape) if err.size else ()
    _say("%s max_abs_err=%.3e at %s" % (what, mx, where))
    return mx


CASES = [
    # B, H, Hkv, n, m, d, dtype, causal, alibi, lens
    (2, 8, 2, 300, 300, 64, "bf16", "top_left", False, (1, 300)),
    (2, 8, 1, 200, 333, 128, "bf16", False, False, (100, 333)),
    (1, 6, 3, 257, 257, 128, "bf16", "top_left", True, None),
    (2, 4, 4, 190, 190, 64, "bf16", False, True, (0, 190)),
    (2, 4, 2, 1, 700, 128, "bf16", "bottom_right", False, (1, 700)),
    (3, 4, 1, 5, 1000, 64, "bf16", "bottom_right", True, (3, 1000)),
    (2, 4, 2, 77, 300, 128, "bf16", "bottom_right", True, (50, 300)),
    (2, 2, 2, 300, 120, 64, "bf16", "bottom_right", False, (10, 120)),
    (2, 4, 2, 129, 129, 64, "f32", "top_left", True, (1, 129)),
    (2, 4, 1, 9, 400, 128, "f32", "bottom_right", True, (1, 400)),
    (1, 2, 2, 100, 250, 64, "f32", False, True, None),
    # causal with ALiBi (key walk from the diagonal down): ragged lengths;
    # bottom-right with rows that see no key; two key groups; d = 128
    (2, 8, 4, 520, 520, 64, "bf16", "top_left", True, (1, 520)),
    (2, 4, 2, 300, 200, 64, "bf16", "bottom_right", True, (10, 200)),
    (1, 4, 4, 1100, 1100, 64, "bf16", "top_left", True, None),
    (1, 4, 2, 1200, 1500, 64, "bf16", "bottom_right", True, (700, 1500)),
    (2, 8, 2, 600, 600, 128, "bf16", "top_left", True, (1, 600)),
    (2, 4, 2, 300, 900, 128, "bf16", "bottom_right", True, (200, 900)),
    (1, 4, 4, 1200, 1200, 128, "bf16", "top_left", True, None),
    (1, 4, 2, 300, 300, 128, "f32", "top_left", True, (1, 300)),
    # block-index decode by launch-time divisors that are not powers of two:
    # K/V heads pinned to XCDs (batch x H_kv a multiple of 8) with groups of 3
    # and 5 K/V heads per batch, and the plain order with B x H = 15
    (8, 12, 4, 256, 256, 64, "bf16", "top_left", False, None),
    (8, 15, 5, 200, 300, 128, "bf16", False, True, (1, 300)),
    (8, 6, 2, 130, 400, 64, "bf16", "bottom_right", True, (130, 400)),
    (3, 5, 5, 300, 300, 64, "bf16", "top_left", False, (1, 300)),
]


@pytest.mark.parametrize("B,H,Hkv,n,m,d,dt,causal,alibi,lens", CASES)
def test_forward_ex_parity(gpu, B, H, Hkv, n, m, d, dt, causal, alibi, lens):
    _say("case B=%d H=%d Hkv=%d n=%d m=%d d=%d %s causal=%s alibi=%s lens=%s"
         % (B, H, Hkv, n, m, d, dt, causal, alibi, lens))
    q, k, v, kl = draw(B, H, Hkv, n, m, d, dt, seed=500 + n + m + d + H, lens=lens)
    if kl is not None and lens[0] == 0:
        kl[0] = 0
    sl = slopes(H) if alibi else None
    o, lse = gpu_ex(q, k, v, kl, causal, sl)
    o_ref, lse_ref = oracle.attention_ex(q, k, v, key_lens=kl, causal=causal,
                                         alibi_slopes=sl, scale=mha.default_scale(d),
                                         return_lse=True)
    assert torch.isfinite(o.float()).all()
    assert maxerr(o, o_ref, "O") <= TOL_O[dt]
    assert np.array_equal(np.isneginf(oracle.to_f64(lse)), np.isneginf(lse_ref))
    assert maxerr(lse, lse_ref, "lse") <= TOL_LSE[dt]


def _variant(B, H, Hkv, n, m, d, dt, causal, alibi):
    code = mha.MHA_BF16 if dt == "bf16" else mha.MHA_F32
    mode = {False: 0, "top_left": 1, "bottom_right": 2}[causal]
    return mha.load().mha_forward_kernel_name(B, H, Hkv, n, m, d, code, mode,
                                              int(alibi)).decode()


def _falling_inputs(B, H, n, m, d, dt, step, seed):
    # Key j lies step * (m - 1 - j) along every query's direction: walked
    # from the diagonal down to key 0, each 64-key block scores higher than
    # the one before by 64 * step * scale (46 in log2 units for step 4 at
    # d = 64, 23 for step 2; 33 for step 4 at d = 128, 24 for step 3), more
    # than the slopes below take away (at d = 128 they are divided by 8), so
    # every block's weights pass the on-demand bound: block max, raise,
    # rescale.
    _, _, v, _ = inputs.draw(B, H, n, m, d, d, dt, seed=seed)
    q = torch.zeros(B, H, n, d)
    k = torch.zeros(B, H, m, d)
    q[..., 0] = 1.0
    k[..., 0] = step * torch.arange(m - 1, -1, -1, dtype=torch.float32)
    k[..., 1] = torch.linspace(-1, 1, m)
    q[..., 1] = torch.linspace(1, -1, n)
    dtype = torch.bfloat16 if dt == "bf16" else torch.float32
    return q.to(dtype), k.to(dtype), v


# fp32 takes a smaller step over fewer keys: its scores' exponents reach
# step * m * scale * log2(e) (72 for step 2, m = 200; 76 for step 3 at
# d = 128), whose rounding in fp32 (2^-18 relative) must stay inside the
# 1e-5 tolerance.
@pytest.mark.parametrize("B,H,n,m,d,dt,causal,step,variant", [
    (2, 4, 700, 700, 64, "bf16", "top_left", 4.0, "<__bf16, 64, 4, 1, true, true>"),
    (1, 4, 1100, 1100, 64, "bf16", "top_left", 4.0, "<__bf16, 64, 8, 2, true, true>"),
    (2, 4, 300, 900, 64, "bf16", "bottom_right", 4.0, "<__bf16, 64, 4, 1, true, true>"),
    (1, 2, 200, 200, 64, "f32", "top_left", 2.0, "<float, 64, 4, 1, true, true>"),
    # d = 128: eight waves over 256 rows (the oracle on sampled rows), four
    # waves, two key groups, fp32
    (2, 16, 8192, 8192, 128, "bf16", "top_left", 4.0, "<__bf16, 128, 8, 1, true, true>"),
    (4, 16, 1024, 1024, 128, "bf16", "top_left", 4.0, "<__bf16, 128, 4, 1, true, true>"),
    (1, 4, 320, 1280, 128, "bf16", "bottom_right", 4.0, "<__bf16, 128, 8, 2, true, true>"),
    (1, 2, 200, 200, 128, "f32", "top_left", 3.0, "<float, 128, 4, 1, true, true>"),
])
def test_alibi_causal_falling_scores(gpu, B, H, n, m, d, dt, causal, step, variant):
    _say("ALiBi falling scores B=%d H=%d n=%d m=%d d=%d %s %s step %g"
         % (B, H, n, m, d, dt, causal, step))
    assert _variant(B, H, H, n, m, d, dt, causal, True).endswith(variant)
    q, k, v = _falling_inputs(B, H, n, m, d, dt, step, seed=71)
    sl = slopes(H) if d == 64 else slopes(H) / 8
    o, lse = gpu_ex(q, k, v, None, causal, sl)
    if B * H * n * m <= 1 << 27:
        o_ref, lse_ref = oracle.attention_ex(q, k, v, causal=causal, alibi_slopes=sl,
                                             scale=mha.default_scale(d), return_lse=True)
    else:
        rng = np.random.Generator(np.random.PCG64(72))
        flat = rng.choice(B * H * n, size=768, replace=False)
        rows = np.stack([flat // (H * n), (flat // n) % H, flat % n], 1)
        rows = np.concatenate([rows, [[B - 1, H - 1, n - 1], [0, 0, 0]]]).astype(np.int64)
        o_ref, lse_ref = oracle.attention_ex_rows(q, k, v, rows, causal=causal, alibi_slopes=sl,
                                                  scale=mha.default_scale(d))
        sel = tuple(torch.from_numpy(rows[:, c]) for c in range(3))
        o, lse = o[sel], lse[sel]
    assert maxerr(o, o_ref, "O") <= TOL_O[dt]
    assert maxerr(lse, lse_ref, "lse") <= TOL_LSE[dt]


# Top-left rows past a short sequence's length see only keys far behind
# them: with slope 8 their lse reaches -4000, where fp32 rounding alone is
# 2.4e-4, inside the bf16 tolerance but not the fp32 one; fp32 runs without
# lengths.
@pytest.mark.parametrize("d,dt,causal,lens", [
    (64, "bf16", "top_left", None),
    (64, "bf16", "top_left", (1, 640)),
    (64, "bf16", "bottom_right", (200, 640)),
    (64, "f32", "top_left", None),
    (128, "bf16", "top_left", (1, 640)),
    (128, "bf16", "bottom_right", (200, 640)),
    (128, "f32", "top_left", None),
])
def test_alibi_causal_steep_slopes(gpu, d, dt, causal, lens):
    # Slopes from 8 (a row's weight falls by e^-8 per key of distance, so
    # far keys underflow to 0) to 0 (no bias), on the causal path.
    B, H, n, m = 2, 4, 640, 640
    _say("ALiBi steep slopes d=%d %s %s lens=%s" % (d, dt, causal, lens))
    q, k, v, kl = draw(B, H, H, n, m, d, dt, seed=73, lens=lens)
    # With slope 8 a row's output is nearly its own value row, up to ~4.5
    # for N(0,1) values, where half a bf16 ulp (2^-6) alone would exceed the
    # tolerance: halve the values (exact in either type).
    v = (v.float() * 0.5).to(v.dtype)
    sl = np.array([8.0, 1.0, 0.03, 0.0], np.float32)
    o, lse = gpu_ex(q, k, v, kl, causal, sl)
    o_ref, lse_ref = oracle.attention_ex(q, k, v, key_lens=kl, causal=causal,
                                         alibi_slopes=sl, scale=mha.default_scale(d),
                                         return_lse=True)
    assert maxerr(o, o_ref, "O") <= TOL_O[dt]
    assert np.array_equal(np.isneginf(oracle.to_f64(lse)), np.isneginf(lse_ref))
    assert maxerr(lse, lse_ref, "lse") <= TOL_LSE[dt]



def far_inputs(B, H, Hkv, n, m, d, dt, seed):
    """Inputs whose every score lies far below 0: q = 48 e0 and key j =
    (-48 + delta_j) e0 with delta_j in {0, 0.25, 0.5, 0.75}, exact in bf16
    and fp32, and so are the dot products (-2304 + 48 delta_j).  Scaled to
    log2 units they lie below -290 (d = 128) or -415 (d = 64), so a weight
    taken against 0 instead of the row max underflows to exactly 0.  Values
    come from the shared generator."""
    _, _, v, _ = inputs.draw(B, Hkv, 1, m, d, d, dt, seed=seed)
    q = torch.zeros(B, H, n, d)
    k = torch.zeros(B, Hkv, m, d)
    q[..., 0] = 48.0
    k[..., 0] = -48.0 + 0.25 * (torch.arange(m) % 4).float()
    dtype = torch.bfloat16 if dt == "bf16" else torch.float32
    return q.to(dtype), k.to(dtype), v


# Causal ALiBi walks its keys backwards, so a row whose first walked blocks
# lie past its diagonal meets its first valid key with no running max yet;
# that block must take the exact path even though its weights against 0
# all underflow (a sum of 0).  Without ALiBi (the forward walk) the first
# block holds key 0.  fp32 adds the bias to raw scores near -2300, a rounding
# of up to 2300 * 2^-24 that moves each weight by about 1e-5 relative: its
# values are scaled by 1/4 (exact) so that O stays inside the 1e-5 bar, and
# its log-sum-exp near -200, carrying the same rounding, is not compared.
@pytest.mark.parametrize("B,H,Hkv,n,m,d,dt,causal,alibi,lens,variant", [
    (2, 4, 4, 300, 300, 64, "bf16", "top_left", True, None, "<__bf16, 64, 4, 1, true, true>"),
    (1, 4, 2, 1100, 1100, 64, "bf16", "top_left", True, None, "<__bf16, 64, 8, 2, true, true>"),
    (2, 4, 4, 200, 640, 64, "bf16", "bottom_right", True, (300, 640),
     "<__bf16, 64, 4, 1, true, true>"),
    (2, 4, 4, 300, 300, 128, "bf16", "top_left", True, (150, 300),
     "<__bf16, 128, 4, 1, true, true>"),
    (1, 4, 4, 320, 1280, 128, "bf16", "bottom_right", True, None,
     "<__bf16, 128, 8, 2, true, true>"),
    (2, 16, 4, 8192, 8192, 128, "bf16", "top_left", True, None,
     "<__bf16, 128, 8, 1, true, true>"),
    (1, 2, 2, 200, 200, 64, "f32", "top_left", True, None, "<float, 64, 4, 1, true, true>"),
    (1, 2, 2, 200, 200, 128, "f32", "bottom_right", True, (120, 200),
     "<float, 128, 4, 1, true, true>"),
    # the forward walk, with and without a causal mask
    (2, 4, 4, 300, 300, 64, "bf16", "top_left", False, (100, 300),
     "<__bf16, 64, 4, 1, true, false>"),
    (2, 4, 2, 150, 400, 128, "bf16", False, True, (1, 400), "<__bf16, 128, 4, 1, false, true>"),
])
def test_far_scores_first_valid_key(gpu, B, H, Hkv, n, m, d, dt, causal, alibi, lens, variant):
    _say("far scores B=%d H=%d Hkv=%d n=%d m=%d d=%d %s %s alibi=%s lens=%s"
         % (B, H, Hkv, n, m, d, dt, causal, alibi, lens))
    assert _variant(B, H, Hkv, n, m, d, dt, causal, alibi).endswith(variant)
    q, k, v = far_inputs(B, H, Hkv, n, m, d, dt, seed=81)
    if dt == "f32":
        v = v * 0.25
    kl = None
    if lens is not None:
        kl = np.linspace(lens[0], lens[1], B).astype(np.int32)
    sl = slopes(H) if alibi else None
    o, lse = gpu_ex(q, k, v, kl, causal, sl)
    if B * H * n * m <= 1 << 27:
        o_ref, lse_ref = oracle.attention_ex(q, k, v, key_lens=kl, causal=causal,
                                             alibi_slopes=sl, return_lse=True)
    else:
        rng = np.random.Generator(np.random.PCG64(82))
        flat = rng.choice(B * H * n, size=512, replace=False)
        rows = np.stack([flat // (H * n), (flat // n) % H, flat % n], 1)
        rows = np.concatenate([rows, [[0, 0, 0], [0, 0, 1], [B - 1, H - 1, n - 1]]]).astype(np.int64)
        o_ref, lse_ref = oracle.attention_ex_rows(q, k, v, rows, key_lens=kl, causal=causal,
                                                  alibi_slopes=sl)
        sel = tuple(torch.from_numpy(rows[:, c]) for c in range(3))
        o, lse = o[sel], lse[sel]
    assert maxerr(o, o_ref, "O") <= TOL_O[dt]
    assert np.array_equal(np.isneginf(oracle.to_f64(lse)), np.isneginf(lse_ref))
    if dt == "bf16":
        assert maxerr(lse, lse_ref, "lse") <= TOL_LSE[dt]

WCASES = [
    # B, H, Hkv, n, m, d, dtype, causal, alibi, lens
    (2, 4, 2, 150, 200, 64, "bf16", False, False, (30, 200)),
    (1, 4, 4, 130, 130, 128, "bf16", "top_left", True, None),
    (2, 4, 1, 7, 301, 64, "bf16", "bottom_right", True, (5, 301)),
    (2, 2, 2, 66, 97, 64, "bf16", False, False, None),          # m % 4 != 0
    (1, 2, 1, 65, 131, 128, "f32", "top_left", False, None),    # m % 4 != 0
    (2, 2, 2, 40, 120, 64, "f32", "bottom_right", True, (0, 120)),
    (2, 4, 2, 100, 256, 128, "bf16", "top_left", True, None),   # m % 8 == 0: staged rows
    (1, 3, 3, 70, 264, 128, "f32", False, False, (100, 264)),   # staged rows, fp32
    (2, 2, 1, 33, 132, 64, "bf16", "bottom_right", False, (7, 132)),  # m % 8 == 4
]


@pytest.mark.parametrize("B,H,Hkv,n,m,d,dt,causal,alibi,lens", WCASES)
def test_attention_weights_parity(gpu, B, H, Hkv, n, m, d, dt, causal, alibi, lens):
    _say("weights B=%d H=%d Hkv=%d n=%d m=%d d=%d %s causal=%s alibi=%s lens=%s"
         % (B, H, Hkv, n, m, d, dt, causal, alibi, lens))
    q, k, v, kl = draw(B, H, Hkv, n, m, d, dt, seed=900 + n + m + d, lens=lens)
    if kl is not None and lens[0] == 0:
        kl[0] = 0
    sl = slopes(H) if alibi else None
    o, lse, a = gpu_ex(q, k, v, kl, causal, sl, weights=True)
    o_ref, lse_ref, _, a_ref = oracle.attention_ex(
        q, k, v, key_lens=kl, causal=causal, alibi_slopes=sl, scale=mha.default_scale(d),
        return_lse=True, return_weights=True)
    assert a.dtype == q.dtype and tuple(a.shape) == (B, H, n, m)
    assert maxerr(o, o_ref, "O") <= TOL_O[dt]
    assert maxerr(a, a_ref, "A") <= TOL_A[dt]
    # masked pairs are exactly zero, and nothing else is NaN/Inf
    a64 = oracle.to_f64(a)
    assert np.all(a64[a_ref == 0.0] == 0.0)
    assert np.all(np.isfinite(a64))
    if dt == "f32":
        rows = a_ref.sum(-1) > 0
        np.testing.assert_allclose(a64.sum(-1)[rows], 1.0, atol=1e-5)


def test_forward_ex_equals_forward_on_the_core_operation(gpu):
    # H_kv = H, no bias: the same kernel and the same bits as mha_forward.
    for causal in (False, True):
        q, k, v, kl = inputs.draw(2, 4, 200, 200, 64, 64, "bf16", seed=31, lens=(50, 200))
        qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
        kld = torch.as_tensor(kl).to(DEV)
        a = mha.forward(qd, kd, vd, key_lens=kld, causal=causal)
        b = mha.forward_ex(qd, kd, vd, key_lens=kld, causal=causal)
        torch.cuda.synchronize()
        assert torch.equal(a, b)


def test_gqa_equals_repeated_heads_bitwise(gpu):
    # Reading K/V head t // group is the same computation as repeating the
    # K/V heads: the outputs agree bit for bit.
    B, H, Hkv, n, d = 2, 8, 2, 160, 128
    q, k, v, _ = draw(B, H, Hkv, n, n, d, "bf16", seed=77)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    rep = lambda t: t.repeat_interleave(H // Hkv, dim=1).contiguous()  # noqa: E731
    a = mha.forward_ex(qd, kd, vd, causal=True)
    b = mha.forward(qd, rep(kd), rep(vd), causal=True)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_bottom_right_full_cache_equals_top_left_bitwise(gpu):
    # With n == m and every key filled the two alignments coincide.
    q, k, v, _ = inputs.draw(2, 4, 300, 300, 64, 64, "bf16", seed=41, lens=None)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    a = mha.forward_ex(qd, kd, vd, causal="top_left")
    b = mha.forward_ex(qd, kd, vd, causal="bottom_right")
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_decode_long_cache_sampled_rows(gpu):
    # One decoding step against a long cache: B=4, H=32 query heads over 8
    # K/V heads, 4 new tokens each, caches of up to 16384 keys (of capacity
    # 16384), ALiBi.  The oracle evaluates every output row here.
    B, H, Hkv, n, m, d = 4, 32, 8, 4, 16384, 128
    q, k, v, kl = draw(B, H, Hkv, n, m, d, "bf16", seed=2024, lens=(1000, m))
    kl[0] = m
    sl = slopes(H)
    o, lse = gpu_ex(q, k, v, kl, "bottom_right", sl)
    rows = np.array([[b, t, i] for b in range(B) for t in range(H) for i in range(n)], np.int64)
    ref, lref = oracle.attention_ex_rows(q, k, v, rows, key_lens=kl, causal="bottom_right",
                                         alibi_slopes=sl, scale=mha.default_scale(d))
    got = o[rows[:, 0], rows[:, 1], rows[:, 2]]
    assert maxerr(got, ref, "O") <= TOL_O["bf16"]
    assert maxerr(lse.reshape(-1), lref, "lse") <= TOL_LSE["bf16"]


@pytest.mark.parametrize("name", ["gqa_prefill_n4096", "alibi_causal_n2048"])
def test_extended_workload_sampled_rows(gpu, name):
    # The benchmarked extended workloads at full size, in the launch
    # configuration bench.py times; the oracle evaluates sampled rows.
    w = inputs.EXT_WORKLOADS[name]
    _say("extended workload %s (sampled rows)" % name)
    q, k, v, kl, sl = inputs.draw_ex(w)
    o, lse = gpu_ex(q, k, v, kl, w.causal, sl, scale=w.scale)
    rng = np.random.Generator(np.random.PCG64(99))
    fixed = [0, 1, 63, 64, 127, 128, 255, 256, w.n - 129, w.n - 1]
    rows = []
    for b in range(w.B):
        for t in range(w.H):
            picks = sorted(set(fixed) | set(rng.integers(0, w.n, 6).tolist()))
            rows += [[b, t, i] for i in picks]
    rows = np.array(rows, np.int64)
    ref, lref = oracle.attention_ex_rows(q, k, v, rows, key_lens=kl, causal=w.causal,
                                         alibi_slopes=sl, scale=w.scale)
    got = o[rows[:, 0], rows[:, 1], rows[:, 2]]
    assert maxerr(got, ref, "O") <= TOL_O[w.dtype]
    gl = lse[rows[:, 0], rows[:, 1], rows[:, 2]]
    assert maxerr(gl, lref, "lse") <= TOL_LSE[w.dtype]


def test_weights_workload_full(gpu):
    w = inputs.EXT_WORKLOADS["weights_n512"]
    _say("extended workload %s (every element)" % w.name)
    q, k, v, kl, sl = inputs.draw_ex(w)
    o, lse, a = gpu_ex(q, k, v, kl, w.causal, sl, scale=w.scale, weights=True)
    o_ref, lse_ref, _, a_ref = oracle.attention_ex(
        q, k, v, key_lens=kl, causal=w.causal, alibi_slopes=sl, scale=w.scale,
        return_lse=True, return_weights=True)
    assert maxerr(o, o_ref, "O") <= TOL_O[w.dtype]
    assert maxerr(lse, lse_ref, "lse") <= TOL_LSE[w.dtype]
    assert maxerr(a, a_ref, "A") <= TOL_A[w.dtype]
    assert np.all(oracle.to_f64(a)[a_ref == 0.0] == 0.0)


def test_weights_at_the_per_head_limit(gpu):
    # A head of the weights is n x m elements and must stay under 2 GiB (the
    # kernels' 32-bit offsets): n = m = 32767 bf16 is 2,147,352,578 bytes.
    # Sampled rows, among them the last, against the oracle on those rows.
    n = m = 32767
    d = 64
    L = m - 3
    _say("weights at the limit: n=m=%d d=%d bf16, L=%d (%.4f GiB per head)"
         % (n, d, L, n * m * 2 / 2 ** 30))
    q, k, v, _ = inputs.draw(1, 1, n, m, d, d, "bf16", seed=41)
    kl = np.array([L], np.int32)
    o, lse, a = mha.forward_ex(q.to(DEV), k.to(DEV), v.to(DEV),
                               key_lens=torch.as_tensor(kl).to(DEV),
                               return_lse=True, need_weights=True)
    torch.cuda.synchronize()
    rng = np.random.Generator(np.random.PCG64(42))
    rows = np.unique(np.concatenate([[0, 1, 31, 32], np.arange(n - 40, n),
                                     rng.integers(0, n, 20)]))
    idx = torch.as_tensor(rows, device=DEV)
    a_s = a[0, 0].index_select(0, idx).cpu().reshape(1, 1, len(rows), m)
    o_s = o[0, 0].index_select(0, idx).cpu().reshape(1, 1, len(rows), d)
    qs = q[0, 0][torch.as_tensor(rows)].reshape(1, 1, len(rows), d)
    o_ref, _, _, a_ref = oracle.attention_ex(qs, k, v, key_lens=kl, scale=mha.default_scale(d),
                                             return_lse=True, return_weights=True)
    assert maxerr(o_s, o_ref, "O") <= TOL_O["bf16"]
    assert maxerr(a_s, a_ref, "A") <= TOL_A["bf16"]
    a64 = oracle.to_f64(a_s)
    assert np.all(a64[..., L:] == 0.0)
    assert np.all(np.isfinite(a64))
    del o, lse, a
    torch.cuda.empty_cache()
