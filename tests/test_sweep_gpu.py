"""GPU parity on a seeded random sweep of shapes and options.

Each case draws its own shape and options from a fixed generator: batch and
head counts, grouped K/V heads, n and m from 1 to a few hundred (so walks
span several key blocks and end in a ragged tail), d in {64, 128}, bf16 or
fp32, no mask / top-left / bottom-right causal alignment, optional ALiBi
slopes and key lengths (sometimes 0).  Every element of O and of the
log-sum-exp is compared with the oracle, to the bars of the other parity
tests.  The decode entry point gets a sweep of its own (n new queries
against a cache of capacity m).

One further case sends a large non-causal grid with key padding through
the eight-wave workgroups (sampled rows against the oracle).
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
DEV = "cuda:0"
MODES = [False, "top_left", "bottom_right"]


def _say(msg):
    print(msg, flush=True)


def _case(i):
    """Shape and options of sweep case i (a pure function of i)."""
    rng = np.random.Generator(np.random.PCG64(10_000 + i))
    dt = "f32" if rng.random() < 0.2 else "bf16"
    d = int(rng.choice([64, 128]))
    Hkv = int(rng.integers(1, 4))
    H = Hkv * int(rng.integers(1, 4))
    B = int(rng.integers(1, 4))
    n = int(rng.integers(1, 400))
    m = int(rng.integers(1, 400))
    mode = MODES[int(rng.integers(0, 3))]
    if mode == "top_left" and rng.random() < 0.5:
        m = n  # self-attention, the common causal case
    alibi = bool(rng.random() < 0.3)
    lens = None
    if rng.random() < 0.6:
        lo = 0 if rng.random() < 0.2 else int(rng.integers(1, m + 1))
        lens = (lo, m)
    return dict(B=B, H=H, Hkv=Hkv, n=n, m=m, d=d, dt=dt, mode=mode, alibi=alibi, lens=lens,
                seed=20_000 + i)


def _draw(c):
    q, _, _, _ = inputs.draw(c["B"], c["H"], c["n"], 1, c["d"], c["d"], c["dt"],
                             seed=c["seed"], lens=None)
    _, k, v, kl = inputs.draw(c["B"], c["Hkv"], 1, c["m"], c["d"], c["d"], c["dt"],
                              seed=c["seed"] + 7919, lens=c["lens"])
    sl = inputs.alibi_slopes(c["H"]) if c["alibi"] else None
    return q, k, v, kl, sl


def _dev(t):
    return None if t is None else torch.as_tensor(t).to(DEV)


def _maxerr(got, ref):
    g = oracle.to_f64(got)
    both_inf = np.isneginf(g) & np.isneginf(ref)
    with np.errstate(invalid="ignore"):  # -inf - -inf: both rows have no valid key
        err = np.where(both_inf, 0.0, np.abs(g - ref))
    return float(err.max()) if err.size else 0.0


@pytest.mark.parametrize("i", range(40))
def test_forward_ex_sweep(gpu, i):
    c = _case(i)
    _say("sweep case %d: %s" % (i, c))
    q, k, v, kl, sl = _draw(c)
    o, lse = mha.forward_ex(q.to(DEV), k.to(DEV), v.to(DEV), key_lens=_dev(kl),
                            causal=c["mode"], alibi_slopes=_dev(sl), return_lse=True)
    torch.cuda.synchronize()
    o, lse = o.cpu(), lse.cpu()
    ref_o, ref_lse = oracle.attention_ex(q, k, v, key_lens=kl, causal=c["mode"],
                                         alibi_slopes=sl, return_lse=True)
    eo, el = _maxerr(o, ref_o), _maxerr(lse, ref_lse)
    _say("  O max_abs_err=%.3e  lse max_abs_err=%.3e" % (eo, el))
    assert torch.isfinite(o.float()).all()
    assert eo <= TOL_O[c["dt"]]
    assert el <= TOL_LSE[c["dt"]]


def _dcase(i):
    rng = np.random.Generator(np.random.PCG64(30_000 + i))
    dt = "f32" if rng.random() < 0.2 else "bf16"
    d = int(rng.choice([64, 128]))
    Hkv = int(rng.integers(1, 5))
    H = Hkv * int(rng.choice([1, 2, 4, 8]))
    B = int(rng.integers(1, 4))
    n = int(rng.integers(1, 5))
    m = int(rng.integers(n, 3000))
    alibi = bool(rng.random() < 0.3)
    lens = None
    if rng.random() < 0.7:
        lens = (int(rng.integers(0, m + 1)), m)
    return dict(B=B, H=H, Hkv=Hkv, n=n, m=m, d=d, dt=dt, mode="bottom_right", alibi=alibi,
                lens=lens, seed=40_000 + i)


@pytest.mark.parametrize("i", range(16))
def test_decode_sweep(gpu, i):
    c = _dcase(i)
    _say("decode sweep case %d: %s" % (i, c))
    q, k, v, kl, sl = _draw(c)
    o = mha.decode(q.to(DEV), k.to(DEV), v.to(DEV), cache_lens=_dev(kl), alibi_slopes=_dev(sl))
    torch.cuda.synchronize()
    ref = oracle.attention_ex(q, k, v, key_lens=kl, causal="bottom_right", alibi_slopes=sl)
    e = _maxerr(o.cpu(), ref)
    _say("  O max_abs_err=%.3e" % e)
    assert e <= TOL_O[c["dt"]]


def test_eight_wave_noncausal_key_padding(gpu):
    """B * H * (n / 256) >= 1024 selects the eight-wave workgroups; key
    lengths end mid-block, so the last block of each walk is masked."""
    B, H, n, d = 2, 8, 16384, 128
    q, k, v, kl = inputs.draw(B, H, n, n, d, d, "bf16", seed=77, lens=(9001, 16383),
                              value_scale=0.5)
    _say("eight-wave non-causal, key_lens %s" % list(kl))
    o = mha.forward(q.to(DEV), k.to(DEV), v.to(DEV), key_lens=_dev(kl))
    torch.cuda.synchronize()
    o = o.cpu()
    rng = np.random.Generator(np.random.PCG64(78))
    rows = [[b, t, i] for b in range(B) for t in range(H)
            for i in sorted(set([0, 255, 256, n - 1]) | set(rng.integers(0, n, 24).tolist()))]
    rows = np.array(rows, np.int64)
    ref = oracle.attention_rows(q, k, v, rows, key_lens=kl)
    got = o[rows[:, 0], rows[:, 1], rows[:, 2]]
    e = _maxerr(got, ref)
    _say("  %d rows: O max_abs_err=%.3e" % (len(rows), e))
    assert torch.isfinite(o.float()).all()
    assert e <= TOL_O["bf16"]


# --- a sweep over the launch variants -------------------------------------------
#
# The small sweep above runs the four-wave workgroups almost everywhere.  These
# cases draw larger shapes so that each lands on a chosen variant of the
# forward kernel, as the launcher's rule picks it: (0) four-wave workgroups on
# walks of 1000-3000 keys, fp32 at times, (1) eight-wave workgroups (at least
# 1024 of 256 rows and an average walk of 48 blocks or more), (2) two key
# groups (at most 256 workgroups of 128 rows and m >= 1024).  The 18 cases
# take every variant with every mask mode, with and without ALiBi; grouped K/V
# heads and key lengths are drawn as above.  The eight-wave cases
# also write outputs larger than the L2s hold, the others smaller ones, so both
# result-store policies run.  Each case compares sampled rows (block edges, the
# last row, random ones) of O and the log-sum-exp with the oracle.

VARIANT_TAG = {0: ", 4, 1, ", 1: ", 8, 1, ", 2: ", 8, 2, "}


def _cdiv(a, b):
    return -(-a // b)


def _vcase(i):
    """Shape and options of variant-sweep case i (a pure function of i)."""
    rng = np.random.Generator(np.random.PCG64(50_000 + i))
    kind = i % 3
    mode = MODES[(i // 3) % 3]
    alibi = i >= 9
    dt = "bf16"
    Hkv = int(rng.choice([1, 2, 4]))
    g = int(rng.choice([1, 2, 4, 8]))
    if kind == 0:
        dt = "f32" if rng.random() < 0.5 else "bf16"
        d = int(rng.choice([64, 128]))
        n = int(rng.integers(1000, 3001))
        m = n if mode == "top_left" else int(rng.integers(max(n, 1000) if mode else 1000, 3001))
        c = _cdiv(n, 128)
        H = Hkv * g
        # 256 < ceil(n/128) * B * H < 1024: neither two key groups nor 8 waves.
        lo = max(1, _cdiv(257, c * H))
        B = int(rng.integers(lo, max(lo, 1023 // (c * H)) + 1))
    elif kind == 1:
        d = 128
        if mode is False:
            n, m, g = int(rng.integers(1025, 1401)), int(rng.integers(3072, 4601)), 8
        elif mode == "top_left":
            n = m = int(rng.integers(5888, 7201))
            g = max(g, 2)
        else:
            n, g = int(rng.integers(769, 2001)), 8
            m = n // 2 + int(rng.integers(2944, 4201))
        H = Hkv * g
        B = _cdiv(1024, _cdiv(n, 256) * H)
    else:
        d = int(rng.choice([64, 128]))
        if mode == "top_left":
            n = m = int(rng.integers(1024, 3001))
        else:
            m = int(rng.integers(1024, 5001))
            n = min(int(rng.integers(1, 701)), m)
        cap = 256 // _cdiv(n, 128)
        while Hkv * g > cap:
            if g > 1:
                g //= 2
            else:
                Hkv //= 2
        H = Hkv * g
        B = int(rng.integers(1, min(cap // H, max(1, 24_000_000 // (Hkv * m * d))) + 1))
    lens = None
    if rng.random() < 0.5:
        lens = (int(rng.integers(0, m + 1)) if rng.random() < 0.2 else int(rng.integers(m // 2, m + 1)), m)
    return dict(kind=kind, B=B, H=H, Hkv=Hkv, n=n, m=m, d=d, dt=dt, mode=mode, alibi=alibi,
                lens=lens, seed=60_000 + i)


def _vrows(c, rng):
    """Sampled (b, t, i): the first and last head, random heads, and in each the
    rows at workgroup and wave edges, the last row and random rows."""
    B, H, n = c["B"], c["H"], c["n"]
    heads = {(0, 0), (B - 1, H - 1)} | {(int(rng.integers(0, B)), int(rng.integers(0, H)))
                                        for _ in range(6)}
    edges = {0, 1, 31, 32, 63, 64, 127, 128, 255, 256, n - 2, n - 1}
    rows = []
    for b, t in sorted(heads):
        ii = {i for i in edges if 0 <= i < n} | set(rng.integers(0, n, 6).tolist())
        rows += [[b, t, i] for i in sorted(ii)]
    return np.array(rows, np.int64)


@pytest.mark.parametrize("i", range(18))
def test_variant_sweep(gpu, i):
    c = _vcase(i)
    code = mha.MHA_BF16 if c["dt"] == "bf16" else mha.MHA_F32
    name = mha.load().mha_forward_kernel_name(c["B"], c["H"], c["Hkv"], c["n"], c["m"], c["d"],
                                              code, mha.mask_mode(c["mode"]),
                                              int(c["alibi"])).decode()
    _say("variant sweep case %d: %s -> %s" % (i, c, name))
    assert VARIANT_TAG[c["kind"]] in name
    q, k, v, kl, sl = _draw(c)
    o, lse = mha.forward_ex(q.to(DEV), k.to(DEV), v.to(DEV), key_lens=_dev(kl),
                            causal=c["mode"], alibi_slopes=_dev(sl), return_lse=True)
    rows = _vrows(c, np.random.Generator(np.random.PCG64(70_000 + i)))
    ri = torch.as_tensor(rows, device=DEV)
    got_o = o[ri[:, 0], ri[:, 1], ri[:, 2]].cpu()
    got_lse = lse[ri[:, 0], ri[:, 1], ri[:, 2]].cpu()
    finite = bool(torch.isfinite(o.float()).all())
    torch.cuda.synchronize()
    ref_o, ref_lse = oracle.attention_ex_rows(q, k, v, rows, key_lens=kl, causal=c["mode"],
                                              alibi_slopes=sl)
    eo, el = _maxerr(got_o, ref_o), _maxerr(got_lse, ref_lse)
    _say("  %d rows: O max_abs_err=%.3e  lse max_abs_err=%.3e" % (len(rows), eo, el))
    assert finite
    assert np.array_equal(np.isneginf(oracle.to_f64(got_lse)), np.isneginf(ref_lse))
    assert eo <= TOL_O[c["dt"]]
    assert el <= TOL_LSE[c["dt"]]
