"""GPU parity of mha_multihead_forward (projections, head split, core,
concat, output projection) against the fp64 multi-head oracle.

The oracle keeps every intermediate in fp64; the library stores Q, K, V, O
and Y in the input dtype, each store a rounding of relative size at most
u = 2^-9 (bf16) or 2^-24 (fp32), and rounds the weights P inside the core
the same way.  With five storage roundings and the rounded P, each adding
at most about one u of the output's scale after the projections, the bar
is 8u * max|Y| for bf16 (2^-6 of the output scale); for fp32 it is the core's
1e-5 at unit scale.  Weights A use the core's bars (5e-3 bf16, 2e-5 fp32).
"""
import numpy as np
import pytest
import torch

import oracle
import transformer_head_scaled_fwd_amd as mha
from transformer_head_scaled_fwd_amd import inputs

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TDT = {"bf16": torch.bfloat16, "f32": torch.float32}


def _say(msg):
    print(msg, flush=True)


def layer_inputs(B, n, m, dm, dt, seed, bias=True, self_attn=False):
    """X ~ N(0, 1); weights and biases ~ U(-1/sqrt(dm), 1/sqrt(dm)) (the
    nn.Linear initialisation range), rounded to the dtype."""
    rng = np.random.Generator(np.random.PCG64(seed))
    rnd = lambda a: torch.from_numpy(a.astype(np.float32)).to(TDT[dt])  # noqa: E731
    xq = rnd(rng.standard_normal((B, n, dm)))
    xk = xq if self_attn else rnd(rng.standard_normal((B, m, dm)))
    xv = xq if self_attn else rnd(rng.standard_normal((B, m, dm)))
    bound = 1.0 / np.sqrt(dm)
    Ws = [rnd(rng.uniform(-bound, bound, (dm, dm))) for _ in range(4)]
    bs = [rnd(rng.uniform(-bound, bound, dm)) if bias else None for _ in range(4)]
    return xq, xk, xv, Ws, bs


def run(xq, xk, xv, Ws, bs, H, kl, causal, weights=False):
    d = lambda t: None if t is None else t.to(DEV)  # noqa: E731
    res = mha.multihead_forward(d(xq), d(xk), d(xv), d(Ws[0]), d(bs[0]), d(Ws[1]), d(bs[1]),
                                d(Ws[2]), d(bs[2]), d(Ws[3]), d(bs[3]), H,
                                key_lens=None if kl is None else torch.as_tensor(kl).to(DEV),
                                causal=causal, need_weights=weights)
    torch.cuda.synchronize()
    return [r.cpu() for r in res] if weights else res.cpu()


def ref(xq, xk, xv, Ws, bs, H, kl, causal, weights=False):
    dm = xq.shape[-1]
    return oracle.multihead(xq, xk, xv, Ws[0], bs[0], Ws[1], bs[1], Ws[2], bs[2], Ws[3],
                            bs[3], H, key_lens=kl, causal=causal,
                            scale=mha.default_scale(dm // H), return_weights=weights)


def tol_y(dt, y_ref):
    return 2.0 ** -6 * float(np.abs(y_ref).max()) if dt == "bf16" else 1e-5


CASES = [
    # B, n, m, d_model, H, dtype, causal, lens, bias, self
    (4, 128, 128, 512, 8, "bf16", False, (16, 128), True, True),     # encoder, base model
    (2, 100, 300, 1024, 16, "bf16", False, (150, 300), True, False),  # cross-attention, big
    (2, 200, 200, 512, 4, "bf16", True, None, False, True),          # decoder, d_k = 128
    (3, 77, 77, 768, 12, "bf16", "bottom_right", (40, 77), True, True),
    (2, 70, 70, 256, 2, "f32", True, (30, 70), True, True),
    (2, 33, 65, 128, 2, "f32", False, None, True, False),
]


@pytest.mark.parametrize("B,n,m,dm,H,dt,causal,lens,bias,self_attn", CASES)
def test_multihead_parity(gpu, B, n, m, dm, H, dt, causal, lens, bias, self_attn):
    _say("multihead B=%d n=%d m=%d d_model=%d H=%d %s causal=%s lens=%s bias=%s self=%s"
         % (B, n, m, dm, H, dt, causal, lens, bias, self_attn))
    xq, xk, xv, Ws, bs = layer_inputs(B, n, m, dm, dt, seed=n + m + dm + H, bias=bias,
                                      self_attn=self_attn)
    kl = None
    if lens is not None:
        kl = np.random.Generator(np.random.PCG64(7)).integers(lens[0], lens[1] + 1,
                                                              size=B).astype(np.int32)
    y = run(xq, xk, xv, Ws, bs, H, kl, causal)
    y_ref = ref(xq, xk, xv, Ws, bs, H, kl, causal)
    err = np.abs(oracle.to_f64(y) - y_ref)
    tol = tol_y(dt, y_ref)
    _say("Y max_abs_err=%.3e (tol %.3e, max|Y| %.3f)" % (err.max(), tol, np.abs(y_ref).max()))
    assert torch.isfinite(y.float()).all()
    assert err.max() <= tol


def test_multihead_weights(gpu):
    B, n, m, dm, H = 2, 64, 96, 512, 8
    xq, xk, xv, Ws, bs = layer_inputs(B, n, m, dm, "bf16", seed=5)
    kl = np.array([96, 50], np.int32)
    y, a = run(xq, xk, xv, Ws, bs, H, kl, False, weights=True)
    y_ref, a_ref = ref(xq, xk, xv, Ws, bs, H, kl, False, weights=True)
    assert np.abs(oracle.to_f64(y) - y_ref).max() <= tol_y("bf16", y_ref)
    ea = np.abs(oracle.to_f64(a) - a_ref).max()
    _say("A max_abs_err=%.3e" % ea)
    assert ea <= 5e-3
    assert np.all(oracle.to_f64(a)[a_ref == 0.0] == 0.0)


@pytest.mark.parametrize("name", ["mha_layer_base_n128", "mha_layer_big_n512"])
def test_multihead_workload_sampled(gpu, name):
    # The benchmarked layer workloads at full size; the oracle evaluates a
    # few whole sequences (every row of each).
    w = inputs.LAYER_WORKLOADS[name]
    _say("layer workload %s" % name)
    xq, xk, xv, Ws, bs, kl = inputs.draw_layer(w)
    y = run(xq, xk, xv, Ws, bs, w.H, kl, w.causal)
    for b in (0, w.B - 1):
        sl = slice(b, b + 1)
        y_ref = ref(xq[sl], xk[sl], xv[sl], Ws, bs, w.H, None if kl is None else kl[sl],
                    w.causal)
        err = np.abs(oracle.to_f64(y[sl]) - y_ref).max()
        _say("batch %d Y max_abs_err=%.3e" % (b, err))
        assert err <= tol_y(w.dtype, y_ref)


def test_multihead_binding_rejects_bad_out_and_workspace(gpu):
    # The library sees only addresses: an output of the wrong size or a
    # workspace in host memory must be refused by the binding, before any
    # launch.
    xq, xk, xv, Ws, bs = layer_inputs(1, 16, 16, 128, "bf16", seed=5)
    d = lambda t: None if t is None else t.to(DEV)  # noqa: E731
    args = [d(xq), d(xk), d(xv), d(Ws[0]), d(bs[0]), d(Ws[1]), d(bs[1]), d(Ws[2]), d(bs[2]),
            d(Ws[3]), d(bs[3]), 2]
    small = torch.empty((1, 8, 128), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(ValueError):
        mha.multihead_forward(*args, out=small)
    host_ws = torch.empty(1 << 20, dtype=torch.uint8)
    with pytest.raises(ValueError):
        mha.multihead_forward(*args, workspace=host_ws)
    y = mha.multihead_forward(*args)
    torch.cuda.synchronize()
    assert tuple(y.shape) == (1, 16, 128)
