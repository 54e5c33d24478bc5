"""GPU parity with every tensor at an odd multiple of its required alignment.

The C ABI asks for 16-byte aligned Q, K, V, O, A and decode workspace, and
4-byte aligned log-sum-exp, slopes and length arrays.  Here each tensor
starts exactly that far past a 256-byte boundary (16 + 32 j bytes, or 4 + 8 j),
inside a buffer of its own whose guard bands on both sides, and every input
byte, the calls must leave as they were; outputs start out as NaN, so an
element the kernels do not write fails the comparison with the oracle.  The
calls go through the C ABI directly (the Python binding allocates its own
outputs).  Bars as in the other parity tests.
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import transformer_head_scaled_fwd_amd as mha
from test_parity_ex_gpu import TOL_A, TOL_LSE, TOL_O, draw, maxerr
from transformer_head_scaled_fwd_amd import inputs

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
GUARD = 4096


def _say(msg):
    print(msg, flush=True)


class Placed:
    """A tensor's bytes at byte offset `off` of a buffer of its own, with
    GUARD bytes of pattern after it (and `off` bytes before)."""

    def __init__(self, t, off, fill=0xA5):
        t = t.contiguous()
        self.nbytes = t.numel() * t.element_size()
        self.off = off
        self.buf = torch.full((off + self.nbytes + GUARD,), fill, dtype=torch.uint8, device=DEV)
        self.view = self.buf[off:off + self.nbytes].view(t.dtype).view(t.shape)
        self.view.copy_(t.to(DEV))
        assert self.view.data_ptr() % 256 == off % 256
        self.before = self.buf.clone()

    @classmethod
    def output(cls, shape, dtype, off):
        # NaN everywhere: an element the call leaves unwritten fails the comparison
        return cls(torch.full(shape, float("nan"), dtype=dtype), off, fill=0x5A)

    def ptr(self):
        return self.view.data_ptr()

    def guards_intact(self):
        b = self.buf.cpu()
        a = self.before.cpu()
        return bool(torch.equal(b[:self.off], a[:self.off]) and
                    torch.equal(b[self.off + self.nbytes:], a[self.off + self.nbytes:]))

    def unchanged(self):
        return bool(torch.equal(self.buf, self.before))


def _code(dt):
    return mha.MHA_BF16 if dt == "bf16" else mha.MHA_F32


@pytest.mark.parametrize("B,H,Hkv,n,m,d,dt,causal,alibi,lens", [
    (2, 4, 2, 150, 300, 128, "bf16", "bottom_right", True, (120, 300)),
    (2, 2, 2, 130, 130, 64, "f32", "top_left", False, (1, 130)),
    (1, 4, 1, 70, 260, 64, "bf16", False, True, None),
])
def test_forward_ex_and_weights_at_odd_offsets(gpu, B, H, Hkv, n, m, d, dt, causal, alibi, lens):
    _say("odd offsets: forward_ex + weights B=%d H=%d Hkv=%d n=%d m=%d d=%d %s %s alibi=%s"
         % (B, H, Hkv, n, m, d, dt, causal, alibi))
    q, k, v, kl = draw(B, H, Hkv, n, m, d, dt, seed=91, lens=lens)
    sl = inputs.alibi_slopes(H) if alibi else None
    tdt = q.dtype
    Q, K, V = Placed(q, 16), Placed(k, 48), Placed(v, 80)
    KL = None if kl is None else Placed(torch.from_numpy(kl), 4)
    SL = None if sl is None else Placed(torch.from_numpy(np.ascontiguousarray(sl, np.float32)), 12)
    O = Placed.output((B, H, n, d), tdt, 112)
    LSE = Placed.output((B, H, n), torch.float32, 20)
    A = Placed.output((B, H, n, m), tdt, 144)
    lib = mha.load()
    mode = mha.mask_mode(causal)
    sc = mha.default_scale(d)
    stream = torch.cuda.current_stream().cuda_stream
    st = lib.mha_forward_ex(Q.ptr(), K.ptr(), V.ptr(), None if KL is None else KL.ptr(), mode,
                            None if SL is None else SL.ptr(), sc, O.ptr(), LSE.ptr(),
                            B, H, Hkv, n, m, d, d, _code(dt), stream)
    assert st == 0, mha.status_string(st)
    st = lib.mha_attention_weights(Q.ptr(), K.ptr(), None if KL is None else KL.ptr(), mode,
                                   None if SL is None else SL.ptr(), sc, LSE.ptr(), A.ptr(),
                                   B, H, Hkv, n, m, d, _code(dt), stream)
    assert st == 0, mha.status_string(st)
    torch.cuda.synchronize()
    for t in (Q, K, V, KL, SL):
        if t is not None:
            assert t.unchanged()
    for t in (O, LSE, A):
        assert t.guards_intact()
    o_ref, lse_ref, _, a_ref = oracle.attention_ex(q, k, v, key_lens=kl, causal=causal,
                                                   alibi_slopes=sl, return_lse=True,
                                                   return_weights=True)
    assert maxerr(O.view.cpu(), o_ref, "O") <= TOL_O[dt]
    assert np.array_equal(np.isneginf(oracle.to_f64(LSE.view.cpu())), np.isneginf(lse_ref))
    assert maxerr(LSE.view.cpu(), lse_ref, "lse") <= TOL_LSE[dt]
    assert maxerr(A.view.cpu(), a_ref, "A") <= TOL_A[dt]


@pytest.mark.parametrize("B,H,Hkv,n,m,d,dt,alibi,lens", [
    (2, 8, 2, 1, 3000, 128, "bf16", False, (1000, 3000)),   # split: workspace in use
    (1, 4, 4, 2, 500, 64, "f32", True, None),
])
def test_decode_at_odd_offsets(gpu, B, H, Hkv, n, m, d, dt, alibi, lens):
    _say("odd offsets: decode B=%d H=%d Hkv=%d n=%d m=%d d=%d %s alibi=%s"
         % (B, H, Hkv, n, m, d, dt, alibi))
    q, k, v, kl = draw(B, H, Hkv, n, m, d, dt, seed=93, lens=lens)
    sl = inputs.alibi_slopes(H) if alibi else None
    Q, K, V = Placed(q, 16), Placed(k, 48), Placed(v, 80)
    KL = None if kl is None else Placed(torch.from_numpy(kl), 4)
    SL = None if sl is None else Placed(torch.from_numpy(np.ascontiguousarray(sl, np.float32)), 12)
    O = Placed.output((B, H, n, d), q.dtype, 112)
    LSE = Placed.output((B, H, n), torch.float32, 20)
    need = mha.decode_workspace_size(B, H, Hkv, n, m, d, _code(dt))
    WS = Placed(torch.zeros(max(need, 16), dtype=torch.uint8), 16)
    lib = mha.load()
    st = lib.mha_decode(Q.ptr(), K.ptr(), V.ptr(), None if KL is None else KL.ptr(),
                        None if SL is None else SL.ptr(), mha.default_scale(d), O.ptr(),
                        LSE.ptr(), WS.ptr(), ctypes.c_int64(WS.nbytes), B, H, Hkv, n, m, d, d,
                        _code(dt), torch.cuda.current_stream().cuda_stream)
    assert st == 0, mha.status_string(st)
    torch.cuda.synchronize()
    for t in (Q, K, V, KL, SL):
        if t is not None:
            assert t.unchanged()
    for t in (O, LSE, WS):
        assert t.guards_intact()
    o_ref, lse_ref = oracle.attention_ex(q, k, v, key_lens=kl, causal="bottom_right",
                                         alibi_slopes=sl, return_lse=True)
    assert maxerr(O.view.cpu(), o_ref, "O") <= TOL_O[dt]
    assert maxerr(LSE.view.cpu(), lse_ref, "lse") <= TOL_LSE[dt]


@pytest.mark.parametrize("B,n,m,dm,H,dt,causal,lens", [
    (2, 100, 140, 512, 8, "bf16", False, (60, 140)),
    (2, 70, 70, 256, 2, "f32", "top_left", (30, 70)),
])
def test_multihead_at_odd_offsets(gpu, B, n, m, dm, H, dt, causal, lens):
    """The layer: X, W, Y, A and the workspace 16 bytes past a 256-byte
    boundary, each bias one element past one (its required alignment)."""
    from test_multihead_gpu import layer_inputs, ref, tol_y
    _say("odd offsets: multihead B=%d n=%d m=%d d_model=%d H=%d %s %s"
         % (B, n, m, dm, H, dt, causal))
    xq, xk, xv, Ws, bs = layer_inputs(B, n, m, dm, dt, seed=95)
    rng = np.random.Generator(np.random.PCG64(96))
    kl = rng.integers(lens[0], lens[1] + 1, size=B).astype(np.int32)
    es = xq.element_size()
    X = [Placed(t, 16 + 32 * i) for i, t in enumerate((xq, xk, xv))]
    W = [Placed(t, 16 + 32 * i) for i, t in enumerate(Ws)]
    Bi = [Placed(t, es * (2 * i + 1)) for i, t in enumerate(bs)]
    KL = Placed(torch.from_numpy(kl), 4)
    Y = Placed.output((B, n, dm), xq.dtype, 176)
    A = Placed.output((B, H, n, m), xq.dtype, 208)
    need = mha.multihead_workspace_size(B, n, m, dm, H, _code(dt), True)
    WS = Placed(torch.zeros(max(need, 16), dtype=torch.uint8), 16)
    lib = mha.load()
    st = lib.mha_multihead_forward(
        X[0].ptr(), X[1].ptr(), X[2].ptr(), W[0].ptr(), Bi[0].ptr(), W[1].ptr(), Bi[1].ptr(),
        W[2].ptr(), Bi[2].ptr(), W[3].ptr(), Bi[3].ptr(), KL.ptr(), mha.mask_mode(causal),
        mha.default_scale(dm // H), Y.ptr(), A.ptr(), WS.ptr(), WS.nbytes, B, n, m, dm, H,
        _code(dt), torch.cuda.current_stream().cuda_stream)
    assert st == 0, mha.status_string(st)
    torch.cuda.synchronize()
    for t in X + W + Bi + [KL]:
        assert t.unchanged()
    for t in (Y, A, WS):
        assert t.guards_intact()
    y_ref, a_ref = ref(xq, xk, xv, Ws, bs, H, kl, causal, weights=True)
    err = np.abs(oracle.to_f64(Y.view.cpu()) - y_ref).max()
    _say("  Y max_abs_err=%.3e" % err)
    assert err <= tol_y(dt, y_ref)
    assert maxerr(A.view.cpu(), a_ref, "A") <= TOL_A[dt]
