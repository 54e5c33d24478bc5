"""The C ABI on the host: the library loads, exports what include/libmha.h
declares, and the argument check returns each documented status before any
HIP call.  No GPU and no kernel launch are involved: every mha_forward call
here carries an argument error, which is rejected on the host."""
import ctypes
import math

import pytest

import transformer_head_scaled_fwd_amd as mha

OK, NULL, SHAPE, DTYPE, UNSUP, SCALE, ALIAS, HIP, ALIGN = range(9)
F32, BF16 = 0, 1


@pytest.fixture(scope="module")
def lib():
    return mha.load()


def test_exports_every_declared_function(lib):
    names = mha.header_functions()
    assert set(names) == {"mha_abi_version", "mha_status_string", "mha_validate",
                          "mha_forward", "mha_validate_ex", "mha_forward_ex",
                          "mha_validate_weights", "mha_attention_weights",
                          "mha_decode_workspace_size", "mha_validate_decode", "mha_decode",
                          "mha_multihead_workspace_size", "mha_multihead_forward",
                          "mha_forward_kernel_name", "mha_validate_multihead",
                          "mha_decode_noalloc"}
    for n in names:
        assert hasattr(lib, n), n
    assert lib.mha_abi_version() == 5


def test_status_strings(lib):
    seen = set()
    for s in range(11):
        txt = lib.mha_status_string(s).decode()
        assert txt and txt not in seen
        seen.add(txt)
    assert lib.mha_status_string(99).decode() == "unknown status"


# Fake, 16-byte aligned, non-overlapping device addresses: mha_validate only
# compares them, it never dereferences them.
Q, K, V, O, KL = 0x10000000, 0x20000000, 0x30000000, 0x40000000, 0x50000000


def val(lib, q=Q, k=K, v=V, kl=None, causal=0, scale=0.125, o=O,
        B=2, H=8, n=128, m=128, dk=64, dv=64, dtype=BF16):
    return lib.mha_validate(q, k, v, kl, causal, scale, o, B, H, n, m, dk, dv, dtype)


def test_valid_arguments(lib):
    assert val(lib) == OK
    assert val(lib, kl=KL, causal=1) == OK
    assert val(lib, n=77, m=1000, dk=128, dv=128, dtype=F32) == OK
    assert val(lib, B=0, q=None, k=None, v=None, o=None) == OK   # nothing to touch
    assert val(lib, m=0, k=None, v=None) == OK                    # zero keys


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), NULL), (dict(k=None), NULL), (dict(v=None), NULL), (dict(o=None), NULL),
    (dict(B=-1), SHAPE), (dict(n=-3), SHAPE), (dict(causal=1, m=129), SHAPE),
    (dict(dtype=2), DTYPE), (dict(dtype=-1), DTYPE),
    (dict(dk=96, dv=96), UNSUP), (dict(dk=64, dv=128), UNSUP), (dict(dk=256, dv=256), UNSUP),
    (dict(n=1 << 24, m=1 << 24), UNSUP),
    (dict(scale=0.0), SCALE), (dict(scale=-1.0), SCALE), (dict(scale=math.inf), SCALE),
    (dict(scale=math.nan), SCALE),
    (dict(o=Q + 64), ALIAS), (dict(o=K), ALIAS), (dict(o=V + 128), ALIAS),
    (dict(kl=O + 16), ALIAS),
    (dict(q=Q + 8), ALIGN), (dict(o=O + 2), ALIGN),
])
def test_each_error_status(lib, kw, status):
    assert val(lib, **kw) == status


# Far-apart fake addresses for tensors near the size limits.
BIG = dict(q=1 << 40, k=2 << 40, v=3 << 40, o=4 << 40)


def test_size_limits(lib):
    # A head's tensor must stay under 2 GiB (32-bit buffer offsets): for
    # bf16 rows of 128 elements that is n, m <= 2^23 - 1.
    lim = (1 << 23) - 1
    assert val(lib, n=lim, m=64, dk=128, dv=128, **BIG) == OK
    assert val(lib, n=lim + 1, m=64, dk=128, dv=128, **BIG) == UNSUP
    assert val(lib, n=64, m=lim, dk=128, dv=128, **BIG) == OK
    assert val(lib, n=64, m=lim + 1, dk=128, dv=128, **BIG) == UNSUP
    assert val(lib, n=(1 << 22) - 1, m=64, dk=128, dv=128, dtype=F32, **BIG) == OK
    assert val(lib, n=1 << 22, m=64, dk=128, dv=128, dtype=F32, **BIG) == UNSUP


def test_grid_limit(lib):
    # The dispatch grid counts work-items in 32 bits: 256 per 128 query rows.
    full = (1 << 32) // 256          # workgroups that would reach 2^32 work-items
    assert val(lib, B=full // 256 - 1, H=256, n=128, m=16, **BIG) == OK
    assert val(lib, B=full // 256, H=256, n=128, m=16, **BIG) == UNSUP
    assert val(lib, B=1, H=1, n=(1 << 22) - 1, m=16, dk=64, dv=64, **BIG) == OK


def test_huge_sizes_are_rejected_not_wrapped(lib):
    for kw in (dict(n=1 << 62), dict(m=1 << 62), dict(B=1 << 40), dict(H=1 << 40),
               dict(B=1 << 31, H=1 << 31)):
        assert val(lib, **dict(BIG, **kw)) == UNSUP, kw


def test_empty_query_axis_with_huge_batch_is_ok(lib):
    # With n = 0 there is nothing to compute and no grid to bound B * H; the
    # byte extents of K and V (B * H * m * d elements) exceed 64 bits and
    # must saturate in the check rather than wrap.
    huge = dict(B=(1 << 31) - 1, H=(1 << 31) - 1, n=0, m=(1 << 23) - 1, dk=128, dv=128)
    assert val(lib, **dict(BIG, **huge)) == OK
    assert val_ex(lib, **dict(BIG, lse=5 << 40, kl=6 << 40, Hkv=huge["H"], **huge)) == OK
    assert val_w(lib, q=1 << 40, k=2 << 40, lse=5 << 40, a=4 << 40, kl=6 << 40,
                 B=huge["B"], H=huge["H"], Hkv=huge["H"], n=0, m=huge["m"], dk=128) == OK
    # and the same batch with one query row is refused by the grid bound
    assert val(lib, **dict(BIG, **dict(huge, n=1))) == UNSUP


def test_q_k_v_may_alias_each_other(lib):
    assert val(lib, k=Q, v=Q) == OK


def test_forward_rejects_on_host_before_any_launch(lib):
    # Argument errors come back from mha_forward itself, without a device.
    st = lib.mha_forward(Q, K, V, None, 1, 0.125, O, 1, 1, 8, 9, 64, 64, BF16, None)
    assert st == SHAPE
    st = lib.mha_forward(Q, K, V, None, 0, -1.0, O, 1, 1, 8, 8, 64, 64, BF16, None)
    assert st == SCALE
    st = lib.mha_forward(Q, K, V, None, 0, 0.125, Q, 1, 1, 8, 8, 64, 64, BF16, None)
    assert st == ALIAS


def test_forward_with_nothing_to_do_returns_ok_without_launch(lib):
    assert lib.mha_forward(None, None, None, None, 0, 0.125, None, 0, 8, 16, 16, 64, 64,
                           BF16, None) == OK
    assert lib.mha_forward(Q, K, V, None, 0, 0.125, None, 2, 8, 0, 16, 64, 64,
                           BF16, None) == OK


def test_binding_validate_uses_library_check():
    import torch
    q = torch.zeros(1, 2, 16, 64, dtype=torch.bfloat16)
    k = torch.zeros(1, 2, 17, 64, dtype=torch.bfloat16)
    out = torch.zeros(1, 2, 16, 64, dtype=torch.bfloat16)
    assert mha.validate(q, k, k, out=out) == OK
    assert mha.validate(q, k, k, causal=True, out=out) == SHAPE
    assert mha.validate(q, k, k, out=q) == ALIAS
    with pytest.raises(TypeError):
        mha.validate(q.half(), k.half(), k.half(), out=out)


def test_forward_refuses_cpu_tensors():
    import torch
    q = torch.zeros(1, 1, 8, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        mha.forward(q, q, q)


def test_multihead_refuses_cpu_tensors():
    import torch
    x = torch.zeros(1, 8, 64, dtype=torch.bfloat16)
    W = torch.zeros(64, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        mha.multihead_forward(x, x, x, W, None, W, None, W, None, W, None, 1)


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(mha, "_lib", None)
    monkeypatch.setattr(mha, "LIB_PATH", str(tmp_path / "absent.so"))
    with pytest.raises(RuntimeError, match="not built"):
        mha.load()


# --- extended forward and weights ------------------------------------------------

LSE, SL, A = 0x60000000, 0x70000000, 0x80000000
MODE = 9


def val_ex(lib, q=Q, k=K, v=V, kl=None, mode=0, sl=None, scale=0.125, o=O, lse=None,
           B=2, H=8, Hkv=8, n=128, m=128, dk=64, dv=64, dtype=BF16):
    return lib.mha_validate_ex(q, k, v, kl, mode, sl, scale, o, lse, B, H, Hkv, n, m, dk, dv,
                               dtype)


def val_w(lib, q=Q, k=K, kl=None, mode=0, sl=None, scale=0.125, lse=LSE, a=A,
          B=2, H=8, Hkv=8, n=128, m=128, dk=64, dtype=BF16):
    return lib.mha_validate_weights(q, k, kl, mode, sl, scale, lse, a, B, H, Hkv, n, m, dk,
                                    dtype)


def test_valid_extended_arguments(lib):
    assert val_ex(lib) == OK
    assert val_ex(lib, Hkv=1, mode=2, n=1, m=4096, sl=SL, lse=LSE, kl=KL) == OK
    assert val_ex(lib, Hkv=2, mode=1, n=100, m=300) == OK   # top-left accepts n != m here
    assert val_ex(lib, m=0, k=None, v=None, lse=LSE) == OK
    assert val_w(lib) == OK
    assert val_w(lib, Hkv=4, mode=2, n=3, m=1000, sl=SL, kl=KL) == OK
    assert val_w(lib, m=0, k=None, a=None) == OK


@pytest.mark.parametrize("kw,status", [
    (dict(Hkv=3), SHAPE), (dict(Hkv=0), SHAPE), (dict(Hkv=-1), SHAPE), (dict(Hkv=16), SHAPE),
    (dict(mode=3), MODE), (dict(mode=-1), MODE),
    (dict(lse=O + 64), ALIAS), (dict(lse=Q), ALIAS), (dict(lse=KL, kl=KL), ALIAS),
    (dict(sl=O), ALIAS), (dict(sl=LSE, lse=LSE), ALIAS),
    (dict(lse=LSE + 2), ALIGN), (dict(sl=SL + 1), ALIGN),
    (dict(scale=0.0), SCALE), (dict(dk=96, dv=96), UNSUP), (dict(k=None), NULL),
])
def test_each_extended_error_status(lib, kw, status):
    assert val_ex(lib, **kw) == status


@pytest.mark.parametrize("kw,status", [
    (dict(Hkv=3), SHAPE), (dict(mode=5), MODE), (dict(lse=None), NULL), (dict(a=None), NULL),
    (dict(a=Q), ALIAS), (dict(a=LSE - 64), ALIAS), (dict(a=K + 16), ALIAS),
    (dict(a=A + 8), ALIGN), (dict(lse=LSE + 1), ALIGN),
    (dict(n=1 << 16, m=1 << 16), UNSUP), (dict(dtype=7), DTYPE),
])
def test_each_weights_error_status(lib, kw, status):
    assert val_w(lib, **kw) == status


def test_extended_calls_reject_on_host(lib):
    st = lib.mha_forward_ex(Q, K, V, None, 4, None, 0.125, O, None, 1, 2, 2, 8, 8, 64, 64,
                            BF16, None)
    assert st == MODE
    st = lib.mha_attention_weights(Q, K, None, 0, None, 0.125, LSE, Q, 1, 2, 2, 8, 8, 64,
                                   BF16, None)
    assert st == ALIAS
    assert lib.mha_attention_weights(Q, K, None, 0, None, 0.125, LSE, A, 1, 2, 2, 8, 0, 64,
                                     BF16, None) == OK


def test_binding_mask_modes():
    assert mha.mask_mode(False) == 0 and mha.mask_mode(True) == 1
    assert mha.mask_mode("top_left") == 1 and mha.mask_mode("bottom_right") == 2
    with pytest.raises(ValueError):
        mha.mask_mode("upper")


def test_binding_validate_ex_uses_library_check():
    import torch
    q = torch.zeros(1, 4, 16, 64, dtype=torch.bfloat16)
    k = torch.zeros(1, 2, 17, 64, dtype=torch.bfloat16)
    out = torch.zeros(1, 4, 16, 64, dtype=torch.bfloat16)
    assert mha.validate_ex(q, k, k, causal="bottom_right", out=out) == OK
    k3 = torch.zeros(1, 3, 17, 64, dtype=torch.bfloat16)
    assert mha.validate_ex(q, k3, k3, out=out) == SHAPE


# --- decode ----------------------------------------------------------------------

WSPACE = 0x90000000
WS = 10


def ws_size(B=8, H=32, Hkv=8, n=1, m=16384, d=128, dtype=BF16):
    import ctypes
    out = ctypes.c_int64(-1)
    st = mha.load().mha_decode_workspace_size(B, H, Hkv, n, m, d, dtype, ctypes.byref(out))
    return st, out.value


def test_decode_workspace_size():
    st, big = ws_size()
    assert st == OK and big > 0
    # a grid that already fills the device needs no split, hence no workspace
    st, none = ws_size(B=256, H=32, Hkv=32, m=4096)
    assert st == OK and none == 0
    assert ws_size(Hkv=3)[0] == SHAPE
    assert ws_size(d=96)[0] == UNSUP
    assert ws_size(B=0) == (OK, 0)
    # the size grows with the rows that need partial results
    assert ws_size(n=4)[1] > big


def val_dec(lib, ws=WSPACE, wsb=1 << 30, q=Q, k=K, v=V, kl=None, sl=None, o=O, lse=None,
            B=8, H=32, Hkv=8, n=1, m=16384, d=128, dtype=BF16):
    return lib.mha_validate_decode(q, k, v, kl, sl, 0.125, o, lse, ws, wsb, B, H, Hkv, n, m,
                                   d, d, dtype)


def test_decode_validation(lib):
    need = ws_size()[1]
    assert val_dec(lib, wsb=need) == OK
    assert val_dec(lib, wsb=need - 1) == WS
    assert val_dec(lib, ws=None) == WS
    assert val_dec(lib, ws=WSPACE + 8) == WS
    assert val_dec(lib, ws=O) == WS                      # overlaps the output
    assert val_dec(lib, Hkv=5) == SHAPE
    assert val_dec(lib, B=64, H=32, Hkv=32, m=512, ws=None, wsb=0) == OK
    st = lib.mha_decode(Q, K, V, None, None, 0.125, O, None, None, 0, 8, 32, 8, 1, 16384,
                        128, 128, BF16, None)
    assert st == WS


# --- multi-head layer --------------------------------------------------------------

def mh_size(B=4, n=128, m=128, dm=512, H=8, dtype=BF16, w=0):
    import ctypes
    out = ctypes.c_int64(-1)
    st = mha.load().mha_multihead_workspace_size(B, n, m, dm, H, dtype, w, ctypes.byref(out))
    return st, out.value


def test_multihead_workspace_size():
    st, b = mh_size()
    assert st == OK and b >= 4 * 4 * 128 * 512 * 2
    assert mh_size(w=1)[1] > b                       # room for the row log-sum-exp
    assert mh_size(dm=500)[0] == SHAPE               # not a multiple of H
    assert mh_size(dm=256, H=8)[0] == UNSUP          # d_k = 32
    assert mh_size(dtype=3)[0] == DTYPE


XQ, WQ, WK, WV, WO, Y_, WS_ = (0x100000000 + i * 0x10000000 for i in range(7))


def mh_call(lib, ws=WS_, wsb=1 << 27, y=Y_, a=None, mode=0, scale=0.125, B=4, n=128, m=128,
            dm=512, H=8):
    return lib.mha_multihead_forward(XQ, XQ, XQ, WQ, None, WK, None, WV, None, WO, None, None,
                                     mode, scale, y, a, ws, wsb, B, n, m, dm, H, BF16, None)


def test_multihead_rejects_on_host(lib):
    need = mh_size()[1]
    assert mh_call(lib, wsb=need - 1) == WS
    assert mh_call(lib, ws=None) == WS
    assert mh_call(lib, ws=WQ) == WS                 # workspace over a weight
    assert mh_call(lib, y=XQ) == ALIAS               # output over the input
    assert mh_call(lib, y=Y_ + 4) == ALIGN
    assert mh_call(lib, mode=7) == MODE
    assert mh_call(lib, scale=-1.0) == SCALE
    assert mh_call(lib, H=5) == SHAPE
    assert mh_call(lib, B=0) == OK                   # nothing to do


def test_forward_kernel_name_follows_the_variant_rule(lib):
    """The instance a launch of these sizes takes, spelled as profilers print
    it; None for arguments the forward pass refuses."""
    def name(B, H, Hkv, n, m, d, dtype=BF16, mode=0, alibi=0):
        r = lib.mha_forward_kernel_name(B, H, Hkv, n, m, d, dtype, mode, alibi)
        return None if r is None else r.decode()
    # the long causal workload: 64 query blocks of 256 rows x 16 heads
    assert name(1, 16, 16, 16384, 16384, 128, mode=1) == \
        "mha::attn_fwd_kernel<__bf16, 128, 8, 1, true, false>"
    # long causal walks at d = 128 keep eight waves; shorter ones take four
    assert name(2, 16, 16, 8192, 8192, 128, mode=1).endswith("<__bf16, 128, 8, 1, true, false>")
    assert name(4, 16, 16, 4096, 4096, 128, mode=1).endswith("<__bf16, 128, 4, 1, true, false>")
    assert name(4, 16, 16, 4096, 4096, 128, mode=0).endswith("<__bf16, 128, 8, 1, false, false>")
    assert name(8, 8, 8, 2048, 2048, 128, mode=0).endswith("<__bf16, 128, 4, 1, false, false>")
    # n = 128, d = 64: four-wave workgroups; one per 128 rows
    assert name(32, 8, 8, 128, 128, 64) == "mha::attn_fwd_kernel<__bf16, 64, 4, 1, false, false>"
    # few query blocks and a long key axis: two key groups
    assert name(8, 16, 16, 256, 1024, 64) == "mha::attn_fwd_kernel<__bf16, 64, 8, 2, false, false>"
    assert name(1, 8, 8, 16, 16, 64, dtype=F32) == \
        "mha::attn_fwd_kernel<float, 64, 4, 1, false, false>"
    assert name(2, 8, 2, 4096, 4096, 128, mode=2, alibi=1).endswith("true, true>")
    assert name(1, 8, 8, 16, 16, 96) is None
    assert name(1, 8, 3, 16, 16, 64) is None
    assert name(1, 8, 8, 16, 16, 64, dtype=7) is None
    assert name(1, 8, 8, 16, 16, 64, mode=3) is None


def test_decode_noalloc_rejects_on_host(lib):
    # Argument errors come back before any HIP call (no device here).
    st = lib.mha_decode_noalloc(Q, K, V, None, None, 0.125, O, None, 8, 32, 5, 1, 16384,
                                128, 128, BF16, None)
    assert st == SHAPE
    st = lib.mha_decode_noalloc(Q, K, V, None, None, 0.125, Q, None, 8, 32, 8, 1, 16384,
                                128, 128, BF16, None)
    assert st == ALIAS
    st = lib.mha_decode_noalloc(Q, K, V, None, None, 0.125, O, None, 8, 32, 8, 1, 16384,
                                96, 96, BF16, None)
    assert st == UNSUP
    assert lib.mha_decode_noalloc(None, None, None, None, None, 0.125, None, None, 0, 32, 8, 1,
                                  16384, 128, 128, BF16, None) == OK
