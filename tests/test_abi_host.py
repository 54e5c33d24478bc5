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
                          "mha_forward"}
    for n in names:
        assert hasattr(lib, n), n
    assert lib.mha_abi_version() == 1


def test_status_strings(lib):
    seen = set()
    for s in range(9):
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


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(mha, "_lib", None)
    monkeypatch.setattr(mha, "LIB_PATH", str(tmp_path / "absent.so"))
    with pytest.raises(RuntimeError, match="not built"):
        mha.load()
