"""mha_decode_noalloc, the decode entry point for callers that cannot
allocate, against mha_decode with a caller's workspace (through the C ABI).

Both run the same kernels on the same split plan, so their outputs must be
identical bit for bit; each is also checked against the oracle on sampled
rows.  Three calls in a row: the first needs the most scratch, the second
is smaller (fewer rows, more splits), the third needs none.  The
library's scratch keeps the last call's contents; no call may read them.
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import transformer_head_scaled_fwd_amd as mha
from transformer_head_scaled_fwd_amd import inputs

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TOL = 1.5e-2

CASES = [
    # B, H, H_kv, n, m, d, lens: 64 units of 32 rows over 4 splits
    (8, 32, 8, 1, 16384, 128, (8192, 16384)),
    # smaller: one sequence, 32 units over 8 splits, d = 64
    (1, 32, 32, 1, 8192, 64, None),
    # no split at all: 512 units fill the device
    (64, 8, 8, 1, 2048, 128, (1, 2048)),
]


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def test_noalloc_decode_matches_workspace_decode(gpu):
    lib = mha.load()
    needs = []
    for i, (B, H, Hkv, n, m, d, lens) in enumerate(CASES):
        print("no-alloc decode case", i, (B, H, Hkv, n, m, d, lens), flush=True)
        rng = np.random.Generator(np.random.PCG64(1500 + i))
        q = torch.from_numpy(rng.standard_normal((B, H, n, d)).astype(np.float32)).bfloat16()
        k = torch.from_numpy(rng.standard_normal((B, Hkv, m, d)).astype(np.float32)).bfloat16()
        v = torch.from_numpy(rng.standard_normal((B, Hkv, m, d)).astype(np.float32)).bfloat16()
        kl = None if lens is None else rng.integers(lens[0], lens[1] + 1, size=B).astype(np.int32)
        qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
        kld = None if kl is None else torch.as_tensor(kl).to(DEV)
        need = mha.decode_workspace_size(B, H, Hkv, n, m, d, mha.MHA_BF16)
        needs.append(need)
        ws = torch.empty(max(need, 16), dtype=torch.uint8, device=DEV)
        ws.view(torch.float32).fill_(float("nan"))
        o_ws = torch.empty_like(qd)
        o_na = torch.full_like(qd, float("nan"))
        lse_ws = torch.empty(B, H, n, dtype=torch.float32, device=DEV)
        lse_na = torch.full_like(lse_ws, float("nan"))
        scale = mha.default_scale(d)
        stream = torch.cuda.current_stream().cuda_stream
        st = lib.mha_decode(_ptr(qd), _ptr(kd), _ptr(vd), _ptr(kld), None, scale, _ptr(o_ws),
                            _ptr(lse_ws), _ptr(ws), ws.numel(), B, H, Hkv, n, m, d, d,
                            mha.MHA_BF16, stream)
        assert st == 0, mha.status_string(st)
        st = lib.mha_decode_noalloc(_ptr(qd), _ptr(kd), _ptr(vd), _ptr(kld), None, scale,
                                    _ptr(o_na), _ptr(lse_na), B, H, Hkv, n, m, d, d,
                                    mha.MHA_BF16, stream)
        assert st == 0, mha.status_string(st)
        torch.cuda.synchronize()
        assert torch.equal(o_na, o_ws) and torch.equal(lse_na, lse_ws), i
        rows = np.array([[b, t, 0] for b in range(B) for t in range(H)][::max(1, B * H // 64)],
                        np.int64)
        ref, _ = oracle.attention_ex_rows(q, k, v, rows, key_lens=kl, causal="bottom_right")
        got = oracle.to_f64(o_na.cpu()[rows[:, 0], rows[:, 1], rows[:, 2]])
        assert float(np.abs(got - ref).max()) <= TOL, i
    assert needs[0] > needs[1] > 0 and needs[2] == 0


def test_noalloc_decode_refuses_bad_arguments_on_the_host(gpu):
    lib = mha.load()
    q = torch.zeros(1, 4, 1, 64, dtype=torch.bfloat16, device=DEV)
    k = torch.zeros(1, 3, 64, 64, dtype=torch.bfloat16, device=DEV)
    st = lib.mha_decode_noalloc(_ptr(q), _ptr(k), _ptr(k), None, None, 0.125, _ptr(q), None,
                                1, 4, 3, 1, 64, 64, 64, mha.MHA_BF16, None)
    assert st == 2          # H not a multiple of H_kv
    st = lib.mha_decode_noalloc(None, None, None, None, None, 0.125, None, None,
                                0, 4, 4, 1, 64, 64, 64, mha.MHA_BF16, None)
    assert st == 0          # nothing to do
