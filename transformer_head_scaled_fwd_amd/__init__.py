"""libmha: multi-head scaled dot-product attention forward on MI355X (gfx950).

Thin Python binding over the C ABI in include/libmha.h.  This module only
marshals arguments (device pointers, sizes, the current HIP stream); every
step of the attention runs in the HIP kernels of libmha.so.  torch supplies
device memory and the stream.  There is no fallback: if libmha.so is not
built, every call raises.

    import transformer_head_scaled_fwd_amd as mha
    o = mha.forward(q, k, v, key_lens=None, causal=False, scale=None)
    o, lse, a = mha.forward_ex(q, k, v, causal="bottom_right", alibi_slopes=s,
                               return_lse=True, need_weights=True)

q [B,H,n,d], k [B,H,m,d], v [B,H,m,d] contiguous bf16 or fp32 tensors on
one GPU; key_lens an int32 tensor [B] on the same GPU (or None); scale
defaults to the fp32 value of 1/sqrt(d).
"""
from __future__ import annotations

import ctypes
import math
import os
import re

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmha.so")
HEADER_PATH = os.path.join(os.path.dirname(_PKG), "include", "libmha.h")

MHA_F32 = 0
MHA_BF16 = 1

_lib = None


class MhaError(ValueError):
    """A non-zero status from libmha; .status holds the code."""

    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


def load():
    """Load libmha.so (once).  Raises RuntimeError if it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            "libmha.so is not built (expected at %s); run "
            "`python -m transformer_head_scaled_fwd_amd.build`" % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    lib.mha_abi_version.argtypes = []
    lib.mha_abi_version.restype = i32
    lib.mha_status_string.argtypes = [i32]
    lib.mha_status_string.restype = ctypes.c_char_p
    lib.mha_validate.argtypes = [vp, vp, vp, vp, i32, ctypes.c_float, vp,
                                 i64, i64, i64, i64, i64, i64, i32]
    lib.mha_validate.restype = i32
    lib.mha_forward.argtypes = [vp, vp, vp, vp, i32, ctypes.c_float, vp,
                                i64, i64, i64, i64, i64, i64, i32, vp]
    lib.mha_forward.restype = i32
    fl = ctypes.c_float
    lib.mha_validate_ex.argtypes = [vp, vp, vp, vp, i32, vp, fl, vp, vp,
                                    i64, i64, i64, i64, i64, i64, i64, i32]
    lib.mha_validate_ex.restype = i32
    lib.mha_forward_ex.argtypes = [vp, vp, vp, vp, i32, vp, fl, vp, vp,
                                   i64, i64, i64, i64, i64, i64, i64, i32, vp]
    lib.mha_forward_ex.restype = i32
    lib.mha_validate_weights.argtypes = [vp, vp, vp, i32, vp, fl, vp, vp,
                                         i64, i64, i64, i64, i64, i64, i32]
    lib.mha_validate_weights.restype = i32
    lib.mha_attention_weights.argtypes = [vp, vp, vp, i32, vp, fl, vp, vp,
                                          i64, i64, i64, i64, i64, i64, i32, vp]
    lib.mha_attention_weights.restype = i32
    lib.mha_decode_workspace_size.argtypes = [i64, i64, i64, i64, i64, i64, i32,
                                              ctypes.POINTER(i64)]
    lib.mha_decode_workspace_size.restype = i32
    lib.mha_validate_decode.argtypes = [vp, vp, vp, vp, vp, fl, vp, vp, vp, i64,
                                        i64, i64, i64, i64, i64, i64, i64, i32]
    lib.mha_validate_decode.restype = i32
    lib.mha_decode.argtypes = [vp, vp, vp, vp, vp, fl, vp, vp, vp, i64,
                               i64, i64, i64, i64, i64, i64, i64, i32, vp]
    lib.mha_decode.restype = i32
    lib.mha_decode_noalloc.argtypes = [vp, vp, vp, vp, vp, fl, vp, vp,
                                       i64, i64, i64, i64, i64, i64, i64, i32, vp]
    lib.mha_decode_noalloc.restype = i32
    lib.mha_multihead_workspace_size.argtypes = [i64, i64, i64, i64, i64, i32, i32,
                                                 ctypes.POINTER(i64)]
    lib.mha_multihead_workspace_size.restype = i32
    lib.mha_multihead_forward.argtypes = [vp] * 11 + [vp, i32, fl, vp, vp, vp, i64,
                                                      i64, i64, i64, i64, i64, i32, vp]
    lib.mha_multihead_forward.restype = i32
    lib.mha_validate_multihead.argtypes = [vp] * 11 + [vp, i32, fl, vp, vp, vp, i64,
                                                       i64, i64, i64, i64, i64, i32]
    lib.mha_validate_multihead.restype = i32
    lib.mha_forward_kernel_name.argtypes = [i64, i64, i64, i64, i64, i64, i32, i32, i32]
    lib.mha_forward_kernel_name.restype = ctypes.c_char_p
    _lib = lib
    return lib


def header_functions():
    """Names of the functions include/libmha.h declares."""
    with open(HEADER_PATH, encoding="utf-8") as f:
        text = f.read()
    return sorted(set(re.findall(r"^\s*(?:int|mha_status|const char \*)\s*(mha_\w+)\s*\(", text, re.M)))


def abi_version() -> int:
    return int(load().mha_abi_version())


def status_string(status: int) -> str:
    return load().mha_status_string(int(status)).decode()


def _check(status: int):
    if status != 0:
        raise MhaError(status, status_string(status))


def default_scale(d: int) -> float:
    """fp32 value of 1/sqrt(d), the scale of the pages' attention."""
    import numpy as np
    return float(np.float32(1.0 / math.sqrt(d)))


def _dtype_code(t):
    import torch
    if t.dtype == torch.bfloat16:
        return MHA_BF16
    if t.dtype == torch.float32:
        return MHA_F32
    raise TypeError("libmha takes bfloat16 or float32 tensors, got %s" % t.dtype)


def validate(q, k, v, key_lens=None, causal=False, scale=None, out=None) -> int:
    """Run the library's host-side argument check only; returns the status."""
    B, H, n, dk = q.shape
    m, dv = k.shape[2], v.shape[3]
    sc = default_scale(dk) if scale is None else float(scale)
    return int(load().mha_validate(
        q.data_ptr(), k.data_ptr(), v.data_ptr(),
        None if key_lens is None else key_lens.data_ptr(), int(bool(causal)), sc,
        None if out is None else out.data_ptr(), B, H, n, m, dk, dv, _dtype_code(q)))


def forward(q, k, v, key_lens=None, causal=False, scale=None, out=None, stream=None):
    """O = softmax(scale * Q K^T + mask) V per (batch, head), on the GPU.

    Enqueued on `stream` (default: torch's current stream); returns `out`
    (allocated if not given) without synchronizing.
    """
    import torch
    lib = load()
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be 4-D [B, H, L, d]")
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k, v must share one dtype")
    code = _dtype_code(q)
    dev = q.device
    if dev.type != "cuda" or k.device != dev or v.device != dev:
        raise ValueError("q, k, v must be on the same GPU")
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not t.is_contiguous():
            raise ValueError("%s must be contiguous" % name)
    B, H, n, dk = q.shape
    m = k.shape[2]
    dv = v.shape[3]
    if k.shape[0] != B or k.shape[1] != H or k.shape[3] != dk or \
            v.shape[0] != B or v.shape[1] != H or v.shape[2] != m:
        raise ValueError("shape mismatch: q %s, k %s, v %s"
                         % (tuple(q.shape), tuple(k.shape), tuple(v.shape)))
    kl_ptr = None
    if key_lens is not None:
        if key_lens.dtype != torch.int32 or key_lens.device != dev or \
                tuple(key_lens.shape) != (B,) or not key_lens.is_contiguous():
            raise ValueError("key_lens must be a contiguous int32 tensor [B] on the GPU of q")
        kl_ptr = key_lens.data_ptr()
    if out is None:
        out = torch.empty((B, H, n, dv), dtype=q.dtype, device=dev)
    elif out.shape != (B, H, n, dv) or out.dtype != q.dtype or out.device != dev \
            or not out.is_contiguous():
        raise ValueError("out must be a contiguous [B, H, n, d_v] tensor like q")
    sc = default_scale(dk) if scale is None else float(scale)
    if stream is None:
        stream = torch.cuda.current_stream(dev).cuda_stream
    with torch.cuda.device(dev):
        st = lib.mha_forward(q.data_ptr(), k.data_ptr(), v.data_ptr(), kl_ptr,
                             int(bool(causal)), sc, out.data_ptr(),
                             B, H, n, m, dk, dv, code, stream)
    _check(st)
    return out


MHA_MASK_NONE = 0
MHA_MASK_CAUSAL = 1
MHA_MASK_CAUSAL_BOTTOM_RIGHT = 2
_MODES = {False: MHA_MASK_NONE, None: MHA_MASK_NONE, "none": MHA_MASK_NONE,
          True: MHA_MASK_CAUSAL, "top_left": MHA_MASK_CAUSAL,
          "bottom_right": MHA_MASK_CAUSAL_BOTTOM_RIGHT}


def mask_mode(causal) -> int:
    """MHA_MASK_* code of causal = False / True / 'top_left' / 'bottom_right'."""
    if causal not in _MODES:
        raise ValueError("causal must be False, True, 'top_left' or 'bottom_right'")
    return _MODES[causal]


def _device_args(q, k, v, key_lens, alibi_slopes):
    """Checks shared by the extended calls; returns (B, H, Hkv, n, m, dk, dv,
    dtype code, key_lens ptr, slopes ptr)."""
    import torch
    if q.dim() != 4 or k.dim() != 4 or (v is not None and v.dim() != 4):
        raise ValueError("q, k, v must be 4-D [B, H, L, d]")
    if q.dtype != k.dtype or (v is not None and v.dtype != q.dtype):
        raise TypeError("q, k, v must share one dtype")
    code = _dtype_code(q)
    dev = q.device
    if dev.type != "cuda" or k.device != dev or (v is not None and v.device != dev):
        raise ValueError("q, k, v must be on the same GPU")
    for name, t in (("q", q), ("k", k), ("v", v)):
        if t is not None and not t.is_contiguous():
            raise ValueError("%s must be contiguous" % name)
    B, H, n, dk = q.shape
    Hkv, m = k.shape[1], k.shape[2]
    dv = v.shape[3] if v is not None else dk
    if k.shape[0] != B or k.shape[3] != dk or (
            v is not None and tuple(v.shape[:3]) != (B, Hkv, m)):
        raise ValueError("shape mismatch: q %s, k %s, v %s" % (
            tuple(q.shape), tuple(k.shape), None if v is None else tuple(v.shape)))
    kl_ptr = None
    if key_lens is not None:
        if key_lens.dtype != torch.int32 or key_lens.device != dev or \
                tuple(key_lens.shape) != (B,) or not key_lens.is_contiguous():
            raise ValueError("key_lens must be a contiguous int32 tensor [B] on the GPU of q")
        kl_ptr = key_lens.data_ptr()
    sl_ptr = None
    if alibi_slopes is not None:
        if alibi_slopes.dtype != torch.float32 or alibi_slopes.device != dev or \
                tuple(alibi_slopes.shape) != (H,) or not alibi_slopes.is_contiguous():
            raise ValueError("alibi_slopes must be a contiguous float32 tensor [H] on the GPU of q")
        sl_ptr = alibi_slopes.data_ptr()
    return B, H, Hkv, n, m, dk, dv, code, kl_ptr, sl_ptr


def forward_ex(q, k, v, key_lens=None, causal=False, alibi_slopes=None, scale=None,
               return_lse=False, need_weights=False, out=None, stream=None):
    """The extended forward pass (mha_forward_ex), optionally with the weights.

    k and v may have fewer heads than q (H % H_kv == 0: grouped or
    multi-query attention).  causal: False, True / 'top_left', or
    'bottom_right' (queries aligned to the end of each sequence's L_b
    filled keys, as when decoding against a key/value cache).
    alibi_slopes: float32 [H] on the GPU, or None.  Returns out, then the
    fp32 log-sum-exp [B, H, n] if return_lse, then the weights
    [B, H, n, m] (dtype of q) if need_weights.  Nothing is synchronized.
    """
    import torch
    lib = load()
    B, H, Hkv, n, m, dk, dv, code, kl_ptr, sl_ptr = _device_args(q, k, v, key_lens,
                                                                 alibi_slopes)
    dev = q.device
    if out is None:
        out = torch.empty((B, H, n, dv), dtype=q.dtype, device=dev)
    elif out.shape != (B, H, n, dv) or out.dtype != q.dtype or out.device != dev \
            or not out.is_contiguous():
        raise ValueError("out must be a contiguous [B, H, n, d_v] tensor like q")
    lse = None
    if return_lse or need_weights:
        lse = torch.empty((B, H, n), dtype=torch.float32, device=dev)
    mode = mask_mode(causal)
    sc = default_scale(dk) if scale is None else float(scale)
    if stream is None:
        stream = torch.cuda.current_stream(dev).cuda_stream
    with torch.cuda.device(dev):
        st = lib.mha_forward_ex(q.data_ptr(), k.data_ptr(), v.data_ptr(), kl_ptr, mode,
                                sl_ptr, sc, out.data_ptr(),
                                None if lse is None else lse.data_ptr(),
                                B, H, Hkv, n, m, dk, dv, code, stream)
    _check(st)
    res = (out,)
    if return_lse:
        res += (lse,)
    if need_weights:
        res += (attention_weights(q, k, lse, key_lens=key_lens, causal=causal,
                                  alibi_slopes=alibi_slopes, scale=scale, stream=stream),)
    return res if len(res) > 1 else out


def attention_weights(q, k, lse, key_lens=None, causal=False, alibi_slopes=None,
                      scale=None, out=None, stream=None):
    """A[b,t,i,j] = exp(score - lse) on valid pairs, 0 elsewhere
    (mha_attention_weights); lse from forward_ex with the same arguments."""
    import torch
    lib = load()
    B, H, Hkv, n, m, dk, _, code, kl_ptr, sl_ptr = _device_args(q, k, None, key_lens,
                                                               alibi_slopes)
    dev = q.device
    if lse.dtype != torch.float32 or lse.device != dev or tuple(lse.shape) != (B, H, n) \
            or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 [B, H, n] tensor on the GPU of q")
    if out is None:
        out = torch.empty((B, H, n, m), dtype=q.dtype, device=dev)
    elif out.shape != (B, H, n, m) or out.dtype != q.dtype or out.device != dev \
            or not out.is_contiguous():
        raise ValueError("out must be a contiguous [B, H, n, m] tensor like q")
    sc = default_scale(dk) if scale is None else float(scale)
    if stream is None:
        stream = torch.cuda.current_stream(dev).cuda_stream
    with torch.cuda.device(dev):
        st = lib.mha_attention_weights(q.data_ptr(), k.data_ptr(), kl_ptr, mask_mode(causal),
                                       sl_ptr, sc, lse.data_ptr(), out.data_ptr(),
                                       B, H, Hkv, n, m, dk, code, stream)
    _check(st)
    return out


def _workspace(workspace, dev):
    """A caller's workspace must be contiguous device memory on the GPU of the
    other tensors: the library only sees its address and size."""
    if workspace is not None and (workspace.device != dev or not workspace.is_contiguous()):
        raise ValueError("workspace must be a contiguous tensor on %s" % dev)
    return workspace


def decode_workspace_size(B, H, H_kv, n, m, d, dtype_code) -> int:
    """Bytes of workspace mha_decode needs for these sizes (0: none)."""
    out = ctypes.c_int64(0)
    _check(load().mha_decode_workspace_size(B, H, H_kv, n, m, d, dtype_code, ctypes.byref(out)))
    return int(out.value)


def decode(q, k_cache, v_cache, cache_lens=None, alibi_slopes=None, scale=None,
           return_lse=False, out=None, workspace=None, stream=None):
    """n new queries per sequence against a key/value cache (mha_decode).

    q [B, H, n, d]; k_cache, v_cache [B, H_kv, m, d] with m the capacity;
    cache_lens int32 [B] (filled rows, the new tokens' included) or None.
    Query i is the token at position i + L_b - n.  A workspace of
    decode_workspace_size(...) bytes is allocated when none is given.
    Returns out (and the fp32 log-sum-exp [B, H, n] if return_lse).
    """
    import torch
    lib = load()
    B, H, Hkv, n, m, dk, dv, code, kl_ptr, sl_ptr = _device_args(q, k_cache, v_cache,
                                                                 cache_lens, alibi_slopes)
    dev = q.device
    if out is None:
        out = torch.empty((B, H, n, dv), dtype=q.dtype, device=dev)
    elif out.shape != (B, H, n, dv) or out.dtype != q.dtype or out.device != dev \
            or not out.is_contiguous():
        raise ValueError("out must be a contiguous [B, H, n, d_v] tensor like q")
    lse = torch.empty((B, H, n), dtype=torch.float32, device=dev) if return_lse else None
    need = decode_workspace_size(B, H, Hkv, n, m, dk, code)
    workspace = _workspace(workspace, dev)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_ptr = None if workspace is None else workspace.data_ptr()
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    sc = default_scale(dk) if scale is None else float(scale)
    if stream is None:
        stream = torch.cuda.current_stream(dev).cuda_stream
    with torch.cuda.device(dev):
        st = lib.mha_decode(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), kl_ptr, sl_ptr,
                            sc, out.data_ptr(), None if lse is None else lse.data_ptr(),
                            ws_ptr, ws_bytes, B, H, Hkv, n, m, dk, dv, code, stream)
    _check(st)
    return (out, lse) if return_lse else out


def multihead_workspace_size(B, n, m, d_model, num_heads, dtype_code, need_weights=False):
    """Bytes of workspace mha_multihead_forward needs."""
    out = ctypes.c_int64(0)
    _check(load().mha_multihead_workspace_size(B, n, m, d_model, num_heads, dtype_code,
                                               int(bool(need_weights)), ctypes.byref(out)))
    return int(out.value)


def multihead_forward(xq, xk, xv, Wq, bq, Wk, bk, Wv, bv, Wo, bo, num_heads,
                      key_lens=None, causal=False, scale=None, need_weights=False,
                      out=None, workspace=None, stream=None):
    """Multi-head attention with its projections (mha_multihead_forward).

    xq [B, n, d_model], xk / xv [B, m, d_model]; W* [d_model, d_model] in
    nn.Linear's [out, in] layout, b* [d_model] or None; scale defaults to
    1/sqrt(d_model / num_heads).  Returns Y [B, n, d_model], and the
    weights [B, H, n, m] too when need_weights.
    """
    import torch
    lib = load()
    code = _dtype_code(xq)
    dev = xq.device
    if dev.type != "cuda":
        raise ValueError("the tensors must be on a GPU")
    if xq.dim() != 3 or xk.dim() != 3 or xv.dim() != 3:
        raise ValueError("xq, xk, xv must be 3-D [B, L, d_model]")
    tensors = [xq, xk, xv, Wq, Wk, Wv, Wo] + [b for b in (bq, bk, bv, bo) if b is not None]
    for t in tensors:
        if t.dtype != xq.dtype or t.device != dev or not t.is_contiguous():
            raise ValueError("every tensor must be a contiguous %s tensor on %s" % (xq.dtype, dev))
    B, n, dm = xq.shape
    m = xk.shape[1]
    if tuple(xk.shape) != (B, m, dm) or tuple(xv.shape) != (B, m, dm):
        raise ValueError("xk and xv must be [B, m, d_model]")
    for W in (Wq, Wk, Wv, Wo):
        if tuple(W.shape) != (dm, dm):
            raise ValueError("weights must be [d_model, d_model]")
    for b in (bq, bk, bv, bo):
        if b is not None and tuple(b.shape) != (dm,):
            raise ValueError("biases must be [d_model]")
    kl_ptr = None
    if key_lens is not None:
        if key_lens.dtype != torch.int32 or key_lens.device != dev or \
                tuple(key_lens.shape) != (B,) or not key_lens.is_contiguous():
            raise ValueError("key_lens must be a contiguous int32 tensor [B] on the GPU of xq")
        kl_ptr = key_lens.data_ptr()
    H = int(num_heads)
    if out is None:
        out = torch.empty((B, n, dm), dtype=xq.dtype, device=dev)
    elif tuple(out.shape) != (B, n, dm) or out.dtype != xq.dtype or out.device != dev \
            or not out.is_contiguous():
        raise ValueError("out must be a contiguous [B, n, d_model] tensor like xq")
    A = torch.empty((B, H, n, m), dtype=xq.dtype, device=dev) if need_weights else None
    need = multihead_workspace_size(B, n, m, dm, H, code, need_weights)
    workspace = _workspace(workspace, dev)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    sc = default_scale(dm // H) if scale is None else float(scale)
    if stream is None:
        stream = torch.cuda.current_stream(dev).cuda_stream
    ptr = lambda t: None if t is None else t.data_ptr()  # noqa: E731
    with torch.cuda.device(dev):
        st = lib.mha_multihead_forward(
            ptr(xq), ptr(xk), ptr(xv), ptr(Wq), ptr(bq), ptr(Wk), ptr(bk), ptr(Wv), ptr(bv),
            ptr(Wo), ptr(bo), kl_ptr, mask_mode(causal), sc, out.data_ptr(), ptr(A),
            workspace.data_ptr(), workspace.numel() * workspace.element_size(),
            B, n, m, dm, H, code, stream)
    _check(st)
    return (out, A) if need_weights else out


def validate_ex(q, k, v, key_lens=None, causal=False, alibi_slopes=None, scale=None,
                out=None, lse=None) -> int:
    """The host-side check of mha_forward_ex only; returns the status."""
    B, H, n, dk = q.shape
    Hkv, m, dv = k.shape[1], k.shape[2], v.shape[3]
    sc = default_scale(dk) if scale is None else float(scale)
    ptr = lambda t: None if t is None else t.data_ptr()  # noqa: E731
    return int(load().mha_validate_ex(
        ptr(q), ptr(k), ptr(v), ptr(key_lens), mask_mode(causal), ptr(alibi_slopes), sc,
        ptr(out), ptr(lse), B, H, Hkv, n, m, dk, dv, _dtype_code(q)))


__all__ = ["forward", "forward_ex", "attention_weights", "decode", "decode_workspace_size",
           "multihead_forward", "multihead_workspace_size", "validate", "validate_ex",
           "load", "abi_version", "status_string", "header_functions", "default_scale",
           "mask_mode", "MhaError", "LIB_PATH", "MHA_F32", "MHA_BF16", "MHA_MASK_NONE",
           "MHA_MASK_CAUSAL", "MHA_MASK_CAUSAL_BOTTOM_RIGHT"]
