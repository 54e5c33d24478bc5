"""Seeded synthetic inputs for attention workloads.

This module holds no attention arithmetic.  It draws Q, K, V and key lengths
from a seeded generator and rounds them to the storage dtype; the GPU path
and the CPU oracle both receive exactly these bits.

Recipe (one generator per workload):
  * ``numpy.random.Generator(PCG64(seed)).standard_normal(shape)`` in float64,
    drawn in the order Q, K, V, each whole tensor in C order;
  * multiplied by ``value_scale`` (a power of two, so exact), cast to float32,
    then rounded to bfloat16 with round-to-nearest-even for bf16 workloads;
  * then ``key_lens = integers(lo, hi + 1, size=B)`` (inclusive bounds) when
    the workload has key padding.

The shapes follow the pages' workloads: the base model's 8 heads of width 64
and the big model's 16 heads ("序列建模架构的演进与变革（二）" §4.9 and the
hugogu wiki "Transformer" page, which give d_model = 512, h = 8,
d_k = d_v = 64), sentences padded to the batch maximum with lengths up to
512 ("Transformer: 详解" §3.3), and a long causal stress shape.  Values are
iid N(0, 1), for which the variance of q.k is d_k
("序列建模架构的演进与变革（二）" §4.4).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional, Tuple

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    n: int
    m: int
    d: int
    dtype: str                 # "f32" or "bf16"
    causal: bool
    lens: Optional[Tuple[int, int]]   # inclusive (lo, hi) for key_lens, or None
    seed: int
    value_scale: float = 1.0
    note: str = field(default="", compare=False)

    @property
    def scale(self) -> float:
        return float(np.float32(1.0 / np.sqrt(self.d)))

    def metric_flops(self) -> float:
        """4 * B * H * n * m * d, halved for causal attention."""
        f = 4.0 * self.B * self.H * self.n * self.m * self.d
        return f / 2.0 if self.causal else f


WORKLOADS = {
    "fp32_small": Workload(
        "fp32_small", B=1, H=8, n=16, m=16, d=64, dtype="f32", causal=False,
        lens=None, seed=0,
        note="fp32, one batch of 8 heads, 16x16, no mask"),
    "encoder_pad_n128": Workload(
        "encoder_pad_n128", B=32, H=8, n=128, m=128, d=64, dtype="bf16",
        causal=False, lens=(16, 128), seed=1,
        note="encoder self-attention, key padding, lengths U{16..128}"),
    "decoder_causal_n512": Workload(
        "decoder_causal_n512", B=16, H=8, n=512, m=512, d=64, dtype="bf16",
        causal=True, lens=None, seed=2,
        note="decoder causal self-attention, no padding"),
    "cross_n256_m1024": Workload(
        "cross_n256_m1024", B=8, H=16, n=256, m=1024, d=64, dtype="bf16",
        causal=False, lens=(512, 1024), seed=3,
        note="cross-attention, 256 queries vs 1024 keys, key padding U{512..1024}"),
    "causal_n16384_d128": Workload(
        "causal_n16384_d128", B=1, H=16, n=16384, m=16384, d=128, dtype="bf16",
        causal=True, lens=None, seed=4, value_scale=0.5,
        note="long causal self-attention, values N(0,1)*0.5"),
}

ORDER = ["fp32_small", "encoder_pad_n128", "decoder_causal_n512",
         "cross_n256_m1024", "causal_n16384_d128"]


def _round(x64: np.ndarray, dtype: str) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(x64.astype(np.float32)))
    if dtype == "bf16":
        return t.to(torch.bfloat16)   # round to nearest even
    if dtype == "f32":
        return t
    raise ValueError("dtype must be 'f32' or 'bf16'")


def draw(B, H, n, m, dk, dv, dtype, seed, lens=None, value_scale=1.0):
    """Draw (q, k, v, key_lens) on the CPU.

    q, k, v are torch CPU tensors of the storage dtype; key_lens is an int32
    numpy array of shape (B,) or None.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    q = _round(rng.standard_normal((B, H, n, dk)) * value_scale, dtype)
    k = _round(rng.standard_normal((B, H, m, dk)) * value_scale, dtype)
    v = _round(rng.standard_normal((B, H, m, dv)) * value_scale, dtype)
    key_lens = None
    if lens is not None:
        lo, hi = lens
        key_lens = rng.integers(lo, hi + 1, size=B).astype(np.int32)
    return q, k, v, key_lens


def make(w: Workload):
    """Inputs of a named workload: (q, k, v, key_lens)."""
    return draw(w.B, w.H, w.n, w.m, w.d, w.d, w.dtype, w.seed, w.lens,
                w.value_scale)


# --- workloads of the extended entry points ------------------------------------
#
# Grouped K/V heads, ALiBi, bottom-right causal alignment and the weights
# output.  Same recipe; K and V are drawn with H_kv heads, and ALiBi slopes
# are the geometric sequence 2^(-8(t+1)/H) over the heads (an input choice:
# the pages give the slopes only as head-specific constants).

@dataclass(frozen=True)
class ExtWorkload:
    name: str
    B: int
    H: int
    H_kv: int
    n: int
    m: int
    d: int
    dtype: str
    causal: object                    # False, "top_left" or "bottom_right"
    lens: Optional[Tuple[int, int]]
    seed: int
    alibi: bool = False
    weights: bool = False
    decode: bool = False              # run through mha_decode (m = cache capacity)
    value_scale: float = 1.0
    note: str = field(default="", compare=False)

    @property
    def scale(self) -> float:
        return float(np.float32(1.0 / np.sqrt(self.d)))


def alibi_slopes(H: int) -> np.ndarray:
    """fp32 slopes 2^(-8(t+1)/H), t = 0..H-1."""
    return np.array([2.0 ** (-8.0 * (t + 1) / H) for t in range(H)], np.float32)


EXT_WORKLOADS = {
    "gqa_prefill_n4096": ExtWorkload(
        "gqa_prefill_n4096", B=2, H=32, H_kv=8, n=4096, m=4096, d=128, dtype="bf16",
        causal="top_left", lens=None, seed=11,
        note="causal prefill, 32 query heads over 8 K/V heads"),
    "alibi_causal_n2048": ExtWorkload(
        "alibi_causal_n2048", B=8, H=16, H_kv=16, n=2048, m=2048, d=64, dtype="bf16",
        causal="top_left", lens=None, seed=12, alibi=True,
        note="causal self-attention with ALiBi"),
    "weights_n512": ExtWorkload(
        "weights_n512", B=8, H=8, H_kv=8, n=512, m=512, d=64, dtype="bf16",
        causal=False, lens=(256, 512), seed=13, weights=True,
        note="encoder self-attention returning the weights, padding U{256..512}"),
    "decode_gqa_m16384": ExtWorkload(
        "decode_gqa_m16384", B=8, H=32, H_kv=8, n=1, m=16384, d=128, dtype="bf16",
        causal="bottom_right", lens=(8192, 16384), seed=14, decode=True,
        note="one decoding step, 8 sequences, 32 query heads over 8 K/V heads, "
             "caches of capacity 16384 filled to U{8192..16384}"),
    "decode_mha_m8192": ExtWorkload(
        "decode_mha_m8192", B=1, H=32, H_kv=32, n=1, m=8192, d=128, dtype="bf16",
        causal="bottom_right", lens=None, seed=15, decode=True,
        note="one decoding step of one sequence with an 8K context, 32 heads of 128"),
}

EXT_ORDER = ["gqa_prefill_n4096", "alibi_causal_n2048", "weights_n512",
             "decode_gqa_m16384", "decode_mha_m8192"]


def draw_ex(w: ExtWorkload, seed_offset: int = 0):
    """(q, k, v, key_lens, slopes) of an extended workload, on the CPU."""
    rng = np.random.Generator(np.random.PCG64(w.seed + seed_offset))
    q = _round(rng.standard_normal((w.B, w.H, w.n, w.d)) * w.value_scale, w.dtype)
    k = _round(rng.standard_normal((w.B, w.H_kv, w.m, w.d)) * w.value_scale, w.dtype)
    v = _round(rng.standard_normal((w.B, w.H_kv, w.m, w.d)) * w.value_scale, w.dtype)
    key_lens = None
    if w.lens is not None:
        lo, hi = w.lens
        key_lens = rng.integers(lo, hi + 1, size=w.B).astype(np.int32)
    return q, k, v, key_lens, (alibi_slopes(w.H) if w.alibi else None)


# --- the multi-head layer (projections around the core) --------------------------
#
# The pages' base configuration, d_model = 512 with 8 heads of 64
# ("Transformer: 详解" §4.2; "序列建模架构的演进与变革（二）" §4.9), and their
# big model's width d_model = 1024 ("Transformer: 详解" §7.2), here with 16
# heads of 64; sentences padded to the batch maximum, up to 512 tokens.  X ~ N(0, 1); weights and biases ~ U(-1/sqrt(d_model),
# 1/sqrt(d_model)), nn.Linear's initialisation range, rounded to the dtype.

@dataclass(frozen=True)
class LayerWorkload:
    name: str
    B: int
    n: int
    d_model: int
    H: int
    dtype: str
    causal: object
    lens: Optional[Tuple[int, int]]
    seed: int
    note: str = field(default="", compare=False)


LAYER_WORKLOADS = {
    "mha_layer_base_n128": LayerWorkload(
        "mha_layer_base_n128", B=32, n=128, d_model=512, H=8, dtype="bf16", causal=False,
        lens=(16, 128), seed=21, note="encoder self-attention layer, base model"),
    "mha_layer_big_n512": LayerWorkload(
        "mha_layer_big_n512", B=16, n=512, d_model=1024, H=16, dtype="bf16", causal=True,
        lens=None, seed=22, note="decoder self-attention layer, big model, 512 tokens"),
}

LAYER_ORDER = ["mha_layer_base_n128", "mha_layer_big_n512"]


def draw_layer(w: LayerWorkload, seed_offset: int = 0):
    """(x, x, x, [Wq, Wk, Wv, Wo], [bq, bk, bv, bo], key_lens) of a
    self-attention layer workload, on the CPU."""
    rng = np.random.Generator(np.random.PCG64(w.seed + seed_offset))
    x = _round(rng.standard_normal((w.B, w.n, w.d_model)), w.dtype)
    bound = 1.0 / np.sqrt(w.d_model)
    Ws = [_round(rng.uniform(-bound, bound, (w.d_model, w.d_model)), w.dtype) for _ in range(4)]
    bs = [_round(rng.uniform(-bound, bound, w.d_model), w.dtype) for _ in range(4)]
    key_lens = None
    if w.lens is not None:
        lo, hi = w.lens
        key_lens = rng.integers(lo, hi + 1, size=w.B).astype(np.int32)
    return x, x, x, Ws, bs, key_lens



def device_normal(shape, seed: int, dtype: str = "bf16", device: str = "cuda:0") -> torch.Tensor:
    """N(0, 1) values drawn on the device, for tensors too large to draw and
    copy from the host (heads near the 2 GiB limit): torch's seeded device
    generator in float32, then rounded to the storage dtype with
    round-to-nearest-even.  Callers that check such a tensor against the
    oracle copy the rows they sample back to the host, so both sides still
    see the same bits."""
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    return x if dtype == "f32" else x.to(torch.bfloat16)
