"""GPU parity: libmha (HIP kernels through the C ABI) against the CPU oracle.

Every comparison runs both sides on the same seeded input bits.  The bar is
the max-abs error over all compared elements of O: 1e-5 for fp32 inputs and
1.5e-2 for bf16 inputs with fp32 accumulation (V ~ N(0,1) sets the
reference scale at 1.0).  Bit-level checks are used where the method makes
the result exact (a row that sees one key, padding that must not be read).
"""
import numpy as np
import pytest
import torch

import oracle
import transformer_head_scaled_fwd_amd as mha
from conftest import load_golden
from transformer_head_scaled_fwd_amd import inputs

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "bf16": 1.5e-2}
TDT = {"f32": torch.float32, "bf16": torch.bfloat16}


def _say(msg):
    print(msg, flush=True)


def run_gpu(q, k, v, key_lens=None, causal=False, scale=None, dev="cuda:0"):
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    kl = None if key_lens is None else torch.as_tensor(np.asarray(key_lens, np.int32)).to(dev)
    o = mha.forward(qd, kd, vd, key_lens=kl, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return o.cpu()


def compare(o_gpu, o_ref, tol, what=""):
    og = oracle.to_f64(o_gpu)
    err = np.abs(og - o_ref)
    worst = np.unravel_index(np.argmax(err), err.shape) if err.size else ()
    mx = float(err.max()) if err.size else 0.0
    _say("%s max_abs_err=%.3e mean_abs_err=%.3e at %s" %
         (what, mx, float(err.mean()) if err.size else 0.0, worst))
    assert np.all(np.isfinite(og)), "non-finite output"
    assert mx <= tol, "%s: max abs error %.3e > %.1e at %s" % (what, mx, tol, worst)
    return mx


def store_floor(o_ref):
    """Error of merely rounding the exact result to bf16."""
    t = torch.from_numpy(o_ref.astype(np.float32)).to(torch.bfloat16).double().numpy()
    return float(np.abs(t - o_ref).max())


# --- the five workloads ----------------------------------------------------------

@pytest.mark.parametrize("name", ["fp32_small", "encoder_pad_n128",
                                  "decoder_causal_n512", "cross_n256_m1024"])
def test_workload_full_oracle(gpu, name):
    w = inputs.WORKLOADS[name]
    _say("workload %s" % name)
    q, k, v, kl = inputs.make(w)
    o = run_gpu(q, k, v, kl, w.causal, w.scale)
    ref = oracle.attention(q, k, v, key_lens=kl, causal=w.causal, scale=w.scale)
    if w.dtype == "bf16":
        _say("store floor %.3e" % store_floor(ref))
    compare(o, ref, TOL[w.dtype], name)


def test_workload_long_causal_sampled_rows(gpu):
    w = inputs.WORKLOADS["causal_n16384_d128"]
    _say("workload %s (sampled rows)" % w.name)
    q, k, v, kl = inputs.make(w)
    o = run_gpu(q, k, v, kl, w.causal, w.scale)
    rng = np.random.Generator(np.random.PCG64(1234))
    fixed = [0, 1, 31, 32, 63, 64, 127, 128, 129, 255, 256, 4095, 4096, 8191,
             w.n - 129, w.n - 128, w.n - 2, w.n - 1]
    rows = []
    for t in range(w.H):
        picks = sorted(set(fixed) | set(rng.integers(0, w.n, 40).tolist()))
        rows += [[0, t, i] for i in picks]
    rows = np.array(rows, np.int64)
    ref = oracle.attention_rows(q, k, v, rows, key_lens=kl, causal=True, scale=w.scale)
    got = o[rows[:, 0], rows[:, 1], rows[:, 2]]
    compare(got, ref, TOL["bf16"], "%s %d rows" % (w.name, len(rows)))
    assert torch.isfinite(o.float()).all()


def test_workload_long_causal_every_element(gpu):
    """Every element of the long causal workload against the oracle, one head
    at a time (the oracle's row mode over all n rows of the head)."""
    w = inputs.WORKLOADS["causal_n16384_d128"]
    _say("workload %s (every element)" % w.name)
    q, k, v, kl = inputs.make(w)
    o = run_gpu(q, k, v, kl, w.causal, w.scale)
    worst = 0.0
    floor = 0.0
    for t in range(w.H):
        rows = np.stack([np.zeros(w.n, np.int64), np.full(w.n, t, np.int64),
                         np.arange(w.n, dtype=np.int64)], 1)
        ref = oracle.attention_rows(q, k, v, rows, key_lens=kl, causal=True, scale=w.scale)
        floor = max(floor, store_floor(ref))
        worst = max(worst, compare(o[0, t], ref, TOL["bf16"], "%s head %d" % (w.name, t)))
    _say("%s: max_abs_err %.3e over all %d outputs, store floor %.3e"
         % (w.name, worst, o.numel(), floor))


# --- shapes spanning several tiles with ragged tails ------------------------------

CASES = [
    # B, H, n, m, d, dtype, causal, lens
    (2, 3, 300, 300, 64, "bf16", False, (0, 300)),
    (2, 3, 300, 300, 64, "bf16", True, None),
    (2, 2, 333, 333, 128, "bf16", True, (1, 333)),
    (1, 4, 77, 333, 128, "bf16", False, (200, 333)),
    (3, 2, 1, 1, 64, "bf16", False, None),
    (2, 2, 1, 700, 128, "bf16", False, (1, 700)),
    (2, 2, 700, 5, 64, "bf16", False, None),
    (2, 3, 300, 300, 64, "f32", True, (1, 300)),
    (2, 2, 200, 257, 128, "f32", False, (0, 257)),
    (1, 2, 129, 129, 128, "f32", True, None),
]


@pytest.mark.parametrize("B,H,n,m,d,dt,causal,lens", CASES)
def test_ragged_shapes(gpu, B, H, n, m, d, dt, causal, lens):
    _say("case B=%d H=%d n=%d m=%d d=%d %s causal=%s lens=%s" % (B, H, n, m, d, dt, causal, lens))
    q, k, v, kl = inputs.draw(B, H, n, m, d, d, dt, seed=100 + n + m + d, lens=lens)
    if kl is not None and lens[0] == 0:
        kl[0] = 0               # one sequence with no valid key: its output is 0
    o = run_gpu(q, k, v, kl, causal)
    ref = oracle.attention(q, k, v, key_lens=kl, causal=causal)
    compare(o, ref, TOL[dt], "ragged")
    if kl is not None and lens[0] == 0:
        assert torch.count_nonzero(o[0]) == 0


# --- the largest heads the C ABI accepts -------------------------------------------
# A head's tensor must stay under 2 GiB (the kernels address a head with
# 32-bit buffer offsets): for bf16 rows of d = 128 that is n, m <= 2^23 - 1.

def test_max_query_rows_per_head(gpu):
    n, m, d = (1 << 23) - 1, 100, 128
    _say("max query rows: n=%d m=%d d=%d bf16 (Q and O heads of %.4f GiB)"
         % (n, m, d, n * d * 2 / 2 ** 30))
    dev = "cuda:0"
    q = inputs.device_normal((1, 1, n, d), seed=31)
    _, k, v, _ = inputs.draw(1, 1, 1, m, d, d, "bf16", seed=32)
    o = mha.forward(q, k.to(dev), v.to(dev))
    torch.cuda.synchronize()
    rng = np.random.Generator(np.random.PCG64(33))
    rows = np.unique(np.concatenate([np.arange(64), np.arange(n - 200, n),
                                     rng.integers(0, n, 200)]))
    idx = torch.as_tensor(rows, device=dev)
    qs = q[0, 0].index_select(0, idx).cpu().reshape(1, 1, len(rows), d)
    got = o[0, 0].index_select(0, idx).cpu().reshape(1, 1, len(rows), d)
    ref = oracle.attention(qs, k, v)
    compare(got, ref, TOL["bf16"], "max n, %d sampled rows" % len(rows))
    del q, o
    torch.cuda.empty_cache()


def test_max_key_rows_per_head(gpu):
    # Q = 0 makes every valid score equal, so each output row is the mean of
    # the valid value rows ("序列建模架构的演进与变革（二）" §4.3: weights sum to
    # 1).  Rows past the length hold NaN and must never be read.
    n, m, d = 64, (1 << 23) - 1, 128
    L = m - 7
    _say("max key rows: n=%d m=%d (valid %d) d=%d bf16" % (n, m, L, d))
    dev = "cuda:0"
    k = inputs.device_normal((1, 1, m, d), seed=34)
    v = inputs.device_normal((1, 1, m, d), seed=35)
    k[0, 0, L:] = float("nan")
    v[0, 0, L:] = float("nan")
    q = torch.zeros((1, 1, n, d), dtype=torch.bfloat16, device=dev)
    kl = torch.tensor([L], dtype=torch.int32, device=dev)
    o = mha.forward(q, k, v, key_lens=kl)
    torch.cuda.synchronize()
    vh = v[0, 0, :L].cpu()
    total = np.zeros(d)
    for c0 in range(0, L, 1 << 20):
        total += oracle.to_f64(vh[c0:c0 + (1 << 20)]).sum(axis=0)
    ref = np.broadcast_to(total / L, (1, 1, n, d))
    compare(o.cpu(), ref, TOL["bf16"], "max m, Q = 0")
    del k, v, o
    torch.cuda.empty_cache()


# --- the pages' worked examples on the GPU -----------------------------------------

@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_worked_example_4token_padded(gpu, dt):
    g = load_golden("worked_example_4token.json")
    d = 64
    q = torch.zeros(1, 1, 1, d)
    k = torch.zeros(1, 1, 4, d)
    v = torch.zeros(1, 1, 4, d)
    q[0, 0, 0, :2] = torch.tensor(g["q"])
    k[0, 0, :, :2] = torch.tensor(g["K"])
    v[0, 0, :, :2] = torch.tensor(g["V"])
    q, k, v = q.to(TDT[dt]), k.to(TDT[dt]), v.to(TDT[dt])
    scale = float(np.float32(1 / np.sqrt(g["d_k"])))   # zero columns add nothing
    o = run_gpu(q, k, v, scale=scale)
    ref = oracle.attention(q, k, v, scale=scale)
    compare(o, ref, TOL[dt], "4-token example " + dt)
    np.testing.assert_allclose(o[0, 0, 0, :2].double().numpy(), g["printed_output"],
                               atol=g["printed_tolerance"] + (0 if dt == "f32" else 0.01))
    assert torch.count_nonzero(o[0, 0, 0, 2:]) == 0


def test_causal_3x3_example_padded(gpu):
    g = load_golden("causal_softmax_3x3.json")
    d = 64
    q = torch.zeros(1, 1, 3, d)
    q[0, 0, :, :3] = torch.tensor(g["scaled_scores"])
    e = torch.zeros(1, 1, 3, d)
    e[0, 0, :, :3] = torch.eye(3)
    o = run_gpu(q, e, e.clone(), causal=True, scale=1.0)
    A = o[0, 0, :, :3].double().numpy()
    printed = np.array(g["printed_softmax"])
    for r in g["rows_that_follow_from_the_printed_scores"]:
        np.testing.assert_allclose(A[r], printed[r], atol=g["printed_tolerance"])
    x = np.exp(np.array(g["scaled_scores"][2]))
    np.testing.assert_allclose(A[2], x / x.sum(), atol=1e-5)


# --- invariants ------------------------------------------------------------------------

@pytest.mark.parametrize("dt,d", [("bf16", 64), ("bf16", 128), ("f32", 64)])
def test_causal_row0_is_v0_bitwise(gpu, dt, d):
    q, k, v, _ = inputs.draw(2, 3, 200, 200, d, d, dt, seed=7)
    o = run_gpu(q, k, v, causal=True)
    assert torch.equal(o[:, :, 0, :], v[:, :, 0, :])


@pytest.mark.parametrize("causal", [False, True])
def test_zero_query_is_mean_of_valid_values(gpu, causal):
    B, H, n, d = 3, 2, 260, 128
    _, k, v, kl = inputs.draw(B, H, n, n, d, d, "bf16", seed=8, lens=(1, n))
    q = torch.zeros(B, H, n, d, dtype=torch.bfloat16)
    o = run_gpu(q, k, v, kl, causal)
    V = oracle.to_f64(v)
    ref = np.zeros((B, H, n, d))
    for b in range(B):
        for i in range(n):
            cnt = min(i + 1, int(kl[b])) if causal else int(kl[b])
            ref[b, :, i] = V[b, :, :cnt].mean(axis=1)
    compare(o, ref, TOL["bf16"], "Q=0 mean")


@pytest.mark.parametrize("dt,causal", [("bf16", False), ("bf16", True), ("f32", False)])
def test_padding_is_never_read(gpu, dt, causal):
    B, H, n, d = 4, 2, 300, 128
    q, k, v, kl = inputs.draw(B, H, n, n, d, d, dt, seed=9, lens=(1, n))
    o1 = run_gpu(q, k, v, kl, causal)
    k2, v2 = k.clone(), v.clone()
    for b in range(B):
        L = int(kl[b])
        k2[b, :, L:] = float("nan")
        v2[b, :, L:] = float("inf")
        if L + 1 < n:
            k2[b, :, L + 1:] = 1e4
    o2 = run_gpu(q, k2, v2, kl, causal)
    assert torch.equal(o1, o2)


def test_permutation_equivariance(gpu):
    B, H, n, d = 2, 2, 300, 64
    q, k, v, _ = inputs.draw(B, H, n, n, d, d, "bf16", seed=10)
    P = torch.from_numpy(np.random.Generator(np.random.PCG64(3)).permutation(n))
    o = run_gpu(q, k, v)
    op = run_gpu(q[:, :, P].contiguous(), k[:, :, P].contiguous(), v[:, :, P].contiguous())
    compare(op, oracle.to_f64(o[:, :, P]), TOL["bf16"], "P.O")
    okv = run_gpu(q, k[:, :, P].contiguous(), v[:, :, P].contiguous())
    compare(okv, oracle.to_f64(o), TOL["bf16"], "permuted K,V")


def test_deterministic(gpu):
    w = inputs.WORKLOADS["decoder_causal_n512"]
    q, k, v, kl = inputs.make(w)
    outs = [run_gpu(q, k, v, kl, w.causal) for _ in range(3)]
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[1], outs[2])


def test_guard_bands_untouched(gpu):
    B, H, n, d = 2, 3, 130, 128
    q, k, v, kl = inputs.draw(B, H, n, n, d, d, "bf16", seed=12, lens=(1, n))
    dev = "cuda:0"
    total = B * H * n * d
    pad = 4096
    buf = torch.full((total + 2 * pad,), 12345.0, dtype=torch.bfloat16, device=dev)
    out = buf[pad:pad + total].view(B, H, n, d)
    mha.forward(q.to(dev), k.to(dev), v.to(dev),
                key_lens=torch.as_tensor(kl).to(dev), causal=True, out=out)
    torch.cuda.synchronize()
    assert torch.all(buf[:pad] == 12345.0) and torch.all(buf[pad + total:] == 12345.0)
    ref = oracle.attention(q, k, v, key_lens=kl, causal=True)
    compare(out.cpu(), ref, TOL["bf16"], "guarded")


def test_side_stream(gpu):
    q, k, v, kl = inputs.draw(2, 2, 256, 256, 64, 64, "bf16", seed=13, lens=(1, 256))
    s = torch.cuda.Stream()
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    kld = torch.as_tensor(kl).cuda()
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        o = mha.forward(qd, kd, vd, key_lens=kld)
    s.synchronize()
    ref = oracle.attention(q, k, v, key_lens=kl)
    compare(o.cpu(), ref, TOL["bf16"], "side stream")


def test_zero_keys_writes_zeros(gpu):
    q = torch.randn(1, 2, 70, 64).to(torch.bfloat16).cuda()
    k = torch.zeros(1, 2, 0, 64, dtype=torch.bfloat16, device="cuda")
    out = torch.full((1, 2, 70, 64), 7.0, dtype=torch.bfloat16, device="cuda")
    mha.forward(q, k, k.clone(), out=out)
    torch.cuda.synchronize()
    assert torch.count_nonzero(out) == 0


def test_errors_through_binding(gpu):
    q = torch.zeros(1, 1, 8, 64, dtype=torch.bfloat16, device="cuda")
    k = torch.zeros(1, 1, 9, 64, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(mha.MhaError) as e:
        mha.forward(q, k, k.clone(), causal=True)
    assert e.value.status == 2
    q96 = torch.zeros(1, 1, 8, 96, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(mha.MhaError) as e:
        mha.forward(q96, q96.clone(), q96.clone())
    assert e.value.status == 4


@pytest.mark.parametrize("causal", [False, True])
def test_rising_scores_take_the_exact_path(gpu, causal):
    # Scores that climb by far more than the on-demand check allows from one
    # 64-key block to the next: key j is 2j along the query's direction, so
    # a block's scores beat the previous block's by about 23 in log2 units
    # (scale 1/8).  Every block then takes the exact path (block max, raise,
    # rescale); the result must still match the oracle.
    B, H, n, d = 1, 2, 320, 64
    _, _, v, _ = inputs.draw(B, H, n, n, d, d, "bf16", seed=61)
    q = torch.zeros(B, H, n, d)
    k = torch.zeros(B, H, n, d)
    q[..., 0] = 1.0
    k[..., 0] = 2.0 * torch.arange(n, dtype=torch.float32)
    k[..., 1] = torch.linspace(-1, 1, n)          # a little structure off the ramp
    q[..., 1] = torch.linspace(1, -1, n)
    q, k = q.to(torch.bfloat16), k.to(torch.bfloat16)
    o = run_gpu(q, k, v, causal=causal)
    ref = oracle.attention(q, k, v, causal=causal)
    compare(o, ref, TOL["bf16"], "rising scores")


def _variant(B, H, n, m, d, causal):
    name = mha.load().mha_forward_kernel_name(B, H, H, n, m, d, mha.MHA_BF16, int(causal), 0)
    return name.decode()


def _ramp_inputs(B, H, n, m, d, step, seed):
    # Key j lies `step * j` along the query's direction, so the scores of a
    # 64-key block beat those of the block before by 64 * step * scale
    # (about 33 in log2 units for step 4 at d = 128, 45 at d = 64): every
    # block's weights against the running max pass the on-demand bound and
    # the wave takes the exact path (block max, raise, rescale).
    _, _, v, _ = inputs.draw(B, H, n, m, d, d, "bf16", seed=seed)
    q = torch.zeros(B, H, n, d)
    k = torch.zeros(B, H, m, d)
    q[..., 0] = 1.0
    k[..., 0] = step * torch.arange(m, dtype=torch.float32)
    k[..., 1] = torch.linspace(-1, 1, m)
    q[..., 1] = torch.linspace(1, -1, n)
    return q.to(torch.bfloat16), k.to(torch.bfloat16), v


@pytest.mark.parametrize("B,H,n,m,d,causal,variant", [
    # eight waves over 256 query rows (long key walks, the long-sequence
    # workload's variant); the oracle on sampled rows
    (2, 16, 8192, 8192, 128, True, "<__bf16, 128, 8, 1, true, false>"),
    (4, 16, 4096, 3072, 128, False, "<__bf16, 128, 8, 1, false, false>"),
    # four waves over 128 rows, two workgroups per CU
    (4, 16, 1024, 1024, 128, True, "<__bf16, 128, 4, 1, true, false>"),
    # two key groups per workgroup, merged at the end
    (1, 4, 320, 1280, 128, False, "<__bf16, 128, 8, 2, false, false>"),
    (1, 1, 1280, 1280, 64, True, "<__bf16, 64, 8, 2, true, false>"),
])
def test_rising_scores_take_the_exact_path_in_every_variant(gpu, B, H, n, m, d, causal, variant):
    assert _variant(B, H, n, m, d, causal).endswith(variant)
    q, k, v = _ramp_inputs(B, H, n, m, d, 4.0, seed=62)
    o = run_gpu(q, k, v, causal=causal)
    if B * H * n * m <= 1 << 27:
        ref = oracle.attention(q, k, v, causal=causal)
        compare(o, ref, TOL["bf16"], "rising scores, " + variant)
    else:
        rng = np.random.Generator(np.random.PCG64(64))
        flat = rng.choice(B * H * n, size=768, replace=False)
        rows = np.stack([flat // (H * n), (flat // n) % H, flat % n], 1).astype(np.int64)
        rows = np.concatenate([rows, [[B - 1, H - 1, n - 1], [0, 0, 0]]]).astype(np.int64)
        ref = oracle.attention_rows(q, k, v, rows, causal=causal)
        got = o[torch.from_numpy(rows[:, 0]), torch.from_numpy(rows[:, 1]),
                torch.from_numpy(rows[:, 2])]
        compare(got, ref, TOL["bf16"], "rising scores (sampled rows), " + variant)


def test_deterministic_eight_wave_d128(gpu):
    # The eight-wave d = 128 variant that carries the long-sequence
    # workload: bit-identical outputs run after run.
    B, H, n, d = 2, 16, 8192, 128
    assert _variant(B, H, n, n, d, True).endswith("<__bf16, 128, 8, 1, true, false>")
    q, k, v, _ = inputs.draw(B, H, n, n, d, d, "bf16", seed=63, value_scale=0.5)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    outs = [mha.forward(qd, kd, vd, causal=True) for _ in range(3)]
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[1], outs[2])
