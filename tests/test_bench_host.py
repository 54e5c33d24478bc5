"""Host-side arithmetic of the benchmark: the metric's FLOP count, the
algorithmic bytes, the count of valid (query, key) pairs, and the refusal of
more than one GPU.  Each is checked against a value written out by hand
from its definition, or against a brute-force count over every pair."""
import os
import subprocess
import sys

import numpy as np
import pytest

import bench
from transformer_head_scaled_fwd_amd import inputs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_metric_flops_follow_the_formula():
    # 4 * B * H * n * m * d, halved for causal attention.
    W = inputs.WORKLOADS
    assert W["fp32_small"].metric_flops() == 4 * 1 * 8 * 16 * 16 * 64
    assert W["encoder_pad_n128"].metric_flops() == 4 * 32 * 8 * 128 * 128 * 64
    assert W["decoder_causal_n512"].metric_flops() == 4 * 16 * 8 * 512 * 512 * 64 / 2
    assert W["cross_n256_m1024"].metric_flops() == 4 * 8 * 16 * 256 * 1024 * 64
    assert W["causal_n16384_d128"].metric_flops() == 4 * 1 * 16 * 16384 * 16384 * 128 / 2
    assert abs(W["causal_n16384_d128"].metric_flops() - 1.0995e12) < 1e8


def test_algorithmic_bytes_without_padding():
    # Q and O once, K and V once: four tensors of B*H*n*d elements.
    w = inputs.WORKLOADS["causal_n16384_d128"]
    assert bench.algorithmic_bytes(w, None) == 4 * 16 * 16384 * 128 * 2 == 256 << 20
    w = inputs.WORKLOADS["decoder_causal_n512"]
    assert bench.algorithmic_bytes(w, None) == 4 * 16 * 8 * 512 * 64 * 2 == 32 << 20
    w = inputs.WORKLOADS["fp32_small"]
    assert bench.algorithmic_bytes(w, None) == 4 * 8 * 16 * 64 * 4


def test_algorithmic_bytes_count_only_valid_key_rows():
    w = inputs.Workload("t", 3, 2, 10, 20, 64, "bf16", False, (0, 20), 0)
    lens = np.array([0, 7, 25], np.int32)          # the last is clamped to m = 20
    q_and_o = 2 * 3 * 2 * 10 * 64 * 2
    kv = (0 + 7 + 20) * 2 * (64 + 64) * 2           # per head, K and V rows
    assert bench.algorithmic_bytes(w, lens) == q_and_o + kv + 4 * 3


@pytest.mark.parametrize("causal", [False, True])
def test_valid_pairs_against_brute_force(causal):
    rng = np.random.Generator(np.random.PCG64(5))
    n = 37
    w = inputs.Workload("t", 4, 3, n, n, 64, "bf16", causal, (0, n), 0)
    lens = rng.integers(0, n + 3, size=4).astype(np.int32)
    count = 0
    for b in range(4):
        L = min(int(lens[b]), n)
        for i in range(n):
            for j in range(n):
                count += (j < L) and (not causal or j <= i)
    assert bench.valid_pairs(w, lens) == 3 * count


@pytest.mark.parametrize("causal", [False, True, "top_left", "bottom_right"])
def test_visible_keys_against_brute_force(causal):
    n, L = 9, 14
    got = bench.visible_keys(n, L, causal)
    for i in range(n):
        p = i + (L - n if causal == "bottom_right" else 0)   # the query's position
        want = sum(1 for j in range(L) if causal in (False, None) or j <= p)
        assert got[i] == want


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr


def test_cpu_baseline_runs_the_whole_workload_or_distinct_rows():
    import oracle
    w = inputs.Workload("t", 2, 3, 40, 40, 64, "bf16", True, None, 3)
    host = inputs.make(w)
    cpu, rows, ref, dt = bench.cpu_baseline(w, host, max_s=1e6)
    assert rows is None and "all 240 query rows" in cpu["sample"]
    full = oracle.attention(*host[:3], key_lens=host[3], causal=True, scale=w.scale)
    np.testing.assert_array_equal(ref, full)
    # a budget no full run fits: distinct rows, the oracle's values for them
    cpu, rows, ref, dt = bench.cpu_baseline(w, host, max_s=1e-9)
    assert rows is not None and "without replacement" in cpu["sample"]
    assert len({tuple(r) for r in rows}) == len(rows)
    np.testing.assert_array_equal(ref, full[rows[:, 0], rows[:, 1], rows[:, 2]])
    rec = bench.parity(w, host, host[0].new_zeros(host[0].shape), rows=rows, ref=ref)
    assert rec["compared"] == "%d sampled rows" % len(rows)


def test_kernel_hash_ignores_comments_only():
    # The profiles' kernel hash is taken over the code with comments and
    # layout removed: a comment or a blank line leaves it, a token changes it.
    code = "int f(int x) {  // twice\n  return 2 * x; /* doubled */\n}\n"
    assert bench.kernel_code(code) == "int f(int x) { return 2 * x; }"
    assert bench.kernel_code(code.replace("// twice", "// two times")) == bench.kernel_code(code)
    assert bench.kernel_code(code.replace("2 * x", "3 * x")) != bench.kernel_code(code)
