"""Benchmark of the attention forward pass on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One step is one mha_forward call over one batch of the workload (default:
causal self-attention, B=1, H=16, n=m=16384, d=128, bf16), with inputs
already resident in HBM.  W untimed steps, then exactly K timed steps
bracketed by device synchronisation; HIP events on the launch stream give
the per-launch kernel duration.  Prints ONE JSON line with the headline
TFLOP/s (4*B*H*n*m*d, halved for causal), a roofline object for the
kernel, the other workloads (GB/s and TFLOP/s each against its roofline,
inputs rotated over >= 1 GiB so the 256 MB last-level cache cannot serve
repeats), the workloads of the extended entry points (grouped K/V heads,
ALiBi, the weights output), and the CPU oracle timed on a bounded sample of
the headline workload on this host's cores.  The same leg compares the
oracle with each workload's GPU output on the same input bits (every output
of the smaller workloads, the sampled rows of the headline) and reports the
max-abs error, the bf16 store floor and the oracle's time.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import statistics
import sys
import time

import numpy as np

_ROOT = os.path.dirname(os.path.abspath(__file__))
if _ROOT not in sys.path:
    sys.path.insert(0, _ROOT)

PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, published
PEAK_F32_MFMA_TFLOPS = 157.3   # MI355X fp32 matrix/vector, published
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E, published
KERNEL_SRCS = [os.path.join(_ROOT, "transformer_head_scaled_fwd_amd", "csrc", f)
               for f in ("mha_fwd_kernel.hip", "mha_tiles.h")]
TRAFFIC_FILE = os.path.join(_ROOT, "profiles", "hbm_traffic_causal_n16384_d128.md")
HEADLINE = "causal_n16384_d128"
SECONDARY = "encoder_pad_n128"


def algorithmic_bytes(w, key_lens) -> int:
    """Q read once, O written once, only the valid K and V rows read once,
    the int32 lengths; the score matrix contributes nothing."""
    es = 2 if w.dtype == "bf16" else 4
    kv_rows = w.B * w.m if key_lens is None else int(np.clip(key_lens, 0, w.m).sum())
    return es * (2 * w.B * w.H * w.n * w.d + w.H * kv_rows * 2 * w.d) + \
        (4 * w.B if key_lens is not None else 0)


def valid_pairs(w, key_lens) -> int:
    total = 0
    for b in range(w.B):
        L = w.m if key_lens is None else max(0, min(int(key_lens[b]), w.m))
        if w.causal:
            total += int(np.minimum(np.arange(w.n, dtype=np.int64) + 1, L).sum())
        else:
            total += w.n * L
    return total * w.H


def kernel_code(text: str) -> str:
    """The code of a C++ source without its comments and with every run of
    white space made one blank: what the compiler sees of it."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def kernel_source_hash() -> str:
    """Hash of the forward kernel's code (the kernel file and the shared
    device header it includes), comments and layout excluded, so that a
    profile stays matched to a kernel whose comments alone changed."""
    h = hashlib.sha256()
    for p in KERNEL_SRCS:
        with open(p, encoding="utf-8") as f:
            h.update(kernel_code(f.read()).encode())
    return h.hexdigest()[:16]


def recorded_traffic():
    """HBM bytes per launch from the committed rocprofv3 --pmc summary, or
    None when it is absent or was taken on a different kernel source."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    text = open(TRAFFIC_FILE, encoding="utf-8").read()
    h = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]+)", text)
    t = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not h or not t or h.group(1) != kernel_source_hash():
        return None
    return float(t.group(1))


def device_info(torch):
    p = torch.cuda.get_device_properties(0)
    info = {"name": p.name, "cus": p.multi_processor_count}
    arch = getattr(p, "gcnArchName", None)
    if arch:
        info["arch"] = arch
    clk = getattr(p, "clock_rate", None)
    if clk:
        info["clock_mhz"] = clk / 1000.0
        info["bf16_mfma_tflops_from_props"] = p.multi_processor_count * 4096 * clk * 1e3 / 1e12
    return info


def upload(torch, w, seed_offset=0):
    from transformer_head_scaled_fwd_amd import inputs
    q, k, v, kl = inputs.draw(w.B, w.H, w.n, w.m, w.d, w.d, w.dtype, w.seed + seed_offset,
                              w.lens, w.value_scale)
    dev = "cuda:0"
    kld = None if kl is None else torch.as_tensor(kl).to(dev)
    return (q.to(dev), k.to(dev), v.to(dev), kld, kl), (q, k, v, kl)


def prewarm(torch, launch, stream, ms, max_launches=4000):
    """Untimed launches until `ms` milliseconds of GPU time have passed (or
    max_launches): the device raises its clocks over the first tens of
    milliseconds of sustained work, so a short warmup alone leaves the
    timed launches on the ramp.  Returns (GPU ms spent, launches)."""
    spent, count, batch = 0.0, 0, 4
    while spent < ms and count < max_launches:
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(batch):
            launch(count)
            count += 1
        e1.record(stream)
        e1.synchronize()
        spent += e0.elapsed_time(e1)
        batch = min(2 * batch, 64)
    return spent, count


def time_launches(torch, mha, sets, w, steps, warmup, prewarm_ms=0.0):
    """A time-based pre-warm (prewarm_ms of GPU time), `warmup` untimed
    launches, then `steps` launches cycling over `sets`; per-launch event
    pairs and one pair around the whole region, all on the launch stream.
    Returns (region ms, per-launch ms, first output, (prewarm ms, launches))."""
    stream = torch.cuda.current_stream()
    outs = [torch.empty((w.B, w.H, w.n, w.d), dtype=s[0].dtype, device="cuda:0") for s in sets]

    def launch(i):
        q, k, v, kl, _ = sets[i % len(sets)]
        mha.forward(q, k, v, key_lens=kl, causal=w.causal, scale=w.scale,
                    out=outs[i % len(sets)], stream=stream.cuda_stream)

    pw = prewarm(torch, launch, stream, prewarm_ms) if prewarm_ms > 0 else (0.0, 0)
    for i in range(warmup):
        launch(i)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    for i in range(steps):
        ev[i][0].record(stream)
        launch(i)
        ev[i][1].record(stream)
    t1.record(stream)
    torch.cuda.synchronize()
    per = [a.elapsed_time(b) for a, b in ev]
    return t0.elapsed_time(t1), per, outs[0], pw


def time_graph(torch, mha, sets, w, launches=64, replays=5):
    """GPU-side time per launch of a short workload: `launches` launches
    (cycling over the input sets) captured in one HIP graph and replayed, so
    that host launch overhead does not sit between the kernels.  Every
    replay's outputs are checked bit for bit against eager launches, with
    eager work and a synchronisation between replays.  Returns microseconds
    per launch (best replay)."""
    outs = [torch.empty((w.B, w.H, w.n, w.d), dtype=s[0].dtype, device="cuda:0") for s in sets]

    def launch(i):
        q, k, v, kl, _ = sets[i % len(sets)]
        mha.forward(q, k, v, key_lens=kl, causal=w.causal, scale=w.scale,
                    out=outs[i % len(sets)], stream=torch.cuda.current_stream().cuda_stream)

    for i in range(len(sets)):
        launch(i)
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    with torch.cuda.graph(g, stream=side):
        for i in range(launches):
            launch(i)
    torch.cuda.synchronize()
    best = None
    for _ in range(replays):
        for o in outs:
            o.zero_()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        for o, r in zip(outs, ref):
            if not torch.equal(o, r):
                raise RuntimeError("graph replay differs from the eager launches")
        us = e0.elapsed_time(e1) * 1e3 / launches
        best = us if best is None else min(best, us)
    del g
    return best


def time_graph_ext(torch, launch, outs, launches=32, replays=5):
    """GPU-side time per step of a decode workload (its decode and merge
    launches), captured `launches` steps at a time in one HIP graph over the
    rotating input sets, as a serving loop replays its decode steps.  Every
    replay's outputs are checked bit for bit against eager steps, with eager
    work and a synchronisation between replays.  Returns microseconds per
    step (best replay)."""
    nset = len(outs)
    for i in range(nset):
        launch(i)
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    with torch.cuda.graph(g, stream=side):
        for i in range(launches):
            launch(i)
    torch.cuda.synchronize()
    best = None
    for _ in range(replays):
        for o in outs:
            o.zero_()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        for j in range(min(nset, launches)):
            if not torch.equal(outs[j], ref[j]):
                raise RuntimeError("graph replay differs from the eager steps")
        us = e0.elapsed_time(e1) * 1e3 / launches
        best = us if best is None else min(best, us)
    del g
    return best


def time_copy_floor(torch, nbytes, launches=64, replays=5, rotate_bytes=1 << 30):
    """GPU-side time per launch of a plain device copy that reads nbytes/2 and
    writes nbytes/2 (the same HBM bytes as one attention launch), timed like
    time_graph: `launches` copies over rotating buffers (>= 1 GiB in all, so
    the last-level cache cannot serve repeats) captured in one HIP graph.
    It is the floor a launch of this size meets on this device.  Returns
    microseconds per launch (best replay)."""
    half = max(1, nbytes // 2)
    nbuf = max(2, min(64, -(-rotate_bytes // (2 * half))))
    src = [torch.empty(half, dtype=torch.uint8, device="cuda:0").fill_(i % 251) for i in range(nbuf)]
    dst = [torch.empty(half, dtype=torch.uint8, device="cuda:0") for _ in range(nbuf)]
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    with torch.cuda.graph(g, stream=side):
        for i in range(launches):
            dst[i % nbuf].copy_(src[i % nbuf])
    torch.cuda.synchronize()
    best = None
    for _ in range(replays):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / launches
        best = us if best is None else min(best, us)
    if not torch.equal(dst[0], src[0]):
        raise RuntimeError("copy floor: graph copy produced wrong bytes")
    del g, src, dst
    return best


def bench_workload(torch, mha, name, steps, warmup, rotate_bytes=1 << 30, prewarm_ms=0.0):
    from transformer_head_scaled_fwd_amd import inputs
    w = inputs.WORKLOADS[name]
    first, host = upload(torch, w)
    set_bytes = sum(t.numel() * t.element_size() for t in first[:3]) * 4 // 3
    nsets = max(1, min(64, -(-rotate_bytes // max(set_bytes, 1))))
    sets = [first]
    # Distinct input sets so repeats cannot be served from the last-level cache;
    # the extra sets reuse the first set's key lengths so every launch does
    # the same work.
    for s in range(1, nsets):
        q, k, v = (torch.roll(t, shifts=s, dims=0).contiguous() + 0 for t in first[:3])
        sets.append((q, k, v, first[3], first[4]))
    total_ms, per, out0, pw = time_launches(torch, mha, sets, w, steps, warmup, prewarm_ms)
    out0 = out0.cpu()  # the output of the first input set, the host inputs
    graph_us = time_graph(torch, mha, sets, w) if w.metric_flops() < 1e11 else None
    kl = first[4]
    flops = w.metric_flops()
    useful = 4.0 * w.d * valid_pairs(w, kl)
    abytes = algorithmic_bytes(w, kl)
    copy_us = time_copy_floor(torch, abytes) if graph_us is not None else None
    avg = total_ms / steps
    kern = statistics.mean(per)
    peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_F32_MFMA_TFLOPS
    kname = mha.load().mha_forward_kernel_name(w.B, w.H, w.H, w.n, w.m, w.d,
                                               mha.MHA_BF16 if w.dtype == "bf16" else mha.MHA_F32,
                                               1 if w.causal else 0, 0)
    return {
        "workload": name, "kernel": kname.decode() if kname else None,
        "prewarm_ms": pw[0], "prewarm_launches": pw[1],
        "dtype": w.dtype, "seed": w.seed, "B": w.B, "H": w.H, "n": w.n, "m": w.m,
        "d": w.d, "causal": w.causal, "key_lens": None if w.lens is None else list(w.lens),
        "input_sets": len(sets), "launches": steps,
        "ms_per_launch": avg, "kernel_ms_mean": kern, "kernel_ms_median": statistics.median(per),
        "kernel_ms_min": min(per),
        "tflops": flops / (kern * 1e-3) / 1e12,
        "frac_mfma_peak": flops / (kern * 1e-3) / 1e12 / peak,
        "useful_tflops": useful / (kern * 1e-3) / 1e12,
        "gbps": abytes / (kern * 1e-3) / 1e9,
        "frac_hbm": abytes / (kern * 1e-3) / 1e9 / PEAK_HBM_GBS,
        "algorithmic_bytes": abytes, "metric_flops": flops,
        "graph_us_per_launch": graph_us,
        "graph_gbps": None if graph_us is None else abytes / (graph_us * 1e-6) / 1e9,
        "graph_frac_hbm": None if graph_us is None else
        abytes / (graph_us * 1e-6) / 1e9 / PEAK_HBM_GBS,
        "graph_tflops": None if graph_us is None else flops / (graph_us * 1e-6) / 1e12,
        "copy_floor_us": copy_us,
        "copy_floor_gbps": None if copy_us is None else abytes / (copy_us * 1e-6) / 1e9,
        "graph_frac_copy_floor": None if copy_us is None else copy_us / graph_us,
    }, host, sets, out0


def visible_keys(n, L, causal):
    """Visible keys per query row for one sequence with L filled keys."""
    i = np.arange(n, dtype=np.int64)
    if causal in (False, None):
        return np.full(n, L, dtype=np.int64)
    if causal in (True, "top_left"):
        return np.minimum(i + 1, L)
    return np.clip(i + L - n + 1, 0, L)


def bench_ext(torch, mha, name, steps, warmup, rotate_bytes=1 << 30, prewarm_ms=0.0):
    """One extended workload through mha_forward_ex (plus the weights pass
    when it asks for them), timed like the core workloads: a time-based
    pre-warm, `warmup` untimed launches, then event pairs per launch."""
    from transformer_head_scaled_fwd_amd import inputs
    w = inputs.EXT_WORKLOADS[name]
    dev = "cuda:0"
    q, k, v, kl, sl = inputs.draw_ex(w)
    q, k, v = q.to(dev), k.to(dev), v.to(dev)
    kld = None if kl is None else torch.as_tensor(kl).to(dev)
    sld = None if sl is None else torch.as_tensor(sl).to(dev)
    es = q.element_size()
    set_bytes = (q.numel() + k.numel() + v.numel()) * es * 2
    if w.weights:
        set_bytes += w.B * w.H * w.n * w.m * es
    nsets = max(1, min(32, -(-rotate_bytes // max(set_bytes, 1))))
    sets = [(q, k, v)] + [tuple(torch.roll(t, shifts=s, dims=0).contiguous() + 0
                                for t in (q, k, v)) for s in range(1, nsets)]
    outs = [torch.empty((w.B, w.H, w.n, w.d), dtype=q.dtype, device=dev) for _ in sets]
    lses = [torch.empty((w.B, w.H, w.n), dtype=torch.float32, device=dev) for _ in sets]
    wts = [torch.empty((w.B, w.H, w.n, w.m), dtype=q.dtype, device=dev) for _ in sets] \
        if w.weights else None
    stream = torch.cuda.current_stream()

    code = mha.MHA_BF16 if w.dtype == "bf16" else mha.MHA_F32
    ws_bytes = mha.decode_workspace_size(w.B, w.H, w.H_kv, w.n, w.m, w.d, code) \
        if w.decode else 0
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)

    def launch(i):
        j = i % len(sets)
        a, b, c = sets[j]
        lib = mha.load()
        cur = torch.cuda.current_stream().cuda_stream  # the capturing stream under a graph
        mode = mha.mask_mode(w.causal)
        if w.decode:
            st = lib.mha_decode(a.data_ptr(), b.data_ptr(), c.data_ptr(),
                                None if kld is None else kld.data_ptr(),
                                None if sld is None else sld.data_ptr(), w.scale,
                                outs[j].data_ptr(), None, ws.data_ptr(), ws_bytes,
                                w.B, w.H, w.H_kv, w.n, w.m, w.d, w.d, code, cur)
            assert st == 0, st
            return
        st = lib.mha_forward_ex(a.data_ptr(), b.data_ptr(), c.data_ptr(),
                                None if kld is None else kld.data_ptr(), mode,
                                None if sld is None else sld.data_ptr(), w.scale,
                                outs[j].data_ptr(), lses[j].data_ptr() if w.weights else None,
                                w.B, w.H, w.H_kv, w.n, w.m, w.d, w.d,
                                mha.MHA_BF16 if w.dtype == "bf16" else mha.MHA_F32,
                                cur)
        assert st == 0, st
        if w.weights:
            st = lib.mha_attention_weights(a.data_ptr(), b.data_ptr(),
                                           None if kld is None else kld.data_ptr(), mode,
                                           None if sld is None else sld.data_ptr(), w.scale,
                                           lses[j].data_ptr(), wts[j].data_ptr(), w.B, w.H,
                                           w.H_kv, w.n, w.m, w.d,
                                           mha.MHA_BF16 if w.dtype == "bf16" else mha.MHA_F32,
                                           cur)
            assert st == 0, st

    pw = prewarm(torch, launch, stream, prewarm_ms) if prewarm_ms > 0 else (0.0, 0)
    for i in range(warmup):
        launch(i)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    for i in range(steps):
        ev[i][0].record(stream)
        launch(i)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    per = [a.elapsed_time(b) for a, b in ev]
    kern = statistics.mean(per)
    graph_us = time_graph_ext(torch, launch, outs) if w.decode else None
    pairs = 0
    kv_rows = 0
    for b in range(w.B):
        L = w.m if kl is None else int(np.clip(kl[b], 0, w.m))
        vis = visible_keys(w.n, L, w.causal)
        pairs += int(vis.sum()) * w.H
        kv_rows += int(vis.max()) if w.n else 0
    useful = 4.0 * w.d * pairs
    abytes = es * (2 * w.B * w.H * w.n * w.d + w.H_kv * kv_rows * 2 * w.d)
    if w.weights:
        # the weights pass reads Q and the visible K rows again, writes A
        abytes += es * (w.B * w.H * w.n * w.d + w.H_kv * kv_rows * w.d +
                        w.B * w.H * w.n * w.m) + 2 * 4 * w.B * w.H * w.n
    return {
        "workload": name, "entry": "mha_decode" if w.decode else (
            "mha_forward_ex" + (" + mha_attention_weights" if w.weights else "")),
        "workspace_bytes": ws_bytes, "prewarm_ms": pw[0], "prewarm_launches": pw[1],
        "dtype": w.dtype, "B": w.B, "H": w.H, "H_kv": w.H_kv, "n": w.n, "m": w.m, "d": w.d,
        "causal": w.causal, "alibi": w.alibi, "key_lens": None if w.lens is None else list(w.lens),
        "input_sets": len(sets), "launches": steps,
        "kernel_ms_mean": kern, "kernel_ms_median": statistics.median(per),
        "kernel_ms_min": min(per),
        "useful_tflops": useful / (kern * 1e-3) / 1e12,
        "frac_mfma_peak": useful / (kern * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
        "gbps": abytes / (kern * 1e-3) / 1e9,
        "frac_hbm": abytes / (kern * 1e-3) / 1e9 / PEAK_HBM_GBS,
        "graph_us_per_step": graph_us,
        "graph_gbps": None if graph_us is None else abytes / (graph_us * 1e-6) / 1e9,
        "graph_frac_hbm": None if graph_us is None else
        abytes / (graph_us * 1e-6) / 1e9 / PEAK_HBM_GBS,
        "algorithmic_bytes": abytes, "useful_flops": useful,
    }


def bench_layer(torch, mha, name, steps, warmup, rotate_bytes=1 << 30, prewarm_ms=0.0):
    """One multi-head layer workload through mha_multihead_forward: the
    Q/K/V projections, the core and the output projection, timed together
    with HIP events on the launch stream after a time-based pre-warm."""
    from transformer_head_scaled_fwd_amd import inputs
    w = inputs.LAYER_WORKLOADS[name]
    dev = "cuda:0"
    x, _, _, Ws, bs, kl = inputs.draw_layer(w)
    x = x.to(dev)
    Ws = [t.to(dev) for t in Ws]
    bs = [t.to(dev) for t in bs]
    kld = None if kl is None else torch.as_tensor(kl).to(dev)
    es = x.element_size()
    nsets = max(1, min(32, -(-rotate_bytes // (x.numel() * es * 2))))
    xs = [x] + [torch.roll(x, shifts=s, dims=0).contiguous() + 0 for s in range(1, nsets)]
    ys = [torch.empty_like(x) for _ in xs]
    code = mha.MHA_BF16 if w.dtype == "bf16" else mha.MHA_F32
    need = mha.multihead_workspace_size(w.B, w.n, w.n, w.d_model, w.H, code)
    ws = torch.empty(need, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    lib = mha.load()
    mode = mha.mask_mode(w.causal)
    scale = mha.default_scale(w.d_model // w.H)

    def launch(i):
        j = i % len(xs)
        p = xs[j].data_ptr()
        st = lib.mha_multihead_forward(
            p, p, p, Ws[0].data_ptr(), bs[0].data_ptr(), Ws[1].data_ptr(), bs[1].data_ptr(),
            Ws[2].data_ptr(), bs[2].data_ptr(), Ws[3].data_ptr(), bs[3].data_ptr(),
            None if kld is None else kld.data_ptr(), mode, scale, ys[j].data_ptr(), None,
            ws.data_ptr(), need, w.B, w.n, w.n, w.d_model, w.H, code, stream.cuda_stream)
        assert st == 0, st

    pw = prewarm(torch, launch, stream, prewarm_ms) if prewarm_ms > 0 else (0.0, 0)
    for i in range(warmup):
        launch(i)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    for i in range(steps):
        ev[i][0].record(stream)
        launch(i)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    per = [a.elapsed_time(b) for a, b in ev]
    kern = statistics.mean(per)
    dk = w.d_model // w.H
    proj_flops = 4 * 2.0 * w.B * w.n * w.d_model * w.d_model
    pairs = 0
    for b in range(w.B):
        L = w.n if kl is None else int(np.clip(kl[b], 0, w.n))
        pairs += int(visible_keys(w.n, L, w.causal).sum()) * w.H
    core_flops = 4.0 * dk * pairs
    return {
        "workload": name, "entry": "mha_multihead_forward", "dtype": w.dtype, "B": w.B,
        "n": w.n, "d_model": w.d_model, "H": w.H, "causal": w.causal,
        "prewarm_ms": pw[0], "prewarm_launches": pw[1],
        "key_lens": None if w.lens is None else list(w.lens), "input_sets": len(xs),
        "launches": steps, "layer_ms_mean": kern, "layer_ms_median": statistics.median(per),
        "layer_ms_min": min(per),
        "useful_tflops": (proj_flops + core_flops) / (kern * 1e-3) / 1e12,
        "frac_mfma_peak": (proj_flops + core_flops) / (kern * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
        "projection_flops": proj_flops, "core_useful_flops": core_flops,
    }


def cpu_baseline(w, host, max_s):
    """The oracle as it stands, timed on this host's cores over the whole
    headline workload (every query row of every head), its result kept for
    the parity check.  A probe on 64 rows first estimates the full run; only
    if that estimate exceeds max_s seconds does it fall back to distinct
    rows drawn without replacement, as many as fit in max_s / 4."""
    import oracle
    q, k, v, kl = host
    Q, K, V = oracle.to_f64(q), oracle.to_f64(k), oracle.to_f64(v)
    total_rows = w.B * w.H * w.n
    rng = np.random.Generator(np.random.PCG64(2024))

    def rows_of(flat):
        flat = np.sort(flat)
        b, rem = np.divmod(flat, w.H * w.n)
        t, i = np.divmod(rem, w.n)
        return np.stack([b, t, i], 1).astype(np.int64)

    def work(rows):
        keys = rows[:, 2] + 1 if w.causal else np.full(len(rows), w.m)
        if kl is not None:
            keys = np.minimum(keys, np.asarray(kl)[rows[:, 0]])
        return 4.0 * w.d * float(np.maximum(keys, 0).sum())

    probe = rows_of(rng.choice(total_rows, size=min(64, total_rows), replace=False))
    t = time.perf_counter()
    oracle.attention_rows(Q, K, V, probe, key_lens=kl, causal=w.causal, scale=w.scale)
    dt = max(time.perf_counter() - t, 1e-3)
    rate = work(probe) / dt
    all_rows = rows_of(np.arange(total_rows))
    full_work = work(all_rows)
    if full_work / rate <= max_s:
        t = time.perf_counter()
        ref = oracle.attention(Q, K, V, key_lens=kl, causal=w.causal, scale=w.scale)
        dt = time.perf_counter() - t
        rows, f = None, full_work
        sample = ("all %d query rows of the %d heads of %s (the whole workload); useful FLOPs "
                  "4*d*(valid keys) per row; fp64 on the host cores" % (total_rows, w.B * w.H, w.name))
    else:
        target = int(total_rows * (max_s / 4.0) / (full_work / rate))
        rows = rows_of(rng.choice(total_rows, size=max(64, min(target, total_rows)),
                                  replace=False))
        t = time.perf_counter()
        ref = oracle.attention_rows(Q, K, V, rows, key_lens=kl, causal=w.causal, scale=w.scale)
        dt = time.perf_counter() - t
        f = work(rows)
        sample = ("%d distinct query rows drawn without replacement (seeded) from the %d of %s; "
                  "useful FLOPs 4*d*(valid keys) per row; fp64 on the host cores"
                  % (len(rows), total_rows, w.name))
    return {"value": f / dt / 1e12, "unit": "TFLOP/s", "cores": oracle.threads(),
            "kind": "oracle", "seconds": dt, "probe_rate_tflops": rate / 1e12,
            "sample": sample}, rows, ref, dt


TOL = {"f32": 1e-5, "bf16": 1.5e-2}


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo", encoding="utf-8") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def parity(w, host, out, rows=None, ref=None, oracle_s=None):
    """The oracle (timed on this host's cores) against the GPU output of the
    same input bits: max-abs error over every element (the oracle's full
    result `ref`, or a fresh oracle run when it is None), or over the
    sampled rows `rows` with the oracle's result `ref` for them."""
    import oracle
    q, k, v, kl = host
    if ref is None:
        t = time.perf_counter()
        ref = oracle.attention(q, k, v, key_lens=kl, causal=w.causal, scale=w.scale)
        oracle_s = time.perf_counter() - t
    if rows is None:
        got = oracle.to_f64(out)
        compared = "all %d outputs" % got.size
    else:
        import torch
        r = torch.from_numpy(rows)
        got = oracle.to_f64(out[r[:, 0], r[:, 1], r[:, 2]])
        compared = "%d sampled rows" % len(rows)
    err = np.abs(got - ref)
    floor = None
    if w.dtype == "bf16":
        import torch
        r32 = torch.from_numpy(np.ascontiguousarray(ref, dtype=np.float32))
        floor = float(np.abs(r32.to(torch.bfloat16).double().numpy() - ref).max())
    mx = float(err.max()) if err.size else 0.0
    at = [int(x) for x in np.unravel_index(np.argmax(err), err.shape)] if err.size else []
    if rows is not None and at:
        at = [int(x) for x in rows[at[0]]] + at[1:]  # (b, head, row, column)
    return {"compared": compared, "max_abs_err": mx, "max_at": at,
            "mean_abs_err": float(err.mean()) if err.size else 0.0,
            "store_floor": floor, "tol": TOL[w.dtype], "pass": bool(mx <= TOL[w.dtype]),
            "oracle_s": oracle_s, "oracle_threads": oracle.threads(), "cpu_model": cpu_model()}


def calibrate_copy(torch, nbytes):
    """A plain device copy of known size, for scaling HBM byte counters."""
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibrate_copy_bytes": nbytes, "launches": 3}), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--workload", default=HEADLINE)
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle baseline")
    ap.add_argument("--no-others", action="store_true", help="skip the other workloads")
    ap.add_argument("--cpu-max-seconds", type=float, default=150.0,
                    help="longest oracle run the baseline takes on the whole headline workload "
                         "before it samples rows instead")
    ap.add_argument("--prewarm-ms", type=float, default=500.0,
                    help="GPU time of untimed headline launches before the warmup steps")
    ap.add_argument("--prewarm-others-ms", type=float, default=200.0,
                    help="time-based pre-warm before each other workload's timed launches")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="BYTES")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the attention kernel runs on one "
              "device and no multi-GPU path is built (asked for --gpus %d, "
              "WORLD_SIZE=%d)" % (args.gpus, world), file=sys.stderr)
        sys.exit(2)

    import torch
    import transformer_head_scaled_fwd_amd as mha
    from transformer_head_scaled_fwd_amd import inputs
    mha.load()
    if args.calibrate_copy:
        calibrate_copy(torch, args.calibrate_copy)
        return

    if args.workload not in inputs.WORKLOADS:
        # One extended or multi-head-layer workload alone (for profiling):
        # its record, timed like the extended list of the full run.
        if args.workload in inputs.EXT_WORKLOADS:
            rec = bench_ext(torch, mha, args.workload, args.steps, args.warmup,
                            prewarm_ms=args.prewarm_others_ms)
        elif args.workload in inputs.LAYER_WORKLOADS:
            rec = bench_layer(torch, mha, args.workload, args.steps, args.warmup,
                              prewarm_ms=args.prewarm_others_ms)
        else:
            ap.error("unknown workload %r" % args.workload)
        print(json.dumps(rec), flush=True)
        return
    w = inputs.WORKLOADS[args.workload]
    print("bench: %s steps=%d warmup=%d" % (w.name, args.steps, args.warmup),
          file=sys.stderr, flush=True)
    head, host, _, head_out = bench_workload(torch, mha, w.name, args.steps, args.warmup,
                                             prewarm_ms=args.prewarm_ms)
    others = []
    checks = []  # (workload, host inputs, GPU output) for the oracle comparison
    if not args.no_others:
        for name in inputs.ORDER:
            if name == w.name:
                continue
            print("bench: %s" % name, file=sys.stderr, flush=True)
            res, o_host, sets, o_out = bench_workload(torch, mha, name, 200, 20,
                                                      prewarm_ms=args.prewarm_others_ms)
            del sets
            others.append(res)
            checks.append((inputs.WORKLOADS[name], o_host, o_out, res))
            torch.cuda.empty_cache()
    ext = []
    if not args.no_others:
        for name in inputs.EXT_ORDER:
            print("bench: %s" % name, file=sys.stderr, flush=True)
            ext.append(bench_ext(torch, mha, name, 100, 20, prewarm_ms=args.prewarm_others_ms))
            torch.cuda.empty_cache()
        for name in inputs.LAYER_ORDER:
            print("bench: %s" % name, file=sys.stderr, flush=True)
            ext.append(bench_layer(torch, mha, name, 100, 20, prewarm_ms=args.prewarm_others_ms))
            torch.cuda.empty_cache()
    traffic = recorded_traffic() if w.name == HEADLINE else None
    cpu = None
    if not args.no_cpu:
        print("bench: cpu baseline (oracle)", file=sys.stderr, flush=True)
        cpu, rows, ref, dt = cpu_baseline(w, host, args.cpu_max_seconds)
        head["parity"] = parity(w, host, head_out, rows=rows, ref=ref, oracle_s=dt)
        for wk, o_host, o_out, res in checks:
            print("bench: oracle parity %s" % wk.name, file=sys.stderr, flush=True)
            res["parity"] = parity(wk, o_host, o_out)
    bf16 = w.dtype == "bf16"
    peak = PEAK_BF16_TFLOPS if bf16 else PEAK_F32_MFMA_TFLOPS
    kern_s = head["kernel_ms_mean"] * 1e-3
    achieved = head["metric_flops"] / kern_s / 1e12
    sec = next((o for o in others if o["workload"] == SECONDARY), None)
    line = {
        "metric": "attention fwd TFLOP/s and % bf16 MFMA peak (causal n=16384, d=128); "
                  "GB/s at n=128",
        "value": head["metric_flops"] / (head["ms_per_launch"] * 1e-3) / 1e12,
        "unit": "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "prewarm_ms": head["prewarm_ms"], "prewarm_launches": head["prewarm_launches"],
        "ms_per_step": head["ms_per_launch"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if bf16 else "f32", "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "n": w.n, "m": w.m, "d": w.d,
                   "causal": w.causal, "key_lens": None if w.lens is None else list(w.lens),
                   "values": "N(0,1)*%g, seed %d" % (w.value_scale, w.seed)},
        "frac_mfma_peak": head["frac_mfma_peak"],
        "gbps_n128": None if sec is None else (sec["graph_gbps"] or sec["gbps"]),
        "frac_hbm_n128": None if sec is None else (sec["graph_frac_hbm"] or sec["frac_hbm"]),
        "gbps_n128_method": "HIP graph of 64 back-to-back launches over rotating input sets, "
                            "replays checked bit for bit against eager launches; per-launch "
                            "event timing (host launch gaps included) in workloads[].gbps",
        "copy_floor_gbps_n128": None if sec is None else sec["copy_floor_gbps"],
        "frac_copy_floor_n128": None if sec is None else sec["graph_frac_copy_floor"],
        "roofline": {"bound": "mfma" if bf16 else "alu", "achieved": achieved, "peak": peak,
                     "unit": "TFLOP/s", "frac": achieved / peak, "traffic": traffic,
                     "kernel": head["kernel"],
                     "kernel_ms_mean": head["kernel_ms_mean"],
                     "kernel_ms_median": head["kernel_ms_median"],
                     "kernel_source_sha256_16": kernel_source_hash(),
                     "flops_per_launch": head["metric_flops"]},
        "cpu_baseline": cpu,
        "parity_all_pass": None if cpu is None else
        all(r["parity"]["pass"] for r in [head] + others if "parity" in r),
        "workloads": [head] + others,
        "extended": ext,
        "device": device_info(torch),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
