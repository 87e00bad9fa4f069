#!/usr/bin/env python3
"""Benchmark of the decode matrix-vector path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--quick] [--no-cpu]
                    [--only dense,q4,w4a16,lmhead,moe256,moe512,moe512v]
                    [--profile WORKLOAD]  (one workload's graph, for rocprofv3 counter runs)
                    [--summarize-counters FETCH_DIR WRITE_DIR]  (counter CSVs -> markdown)
                    [--summarize-trace TRACE_DIR]  (kernel-trace CSV -> markdown)

The headline step is one pass over the dense BF16 decode matvec set: 36 layer
copies (5.85 GB, far past the 256 MB Infinity Cache) of attn-out 2560x2560,
fused gate+up 2 x 9728x2560 and down 2560x9728, batch 1, each matrix with
its own synthetic N(0,1) activation row, captured in one HIP graph and
replayed K times.  `value` is algorithmic bytes / time in GB/s over exactly
K replays.  Every timed quantity is also sampled 7 times (K replays each):
mean, Student-t 95% interval and coefficient of variation (flagged above
5%).  The same JSON line carries the other workloads (B = 8 dense, Q4_0 x
Q8_1, W4A16, the 248320 x 2560 LM head with its argmax, the 256- and
512-expert MoE layers), tokens/s equivalents, the dependent-launch floor,
the roofline of the dominant kernel, the read probe, a manifest, a GPU
contention check and the CPU oracle's throughput on bounded samples of the
five workloads (single-threaded and on every core of the host's share).
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import math
import os
import platform
import re
import sys
import threading
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0
METRIC = ("achieved HBM GB/s (% of MI355X peak) for batch-1 GEMV; MoE layer µs/token")
REPS = 7               # samples per timed quantity
CV_FLAG = 0.05         # coefficient of variation above which a sample set is flagged


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# ---------------------------------------------------------------------------
# timing helpers
# ---------------------------------------------------------------------------

def capture(fn):
    """Capture fn's launches into a HIP graph (warm-up run first, eagerly)."""
    import torch
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def time_replays(run, steps):
    """Seconds per call of run() over `steps` calls, bracketed by
    synchronize and events on the current stream (the graphs replay on it)."""
    import torch
    torch.cuda.synchronize()
    st = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(st)
    for _ in range(steps):
        run()
    e1.record(st)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / 1e3 / steps


def sample(run, steps, warmup, reps=REPS):
    """reps samples of seconds per call, each over `steps` calls."""
    for _ in range(warmup):
        run()
    return [time_replays(run, steps) for _ in range(reps)]


def stats(samples, scale=1.0):
    """mean, Student-t 95% half-width, coefficient of variation of samples*scale."""
    from scipy import stats as st
    x = [s * scale for s in samples]
    n = len(x)
    m = sum(x) / n
    sd = math.sqrt(sum((v - m) ** 2 for v in x) / (n - 1)) if n > 1 else 0.0
    half = st.t.ppf(0.975, n - 1) * sd / math.sqrt(n) if n > 1 else float("nan")
    cv = sd / m if m else float("nan")
    return dict(mean=m, ci95=half, cv=cv, cv_flag=bool(cv > CV_FLAG), n=n)


def timed_graph(g, steps, warmup):
    """(samples, stats) for replays of graph g."""
    s = sample(g.replay, steps, warmup)
    return s, stats(s)


# ---------------------------------------------------------------------------
# dense BF16
# ---------------------------------------------------------------------------

DENSE_SHAPES = {"attn_out": (2560, 2560), "gate_up": (2 * 9728, 2560), "down": (2560, 9728)}


def dense_bytes(B):
    return sum(2 * N * K + 4 * B * K + 4 * B * N for N, K in DENSE_SHAPES.values())


def build_dense(dev, layers):
    import torch
    import synth
    W = {}
    for name, (N, K) in DENSE_SHAPES.items():
        one = synth.bf16_weights(N, K, 0, "dense", name, device=dev)
        W[name] = torch.empty((layers, N, K), dtype=torch.bfloat16, device=dev)
        W[name][:] = one          # replicate: every layer copy holds its own bytes
        del one
    return W


def dense_section(mm, dev, W, layers, B, steps, warmup, eager=False):
    """One graph over every layer copy; `head` also times exactly `steps`
    replays on their own (the headline measurement).  The pass is one
    dependency chain: attn-out reads the previous layer's down output, gate+up
    reads attn-out's output, down reads the gate half of gate+up's output
    (the elementwise SiLU(gate) * up between them is not part of this set)."""
    import torch
    import synth
    x0 = synth.activations(B, DENSE_SHAPES["attn_out"][1], 0, "dense-x", B, device=dev)
    Y = {n: torch.empty((layers, B, N), device=dev) for n, (N, K) in DENSE_SHAPES.items()}
    n_gate = DENSE_SHAPES["down"][1]

    def step():
        for l in range(layers):
            x = x0 if l == 0 else Y["down"][l - 1]
            mm.gemv_bf16(W["attn_out"][l], x, out=Y["attn_out"][l])
            mm.gemv_bf16(W["gate_up"][l], Y["attn_out"][l], out=Y["gate_up"][l])
            mm.gemv_bf16(W["down"][l], Y["gate_up"][l][:, :n_gate], out=Y["down"][l])
    g = capture(step)
    for _ in range(warmup):
        g.replay()
    t_head = time_replays(g.replay, steps)          # exactly `steps` replays
    samples = [t_head] + [time_replays(g.replay, steps) for _ in range(REPS - 1)]
    st = stats(samples, 1e6 / layers)
    t = t_head
    nbytes = layers * dense_bytes(B)
    res = dict(B=B, layers=layers, launches_per_layer=3, s_per_step=t,
               us_per_layer=t / layers * 1e6, us_per_layer_stats=st,
               GBps=nbytes / t / 1e9, GBps_mean=nbytes / (st["mean"] * layers / 1e6) / 1e9,
               frac_of_peak=nbytes / t / 1e9 / PEAK_HBM_GBPS, bytes_per_step=nbytes,
               tokens_per_s_equiv=B / t)
    if eager:  # the same pass launched from the host one call at a time, no graph
        te = sample(step, 3, 1, reps=3)
        res["eager_us_per_layer"] = stats(te, 1e6 / layers)
    return res


def dominant_kernel(mm, dev, W, layers, steps, warmup):
    """The gate+up GEMV (19456 x 2560, 61% of the dense bytes) alone: its
    launches back to back in one graph; average duration per launch."""
    import torch
    import synth
    N, K = DENSE_SHAPES["gate_up"]
    X = synth.activations(layers, K, 0, "dom-x", device=dev).view(layers, 1, K)
    Y = torch.empty((layers, 1, N), device=dev)

    def step():
        for l in range(layers):
            mm.gemv_bf16(W["gate_up"][l], X[l], out=Y[l])
    g = capture(step)
    s, st = timed_graph(g, steps, warmup)
    t = st["mean"] / layers
    per_launch = 2 * N * K + 4 * K + 4 * N
    return dict(kernel="k_gemv_bf16_xl<1, 5, 8, 1, 5> (gate+up 19456x2560, B=1)", s_per_launch=t,
                us_per_launch_stats=stats(s, 1e6 / layers),
                bytes_per_launch=per_launch, GBps=per_launch / t / 1e9)


def dense_per_matrix(mm, dev, W, layers, B, steps, warmup):
    """Each dense shape alone: its `layers` launches (one per layer copy,
    independent inputs) back to back in one graph; us and GB/s per launch."""
    import torch
    import synth
    out = {}
    for name, (N, K) in DENSE_SHAPES.items():
        X = synth.activations(layers * B, K, 0, "mat-x", name, B, device=dev).view(layers, B, K)
        Y = torch.empty((layers, B, N), device=dev)

        def step():
            for l in range(layers):
                mm.gemv_bf16(W[name][l], X[l], out=Y[l])
        g = capture(step)
        s, st = timed_graph(g, steps, warmup)
        t = st["mean"] / layers
        nbytes = 2 * N * K + 4 * B * K + 4 * B * N
        out[name] = dict(N=N, K=K, us_per_launch_stats=stats(s, 1e6 / layers),
                         GBps=nbytes / t / 1e9, frac_of_peak=nbytes / t / 1e9 / PEAK_HBM_GBPS)
        del g
    return out


def cache_resident(mm, dev, W, reps, steps, warmup):
    """Copy scaling: one layer copy of the dense set (162 MB, within the 256 MB
    Infinity Cache) run `reps` times per graph, against the 36-copy pass; and
    the 1024 x 1024 correctness shape (2 MiB, in L2).  Both are flagged
    cache-resident: they show what the copies defeat, not HBM speed."""
    import torch
    import synth
    x0 = synth.activations(1, DENSE_SHAPES["attn_out"][1], 0, "cache-x", device=dev)
    Y = {n: torch.empty((1, N), device=dev) for n, (N, K) in DENSE_SHAPES.items()}
    n_gate = DENSE_SHAPES["down"][1]

    def step():
        for r in range(reps):
            mm.gemv_bf16(W["attn_out"][0], x0 if r == 0 else Y["down"], out=Y["attn_out"])
            mm.gemv_bf16(W["gate_up"][0], Y["attn_out"], out=Y["gate_up"])
            mm.gemv_bf16(W["down"][0], Y["gate_up"][:, :n_gate], out=Y["down"])
    g = capture(step)
    s, st = timed_graph(g, steps, warmup)
    t = st["mean"] / reps
    one = dict(reps=reps, us_per_layer_stats=stats(s, 1e6 / reps), GBps=dense_bytes(1) / t / 1e9,
               cache_resident=True)
    del g
    W1 = synth.bf16_weights(1024, 1024, 0, "c1", device=dev)
    x1 = synth.activations(1, 1024, 0, "c1", device=dev)
    y1 = torch.empty((1, 1024), device=dev)

    def step1():
        for _ in range(reps):
            mm.gemv_bf16(W1, x1, out=y1)
    g = capture(step1)
    s, st = timed_graph(g, steps, warmup)
    t = st["mean"] / reps
    nb = 2 * 1024 * 1024 + 4 * 1024 + 4 * 1024
    c1 = dict(shape="1024x1024, B=1", us_per_launch_stats=stats(s, 1e6 / reps),
              GBps=nb / t / 1e9, cache_resident=True)
    return one, c1


def launch_floor(mm, dev, steps, warmup, n=200):
    """Time per dependent launch of a one-workgroup kernel (quantize_q8_1 of
    32 values) in a graph of n of them: the fixed cost each launch of a
    decode pass pays before its own work."""
    import torch
    x = torch.ones((1, 32), device=dev)
    q = torch.empty(mm.q8_1_bytes(32, 1), dtype=torch.uint8, device=dev)

    def step():
        for _ in range(n):
            mm.quantize_q8_1(x, out=q)
    g = capture(step)
    s, st = timed_graph(g, max(2, steps // 4), warmup)
    return dict(kernel="k_quantize_q8_1, 1 workgroup", launches_per_graph=n,
                us_per_launch=stats(s, 1e6 / n))


# ---------------------------------------------------------------------------
# Q4_0 x Q8_1
# ---------------------------------------------------------------------------

Q4_SHAPES = [(4096, 4096), (11008, 4096)]


def q4_bytes(B):
    return sum(N * K // 32 * 18 + 4 * B * K + 4 * B * N for N, K in Q4_SHAPES)


def q4_mats(mm, dev, copies):
    import torch
    import synth
    mats = []
    for N, K in Q4_SHAPES:
        qs1, d1 = synth.q4_0_weights(N, K, 0, "q4bench", N, device=dev)
        qs = torch.empty((copies,) + tuple(qs1.shape), dtype=torch.uint8, device=dev)
        d = torch.empty((copies,) + tuple(d1.shape), dtype=torch.float16, device=dev)
        qs[:] = qs1
        d[:] = d1
        mats.append((qs, d))
    Ws = [[mm.Q4_0(qs[c], d[c]) for (qs, d) in mats] for c in range(copies)]
    return mats, Ws


def q4_section(mm, dev, copies, B, steps, warmup, graph_only=False):
    import torch
    import synth
    mats, Ws = q4_mats(mm, dev, copies)
    K = Q4_SHAPES[0][1]
    X = synth.activations(copies * B, K, 0, "q4bench-x", B, device=dev).view(copies, B, K)
    Ys = [[torch.empty((B, N), device=dev) for N, _ in Q4_SHAPES] for _ in range(copies)]
    # B = 1: Q8_1 quantization inside every workgroup of the product (one
    # launch); B >= 2: one quantization pass per product into a scratch
    # buffer, then the product (two launches; each product quantizes its
    # own activations, none is shared)
    xq = torch.empty(mm.q8_1_bytes(K, B), dtype=torch.uint8, device=dev) if B > 1 else None

    def step():
        for c in range(copies):
            for i, W in enumerate(Ws[c]):
                mm.gemv_q4_0(W, x=X[c], xq=xq, out=Ys[c][i])
    g = capture(step)
    if graph_only:
        return g, (mats, Ws, X, Ys, xq)
    s, st = timed_graph(g, steps, warmup)
    t = st["mean"]
    nbytes = copies * q4_bytes(B)
    del mats, Ws
    return dict(B=B, copies=copies, act_quant="in-kernel" if B == 1 else "separate pass",
                launches_per_copy=len(Q4_SHAPES) * (1 if B == 1 else 2),
                stored_GB=copies * sum(N * K // 32 * 18 for N, K in Q4_SHAPES) / 1e9,
                s_per_step=t, us_per_copy=t / copies * 1e6,
                us_per_copy_stats=stats(s, 1e6 / copies), GBps=nbytes / t / 1e9,
                frac_of_peak=nbytes / t / 1e9 / PEAK_HBM_GBPS,
                tokens_per_s_equiv=B / (t / copies * 32))


def w4a16_section(mm, dev, copies, B, steps, warmup, graph_only=False):
    """The Q4_0 shapes with fp32 activations (no Q8_1 step): one launch per
    product at every B."""
    import torch
    import synth
    mats, Ws = q4_mats(mm, dev, copies)
    K = Q4_SHAPES[0][1]
    X = synth.activations(copies * B, K, 0, "w4a16bench-x", B, device=dev).view(copies, B, K)
    Ys = [[torch.empty((B, N), device=dev) for N, _ in Q4_SHAPES] for _ in range(copies)]

    def step():
        for c in range(copies):
            for i, W in enumerate(Ws[c]):
                mm.gemv_q4_0_f32(W, X[c], out=Ys[c][i])
    g = capture(step)
    if graph_only:
        return g, (mats, Ws, X, Ys)
    s, st = timed_graph(g, steps, warmup)
    t = st["mean"]
    nbytes = copies * q4_bytes(B)
    del mats, Ws
    return dict(B=B, copies=copies, launches_per_copy=len(Q4_SHAPES), s_per_step=t,
                us_per_copy=t / copies * 1e6, us_per_copy_stats=stats(s, 1e6 / copies),
                GBps=nbytes / t / 1e9, frac_of_peak=nbytes / t / 1e9 / PEAK_HBM_GBPS)


# ---------------------------------------------------------------------------
# LM head: BF16 GEMV over the vocabulary, then argmax on the device
# ---------------------------------------------------------------------------

LM_VOCAB, LM_HID = 248320, 2560


def lm_head_section(mm, dev, Bs, steps, warmup):
    import torch
    import synth
    W = synth.bf16_weights(LM_VOCAB, LM_HID, 0, "lm_head", device=dev)   # 1.27 GB
    res = dict(vocab=LM_VOCAB, hidden=LM_HID, weight_GB=W.numel() * 2 / 1e9)
    reps = 16  # argmax alone: this many calls per graph, so the replay is not host-bound
    for B in Bs:
        X = synth.activations(B, LM_HID, 0, "lm_head", B, device=dev)
        Y = torch.empty((B, LM_VOCAB), device=dev)
        Ys = synth.normal((reps, B, LM_VOCAB), 1.0, 0, "lm_logits", B, device=dev)
        ids = torch.empty(B, dtype=torch.int32, device=dev)
        vals = torch.empty(B, device=dev)
        ws = torch.empty(mm.argmax_workspace_bytes(LM_VOCAB, B), dtype=torch.uint8, device=dev)
        gemv = lambda: mm.gemv_bf16(W, X, out=Y)

        def amax():
            for r in range(reps):
                mm.argmax_rows(Ys[r], ids=ids, vals=vals, workspace=ws)

        def both():
            gemv()
            mm.argmax_rows(Y, ids=ids, vals=vals, workspace=ws)
        sg, stg = timed_graph(capture(gemv), steps, warmup)
        sa, sta = timed_graph(capture(amax), steps, warmup)
        sb, stb = timed_graph(capture(both), steps, warmup)
        t_g, t_a, t_b = stg["mean"], sta["mean"] / reps, stb["mean"]
        gbytes = 2 * LM_VOCAB * LM_HID + 4 * B * LM_HID + 4 * B * LM_VOCAB
        res[f"B{B}"] = dict(us_gemv=t_g * 1e6, us_gemv_stats=stats(sg, 1e6),
                            us_argmax=t_a * 1e6, us_gemv_argmax=t_b * 1e6,
                            us_gemv_argmax_stats=stats(sb, 1e6),
                            gemv_GBps=gbytes / t_g / 1e9,
                            gemv_frac_of_peak=gbytes / t_g / 1e9 / PEAK_HBM_GBPS,
                            argmax_GBps=4 * B * LM_VOCAB / t_a / 1e9,
                            bytes_to_host_per_token=4)
        del X, Y, Ys, ids, vals, ws
    del W
    torch.cuda.empty_cache()
    return res


# ---------------------------------------------------------------------------
# MoE layers
# ---------------------------------------------------------------------------

MOE_LAYERS = {256: 40, 512: 48}   # layer copies of the two MoE configurations


def moe_launches(B, H):
    if B <= 2:
        return 3
    if B <= 8:
        return 5
    return 6 if H in (1024, 2048) else 5 + (B + 7) // 8


def moe_build(mm, dev, E, k, layers, H=2048, I=512):
    import torch
    import synth
    t1 = synth.moe_layer_tensors(E, H, I, 0, "moebench", E, device=dev)

    def rep(a):
        out = torch.empty((layers,) + tuple(a.shape), dtype=a.dtype, device=dev)
        out[:] = a
        return out
    big = {n: rep(t1[n]) for n in ("router", "gate_qs", "gate_d", "up_qs", "up_d",
                                   "down_qs", "down_d")}
    sh = {n: rep(v) for n, v in t1["shared"].items()}
    del t1
    lay = [mm.MoeLayer(big["router"][l], big["gate_qs"][l], big["gate_d"][l], big["up_qs"][l],
                       big["up_d"][l], big["down_qs"][l], big["down_d"][l], k,
                       shared={n: v[l] for n, v in sh.items()}) for l in range(layers)]
    return lay, (big, sh)


def moe_graph(mm, dev, lay, E, k, B, H=2048):
    import torch
    import synth
    layers = len(lay)
    X = synth.activations(layers * B, H, 0, "moebench-x", E, B, device=dev).view(layers, B, H)
    Y = torch.empty((layers, B, H), device=dev)
    ids = torch.empty((layers, B, k), dtype=torch.int32, device=dev)
    ws = torch.empty((layers, mm.moe_workspace_bytes(lay[0], B)), dtype=torch.uint8,
                     device=dev)

    def step():
        for l in range(layers):
            mm.moe_layer_decode(lay[l], X[l], out=Y[l], workspace=ws[l], ids=ids[l])
    return capture(step), (X, Y, ids, ws)


def moe_section(mm, dev, E, k, layers, Bs, steps, warmup, H=2048, I=512):
    import torch
    lay, keep = moe_build(mm, dev, E, k, layers, H, I)
    expert_bytes = lay[0].expert_bytes()
    stored = layers * (E * H * 4 + (E + 1) * expert_bytes)
    res = dict(E=E, k=k, shared=1, H=H, I=I, layers=layers, stored_GB=stored / 1e9)
    for B in Bs:
        g, bufs = moe_graph(mm, dev, lay, E, k, B, H)
        s, st = timed_graph(g, steps, warmup)
        t = st["mean"]
        idn = bufs[2].cpu().numpy()
        uniq = [len(set(idn[l].ravel().tolist())) for l in range(layers)]
        nbytes = sum(E * H * 4 + 4 * B * H * 2 + (u + 1) * expert_bytes for u in uniq)
        n_cfg = MOE_LAYERS.get(E, layers)
        res[f"B{B}"] = dict(us_per_layer=t / layers * 1e6,
                            us_per_layer_stats=stats(s, 1e6 / layers),
                            us_per_layer_per_token=t / layers / B * 1e6,
                            mean_unique_experts=sum(uniq) / layers,
                            MB_per_layer=nbytes / layers / 1e6, GBps=nbytes / t / 1e9,
                            frac_of_peak=nbytes / t / 1e9 / PEAK_HBM_GBPS,
                            launches_per_layer=moe_launches(B, H),
                            launches_per_token=moe_launches(B, H) * n_cfg / B,
                            tokens_per_s_equiv=B / (t / layers * n_cfg))
        del g, bufs
    if len(Bs) > 1 and 1 in Bs:
        res["ratio_Bmax_B1_time"] = res[f"B{max(Bs)}"]["us_per_layer"] / res["B1"]["us_per_layer"]
    del lay, keep
    torch.cuda.empty_cache()
    return res


# ---------------------------------------------------------------------------
# read probe
# ---------------------------------------------------------------------------

def bw_probe(mm, dev, steps, warmup, gb=8.0):
    """Achievable streaming-read bandwidth: the library's read probe over a
    large buffer (one-shot workgroups, 128-bit non-temporal loads)."""
    import torch
    n = int(gb * 1e9) // 16 * 4
    a = torch.ones(n, dtype=torch.int32, device=dev)
    out = torch.empty(mm.lib().mmv_probe_slots(), dtype=torch.int32, device=dev)
    g = capture(lambda: mm.stream_read(a, out=out))
    s, st = timed_graph(g, max(2, steps // 4), warmup)
    del a, g
    torch.cuda.empty_cache()
    return dict(kind="mmv_stream_read over one buffer (32 KiB per workgroup)", GB=n * 4 / 1e9,
                GBps=n * 4 / st["mean"] / 1e9, s_stats=st)


# ---------------------------------------------------------------------------
# counter runs (rocprofv3 --pmc): one workload's graph plus calibration kernels
# ---------------------------------------------------------------------------

CAL_BYTES = 1 << 30
PROFILE_WORKLOADS = ("dense_gate_up", "q4_b1", "q4_b8", "w4a16_b1", "w4a16_b8", "moe256_b1",
                     "moe512_b8", "q4_ragged_b1")


def q4_ragged_graph(mm, dev, copies):
    """4096 x 11008 Q4_0 at B = 1 (rows of 344 blocks: the whole-row kernels'
    ragged last step), the W4A8 product from fp32 x and the W4A16 product of
    each copy, in one graph."""
    import torch
    import synth
    N, K = 4096, 11008
    qs1, d1 = synth.q4_0_weights(N, K, 0, "q4ragged", N, device=dev)
    qs = torch.empty((copies,) + tuple(qs1.shape), dtype=torch.uint8, device=dev)
    d = torch.empty((copies,) + tuple(d1.shape), dtype=torch.float16, device=dev)
    qs[:] = qs1
    d[:] = d1
    Ws = [mm.Q4_0(qs[c], d[c]) for c in range(copies)]
    X = synth.activations(copies, K, 0, "q4ragged-x", device=dev).view(copies, 1, K)
    Y8 = [torch.empty((1, N), device=dev) for _ in range(copies)]
    Y16 = [torch.empty((1, N), device=dev) for _ in range(copies)]

    def step():
        for c in range(copies):
            mm.gemv_q4_0(Ws[c], x=X[c], out=Y8[c])
            mm.gemv_q4_0_f32(Ws[c], X[c], out=Y16[c])
    return capture(step), (qs, d, Ws, X, Y8, Y16)


def profile_workload(mm, dev, name):
    """Replays one workload's graph 3 times, then the two calibration kernels
    of known traffic: the read probe over exactly 1 GiB (reads only) and an
    int16 fill of exactly 1 GiB (torch, writes only)."""
    import torch
    keep = None
    if name == "dense_gate_up":
        W = build_dense(dev, 36)
        dominant_kernel(mm, dev, W, 36, 3, 1)
    elif name in ("q4_b1", "q4_b8"):
        g, keep = q4_section(mm, dev, 32, 1 if name == "q4_b1" else 8, 0, 0, graph_only=True)
        for _ in range(3):
            g.replay()
    elif name in ("w4a16_b1", "w4a16_b8"):
        g, keep = w4a16_section(mm, dev, 32, 1 if name == "w4a16_b1" else 8, 0, 0,
                                graph_only=True)
        for _ in range(3):
            g.replay()
    elif name == "q4_ragged_b1":
        g, keep = q4_ragged_graph(mm, dev, 32)
        for _ in range(3):
            g.replay()
    elif name in ("moe256_b1", "moe512_b8"):
        E, k, B = (256, 8, 1) if name == "moe256_b1" else (512, 10, 8)
        lay, keep = moe_build(mm, dev, E, k, MOE_LAYERS[E])
        g, bufs = moe_graph(mm, dev, lay, E, k, B)
        for _ in range(3):
            g.replay()
    else:
        raise SystemExit(f"unknown workload {name}; one of {PROFILE_WORKLOADS}")
    torch.cuda.synchronize()
    buf = torch.ones(CAL_BYTES // 4, dtype=torch.int32, device=dev)
    out = torch.empty(mm.lib().mmv_probe_slots(), dtype=torch.int32, device=dev)
    for _ in range(3):
        mm.stream_read(buf, out=out)
    del buf
    fillbuf = torch.empty(CAL_BYTES // 2, dtype=torch.int16, device=dev)
    for _ in range(3):
        fillbuf.fill_(7)
    torch.cuda.synchronize()
    log(f"profile run {name} done; calibration read and fill of {CAL_BYTES} bytes")


def _counter_rows(d, counter):
    """{full kernel name: [per-dispatch counter values]} from rocprofv3 --pmc csv files."""
    paths = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not paths:
        raise SystemExit(f"no counter_collection.csv under {d}")
    out = {}
    for p in paths:
        for r in csv.DictReader(open(p)):
            if r.get("Counter_Name") == counter:
                out.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return out


def _short(name):
    """mmv::k_name<template args> from a full kernel name."""
    name = name.replace("void ", "")
    return re.sub(r"\(.*", "", name) if name.startswith("mmv::") else name[:60]


def summarize_counters(fetch_dir, write_dir, title):
    """Markdown: calibrated HBM bytes per dispatch of every library kernel in
    the two counter runs.  FETCH_SIZE and WRITE_SIZE are in KiB; the factor
    per counter comes from the calibration kernel of the same run (1 GiB read
    by the probe; 1 GiB written by an int16 fill, the largest fill dispatch)."""
    fe, wr = _counter_rows(fetch_dir, "FETCH_SIZE"), _counter_rows(write_dir, "WRITE_SIZE")
    probe = [v for k, vs in fe.items() if "k_stream_read" in k for v in vs]
    fills = [v for k, vs in wr.items() if "FillFunctor" in k for v in vs]
    f_cal = CAL_BYTES / (sum(probe) / len(probe) * 1024) if probe else None
    w_cal = CAL_BYTES / (max(fills) * 1024) if fills else None
    lines = [f"# {title}", "",
             "| kernel | dispatches | FETCH_SIZE KiB/dispatch | WRITE_SIZE KiB/dispatch | "
             "calibrated MB read | calibrated MB written |", "|---|---|---|---|---|---|"]
    for k in sorted(set(fe) | set(wr)):
        if "mmv::" not in k:
            continue
        f = sum(fe.get(k, [0])) / max(1, len(fe.get(k, [])))
        w = sum(wr.get(k, [0])) / max(1, len(wr.get(k, [])))
        fr = f * 1024 * f_cal / 1e6 if f_cal else float("nan")
        wb = w * 1024 * w_cal / 1e6 if w_cal else float("nan")
        lines.append(f"| `{_short(k)}` | {len(fe.get(k, []))} | {f:.1f} | {w:.1f} | {fr:.3f} | "
                     f"{wb:.3f} |")
    lines += ["", f"read calibration factor: {f_cal}", f"write calibration factor: {w_cal}"]
    return "\n".join(lines)


def summarize_trace(trace_dir, title):
    """Markdown: every library kernel's calls and durations from a rocprofv3
    --kernel-trace run, sorted by total time, and the dominant kernel's
    dispatches split by grid size."""
    paths = glob.glob(os.path.join(trace_dir, "**", "*kernel_trace.csv"), recursive=True)
    if not paths:
        raise SystemExit(f"no kernel_trace.csv under {trace_dir}")
    per, grid = {}, {}
    for p in paths:
        for r in csv.DictReader(open(p)):
            if "mmv::" not in r["Kernel_Name"]:
                continue
            k = _short(r["Kernel_Name"])
            us = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
            per.setdefault(k, []).append(us)
            if k.startswith("mmv::k_gemv_bf16_xl<1, 5, 8, 1, 5>"):
                grid.setdefault(int(r["Grid_Size_X"]), []).append(us)
    lines = [f"# {title}", "", "| kernel | calls | avg us | min us | max us |", "|---|---|---|---|---|"]
    for k, v in sorted(per.items(), key=lambda kv: -sum(kv[1])):
        lines.append(f"| `{k}` | {len(v)} | {sum(v) / len(v):.2f} | {min(v):.2f} | {max(v):.2f} |")
    if grid:
        lines += ["", "`k_gemv_bf16_xl<1, 5, 8, 1, 5>` dispatches by grid (threads; 512-thread "
                  "workgroups of 8 rows):", "", "| grid threads | rows (N) | dispatches | avg us | "
                  "min us |", "|---|---|---|---|---|"]
        for gsz, v in sorted(grid.items()):
            lines.append(f"| {gsz} | {gsz // 512 * 8} | {len(v)} | {sum(v) / len(v):.2f} | "
                         f"{min(v):.2f} |")
    return "\n".join(lines)


# ---------------------------------------------------------------------------
# MoE kernel timeline (the timeline build of the library)
# ---------------------------------------------------------------------------

TL_KINDS = [("router", ["start", "end"]),
            ("router (x in LDS)", ["start", "x staged"]),
            ("top-k + row lists", ["start", "top-k done", "lists published"]),
            ("gate/up", ["start", "routing known", "weights issued", "products done",
                         "Q8_1(h) stored"]),
            ("down (one kernel)", ["start", "row lists in LDS", "weights issued",
                                   "Q8_1(h) staged", "stored"]),
            ("down by expert", ["start", "weights issued", "stored"]),
            ("combine", ["start", "stored"])]


def moe_timeline(mm, dev, warmup):
    """Markdown: per kernel of one MoE layer (the last of a graph replay over
    every layer copy), the workgroups' times at each noted point relative to
    the first router workgroup's start (min / median / max, us), and the gaps
    between kernels; also the layer time of this build next to it."""
    import numpy as np
    import torch
    tl_bytes = mm.lib().mmv_timeline(None, 1, None)
    if tl_bytes == 0:
        raise SystemExit("this library notes no timeline: build it with "
                         "`python -m moe_matvec_amd.build --timeline`")
    n_kinds, slots, points = len(TL_KINDS), 4096, 8
    buf = torch.zeros(tl_bytes // 8, dtype=torch.int64, device=dev)
    lines = ["| workload | kernel | workgroups | point | min | median | max |",
             "|---|---|---|---|---|---|---|"]
    gaps = []
    for E, k, Bs in ((256, 8, [1]), (512, 10, [1, 8])):
        layers = MOE_LAYERS[E]
        lay, keep = moe_build(mm, dev, E, k, layers)
        for B in Bs:
            g, bufs = moe_graph(mm, dev, lay, E, k, B)
            s, st = timed_graph(g, 5, warmup)
            torch.cuda.synchronize()
            mm.lib().mmv_timeline(None, 1, torch.cuda.current_stream().cuda_stream)
            g.replay()
            mm.lib().mmv_timeline(buf.data_ptr(), 0, torch.cuda.current_stream().cuda_stream)
            torch.cuda.synchronize()
            a = buf.cpu().numpy().reshape(n_kinds, slots, points).astype(np.float64) / 100.0
            # every router workgroup runs in every layer: their stamps are the last
            # layer's; a workgroup of another kernel that exited early (an
            # unused expert slot) may hold an earlier layer's stamps: dropped
            t0 = min(a[i][a[i][:, 0] > 0, 0].min() for i in (0, 1) if (a[i][:, 0] > 0).any())
            wl = f"E={E} k={k} B={B} ({st['mean'] / layers * 1e6:.2f} us/layer in this build)"
            order = []
            for i, (kname, pnames) in enumerate(TL_KINDS):
                rows = a[i][a[i][:, 0] >= t0]
                if len(rows) == 0:
                    continue
                last = len(pnames) - 1
                rows = rows[rows[:, last] > 0]
                order.append((rows[:, 0].min() - t0, rows[:, last].max() - t0, kname))
                for j, pn in enumerate(pnames):
                    v = rows[:, j] - t0
                    lines.append(f"| {wl} | {kname} | {len(rows)} | {pn} | {v.min():.2f} | "
                                 f"{np.median(v):.2f} | {v.max():.2f} |")
                wl = ""
            order.sort()
            for (s0, e0, n0), (s1, e1, n1) in zip(order, order[1:]):
                gaps.append(f"| E={E} B={B} | {n0} -> {n1} | {s1 - e0:.2f} |")
            del g, bufs
        del lay, keep
        torch.cuda.empty_cache()
    return "\n".join(lines + ["", "Gap from the last workgroup of a kernel to the first of the "
                               "next (us):", "", "| workload | kernels | gap |", "|---|---|---|"]
                      + gaps)


# ---------------------------------------------------------------------------
# CPU baseline: the oracle on bounded samples of the five workloads
# ---------------------------------------------------------------------------

def cpu_info():
    model = platform.processor() or "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:
        avail = os.cpu_count() or 1
    share = int(os.environ.get("OMP_NUM_THREADS", "0") or 0)
    threads = min(avail, share) if share > 0 else avail
    return dict(model=model, nproc=os.cpu_count(), affinity=avail, threads=max(1, threads))


def _cpu_workloads():
    """(name, unit bytes, description, make(seed) -> callable) per workload;
    each callable runs one unit of the workload through the oracle."""
    import numpy as np
    import torch

    import oracle
    import synth

    def bf16(N, K, *tags):
        return synth.bf16_weights(N, K, 0, *tags).view(torch.int16).numpy().view(np.uint16)

    def c1(seed):
        W = bf16(1024, 1024, "c1")
        x = synth.activations(1, 1024, seed, "cpu-c1").numpy()
        return lambda: oracle.gemv_bf16(W, x)

    dense_W = {}

    def c2(seed):
        if not dense_W:
            dense_W.update({n: bf16(N, K, "dense", n) for n, (N, K) in DENSE_SHAPES.items()})
        X = {n: synth.activations(1, K, seed, "cpu-x", n).numpy()
             for n, (N, K) in DENSE_SHAPES.items()}
        return lambda: [oracle.gemv_bf16(dense_W[n], X[n]) for n in DENSE_SHAPES]

    q4 = []

    def c3(seed):
        if not q4:
            q4.extend((synth.q4_0_weights(N, K, 0, "q4bench", N)) for N, K in Q4_SHAPES)
        x = synth.activations(1, 4096, seed, "cpu-c3").numpy()

        def run():
            xq, xds = oracle.quantize_q8_1(x)
            for qs, d in q4:
                oracle.gemv_q4_0(qs.numpy(), d.view(torch.int16).numpy().view(np.uint16), xq, xds)
        return run

    moe = {}

    def moe_cfg(E, k, B):
        # the oracle's time does not depend on the weight values: uniform
        # random codes and scales of the right magnitude (numpy, fast)
        def make(seed):
            if E not in moe:
                rng = np.random.default_rng(E)
                H, I = 2048, 512
                q = lambda *sh: rng.integers(0, 256, sh + (16,), dtype=np.uint8)
                d = lambda *sh: (rng.random(sh, dtype=np.float32) * 0.005 + 0.001).astype(
                    np.float16).view(np.uint16)
                router = (rng.standard_normal((E, H), dtype=np.float32) * 0.02)
                moe[E] = oracle.MoE(router, q(E, I, H // 32), d(E, I, H // 32),
                                    q(E, I, H // 32), d(E, I, H // 32), q(E, H, I // 32),
                                    d(E, H, I // 32), k,
                                    shared=(q(I, H // 32), d(I, H // 32), q(I, H // 32),
                                            d(I, H // 32), q(H, I // 32), d(H, I // 32)))
            X = synth.activations(B, 2048, seed, "cpu-moe", E, B).numpy()
            return lambda: moe[E].layer(X)
        return make

    exp_bytes = 3 * (512 * 2048 // 32) * 18
    return [
        ("C1 BF16 1024x1024, B=1", 2 * 1024 * 1024 + 8 * 1024, "GEMV", c1),
        ("C2 dense BF16 layer (attn-out, gate+up, down), B=1", dense_bytes(1), "layer", c2),
        ("C3 Q4_0 4096^2 + 11008x4096, B=1", q4_bytes(1), "pair", c3),
        ("C4 MoE E=256 top-8 + shared, B=1", 256 * 2048 * 4 + 9 * exp_bytes, "layer",
         moe_cfg(256, 8, 1)),
        ("C5 MoE E=512 top-10 + shared, B=1", 512 * 2048 * 4 + 11 * exp_bytes, "layer",
         moe_cfg(512, 10, 1)),
    ]


def cpu_baseline(budget_s=2.5):
    """Each workload through the oracle: single-threaded for about budget_s,
    then on every core of the host's share (one independent unit per thread,
    the oracle's C code running in parallel: ctypes releases the GIL)."""
    info = cpu_info()
    res = dict(cpu=info, configs={})
    T = info["threads"]
    for name, nbytes, unit, make in _cpu_workloads():
        run = make(0)
        run()  # first call: builds and loads the oracle, touches the data
        n, t0 = 0, time.perf_counter()
        while True:
            run()
            n += 1
            el = time.perf_counter() - t0
            if el >= budget_s:
                break
        single = dict(units=n, seconds=el, us_per_unit=el / n * 1e6, GBps=n * nbytes / el / 1e9)
        runs = [make(1 + i) for i in range(T)]
        counts = [0] * T
        stop = [False]

        def worker(i):
            while not stop[0]:
                runs[i]()
                counts[i] += 1
        th = [threading.Thread(target=worker, args=(i,)) for i in range(T)]
        t0 = time.perf_counter()
        for t in th:
            t.start()
        time.sleep(budget_s)
        stop[0] = True
        for t in th:
            t.join()
        el = time.perf_counter() - t0
        allc = dict(threads=T, units=sum(counts), seconds=el,
                    units_per_s=sum(counts) / el, GBps=sum(counts) * nbytes / el / 1e9)
        res["configs"][name] = dict(unit=unit, algorithmic_bytes_per_unit=nbytes,
                                    single_thread=single, all_cores=allc)
        log(f"cpu oracle {name}: {single['GBps']:.2f} GB/s single, "
            f"{allc['GBps']:.2f} GB/s on {T} threads")
    return res


# ---------------------------------------------------------------------------
# roofline traffic from committed rocprofv3 counter summaries
# ---------------------------------------------------------------------------

def kernel_source_hash():
    p = os.path.join(ROOT, "moe_matvec_amd", "csrc", "gemv_bf16.hip")
    return hashlib.sha256(open(p, "rb").read()).hexdigest()[:16]


def traffic_from_profiles():
    """HBM bytes per launch of the dominant kernel, from the committed
    FETCH_SIZE / WRITE_SIZE summary, if it was taken on the current source."""
    p = os.path.join(ROOT, "profiles", "gemv_bf16_gate_up_b1_counters.md")
    if not os.path.exists(p):
        return None
    text = open(p).read()
    m_hash = re.search(r"source sha256\[:16\]:\s*`?([0-9a-f]{16})", text)
    m_bytes = re.search(r"traffic bytes per launch:\s*([0-9.eE+]+)", text)
    if not (m_hash and m_bytes) or m_hash.group(1) != kernel_source_hash():
        return None
    return float(m_bytes.group(1))


# ---------------------------------------------------------------------------
# manifest and contention gate
# ---------------------------------------------------------------------------

def manifest(torch, dev):
    h = hashlib.sha256()
    for sub in ("include", os.path.join("moe_matvec_amd", "csrc")):
        for p in sorted(glob.glob(os.path.join(ROOT, sub, "*"))):
            h.update(open(p, "rb").read())
    lib = os.path.join(ROOT, "moe_matvec_amd", "libmoe_matvec.so")
    return dict(source_sha256=h.hexdigest()[:16],
                library_sha256=hashlib.sha256(open(lib, "rb").read()).hexdigest()[:16],
                torch=torch.__version__, hip=getattr(torch.version, "hip", None),
                device=torch.cuda.get_device_name(dev), host=platform.node(),
                utc=time.strftime("%Y-%m-%dT%H:%M:%SZ", time.gmtime()), argv=sys.argv[1:])


def contention():
    """Other processes holding the GPU driver open, and the GPU busy percentage,
    sampled before the timed work (a busy GPU makes every number suspect)."""
    me = os.getpid()
    others = []
    for d in glob.glob("/sys/class/kfd/kfd/proc/*"):
        pid = os.path.basename(d)
        if pid.isdigit() and int(pid) != me:
            others.append(int(pid))
    busy = []
    for p in glob.glob("/sys/class/drm/card*/device/gpu_busy_percent"):
        try:
            vals = []
            for _ in range(5):
                vals.append(int(open(p).read().strip()))
                time.sleep(0.01)
            busy.append(max(vals))
        except (OSError, ValueError):
            pass
    flag = bool(others) or any(b > 15 for b in busy)
    return dict(other_kfd_processes=others, gpu_busy_percent_max=busy, contended=flag)


# ---------------------------------------------------------------------------

def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--only", default="dense,q4,w4a16,lmhead,moe256,moe512,moe512v")
    ap.add_argument("--quick", action="store_true", help="fewer layer copies (smoke timing)")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--profile", choices=PROFILE_WORKLOADS,
                    help="run only this workload's graph and the calibration kernels "
                         "(for rocprofv3 counter runs)")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="print a markdown summary of two rocprofv3 counter runs")
    ap.add_argument("--summarize-trace", metavar="TRACE_DIR",
                    help="print a markdown summary of a rocprofv3 --kernel-trace run")
    ap.add_argument("--timeline", action="store_true",
                    help="per-phase timeline of the MoE kernels (needs the timeline build, "
                         "libmoe_matvec_timeline.so)")
    ap.add_argument("--title", default="HBM traffic per dispatch")
    args = ap.parse_args()
    if args.summarize_counters:
        print(summarize_counters(*args.summarize_counters, args.title))
        return
    if args.summarize_trace:
        print(summarize_trace(args.summarize_trace, args.title))
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs on one GPU only: this library has no multi-GPU path "
              "(the matvec would shard by output rows or by experts, with no exchange "
              "inside a layer)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import moe_matvec_amd as mm
    if args.timeline:
        from moe_matvec_amd import build as mmbuild
        if not os.path.exists(mmbuild.SO_TIMELINE):
            raise SystemExit("build the timeline library first: "
                             "python -m moe_matvec_amd.build --timeline")
        mm.library_path = mmbuild.SO_TIMELINE
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.timeline:
        print(moe_timeline(mm, dev, args.warmup))
        return
    if args.profile:
        profile_workload(mm, dev, args.profile)
        return
    only = set(args.only.split(","))
    steps, warmup = args.steps, args.warmup
    dense_layers = 4 if args.quick else 36
    gate = contention()
    if gate["contended"]:
        log(f"WARNING: GPU contended before timing: {gate}")

    log(f"device {torch.cuda.get_device_name(dev)}; building dense BF16 workload "
        f"({dense_layers} layer copies)")
    W = build_dense(dev, dense_layers)
    sections = {}
    head = dense_section(mm, dev, W, dense_layers, 1, steps, warmup, eager=True)
    log(f"dense B=1: {head['GBps']:.0f} GB/s, {head['us_per_layer']:.2f} us/layer "
        f"(mean of {REPS}: {head['us_per_layer_stats']['mean']:.2f} +- "
        f"{head['us_per_layer_stats']['ci95']:.2f})")
    dom = dominant_kernel(mm, dev, W, dense_layers, steps, warmup)
    log(f"dominant kernel: {dom['GBps']:.0f} GB/s, {dom['s_per_launch']*1e6:.2f} us/launch")
    sections["dense_bf16"] = {"B1": head}
    if "dense" in only:
        b8 = dense_section(mm, dev, W, dense_layers, 8, steps, warmup)
        sections["dense_bf16"]["B8"] = b8
        sections["dense_bf16"]["ratio_B8_B1_time"] = b8["s_per_step"] / head["s_per_step"]
        log(f"dense B=8: {b8['GBps']:.0f} GB/s, ratio {sections['dense_bf16']['ratio_B8_B1_time']:.2f}")
        sections["dense_bf16"]["per_matrix"] = {
            f"B{B}": dense_per_matrix(mm, dev, W, dense_layers, B, steps, warmup) for B in (1, 8)}
        for B in (1, 8):
            pm = sections["dense_bf16"]["per_matrix"][f"B{B}"]
            log(f"dense per matrix B={B}: " + ", ".join(
                f"{n} {v['us_per_launch_stats']['mean']:.2f} us" for n, v in pm.items()))
        one, c1 = cache_resident(mm, dev, W, dense_layers, steps, warmup)
        sections["dense_bf16"]["one_copy_cache_resident"] = one
        sections["c1_cache_resident"] = c1
        log(f"one dense copy repeated (cache-resident): {one['GBps']:.0f} GB/s; "
            f"C1 1024x1024: {c1['GBps']:.0f} GB/s")
    del W
    torch.cuda.empty_cache()
    sections["launch_floor"] = launch_floor(mm, dev, steps, warmup)
    fl = sections["launch_floor"]["us_per_launch"]["mean"]
    sections["dense_bf16"]["B1"]["launches_per_token"] = 3 * dense_layers
    sections["dense_bf16"]["B1"]["launch_floor_us_per_token"] = 3 * dense_layers * fl
    log(f"dependent launch floor: {fl:.2f} us per launch")

    if "q4" in only:
        q = {}
        for copies, B in ((8 if args.quick else 32, 1), (8 if args.quick else 32, 8),
                          (8 if args.quick else 128, 1)):
            r = q4_section(mm, dev, copies, B, steps, warmup)
            q[f"copies{copies}_B{B}"] = r
            log(f"q4_0 copies={copies} B={B}: {r['GBps']:.0f} GB/s, {r['us_per_copy']:.2f} us/copy")
            torch.cuda.empty_cache()
        sections["q4_0"] = q
    if "w4a16" in only:
        q = {}
        for copies, B in ((8 if args.quick else 32, 1), (8 if args.quick else 32, 4),
                          (8 if args.quick else 32, 8)):
            r = w4a16_section(mm, dev, copies, B, steps, warmup)
            q[f"copies{copies}_B{B}"] = r
            log(f"w4a16 copies={copies} B={B}: {r['GBps']:.0f} GB/s, {r['us_per_copy']:.2f} us/copy")
            torch.cuda.empty_cache()
        sections["q4_0_w4a16"] = q
    if "lmhead" in only:
        r = lm_head_section(mm, dev, [1, 8], steps, warmup)
        sections["lm_head"] = r
        log("lm head: " + ", ".join(
            f"B{b} gemv {r[f'B{b}']['us_gemv']:.1f} us ({r[f'B{b}']['gemv_GBps']:.0f} GB/s), "
            f"argmax {r[f'B{b}']['us_argmax']:.2f} us" for b in (1, 8)))
    if "moe256" in only:
        r = moe_section(mm, dev, 256, 8, 4 if args.quick else 40, [1], steps, warmup)
        sections["moe_e256_top8"] = r
        log(f"moe E=256: {r['B1']['us_per_layer']:.2f} us/layer, {r['B1']['GBps']:.0f} GB/s")
    if "moe512" in only:
        r = moe_section(mm, dev, 512, 10, 4 if args.quick else 48, [1, 2, 4, 8], steps, warmup)
        sections["moe_e512_top10"] = r
        log("moe E=512: " + ", ".join(f"B{b} {r[f'B{b}']['us_per_layer']:.2f} us"
                                      for b in (1, 2, 4, 8)))
    if "moe512v" in only:  # verify / prefill batches: the row-list path (B > 8)
        r = moe_section(mm, dev, 512, 10, 4 if args.quick else 48, [16, 32, 64], steps, warmup)
        sections["moe_e512_top10_verify"] = r
        log("moe E=512 verify: " + ", ".join(
            f"B{b} {r[f'B{b}']['us_per_layer']:.1f} us ({r[f'B{b}']['us_per_layer_per_token']:.2f}"
            f" us/token, {r[f'B{b}']['GBps']:.0f} GB/s)" for b in (16, 32, 64)))
    sections["bw_probe"] = bw_probe(mm, dev, steps, warmup)
    log(f"read probe: {sections['bw_probe']['GBps']:.0f} GB/s")

    cpu = None
    if not args.no_cpu:
        cb = cpu_baseline()
        sections["cpu_oracle"] = cb
        c2 = cb["configs"]["C2 dense BF16 layer (attn-out, gate+up, down), B=1"]
        cpu = dict(value=c2["all_cores"]["GBps"], unit="GB/s",
                   cores=c2["all_cores"]["threads"], kind="oracle",
                   sample=(f"{c2['all_cores']['units']} dense BF16 layer passes (attn-out, "
                           f"gate+up, down; 162.5 MB of weights, batch 1) by the C oracle on "
                           f"{c2['all_cores']['threads']} threads in "
                           f"{c2['all_cores']['seconds']:.1f} s (one independent pass per "
                           f"thread); single-threaded "
                           f"{c2['single_thread']['GBps']:.3f} GB/s; CPU "
                           f"{cb['cpu']['model']}, nproc {cb['cpu']['nproc']}"))
    traffic = traffic_from_profiles()
    roof = {"bound": "hbm", "achieved": dom["GBps"], "peak": PEAK_HBM_GBPS, "unit": "GB/s",
            "frac": dom["GBps"] / PEAK_HBM_GBPS, "traffic": traffic,
            "frac_of_probe": dom["GBps"] / sections["bw_probe"]["GBps"],
            "kernel": dom["kernel"], "bytes_per_launch": dom["bytes_per_launch"],
            "us_per_launch": dom["s_per_launch"] * 1e6,
            "us_per_launch_stats": dom["us_per_launch_stats"]}
    line = {
        "metric": METRIC,
        "value": head["GBps"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": head["s_per_step"] * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": (f"dense BF16 decode matvec set, batch 1: {dense_layers} layer "
                                "copies of attn-out 2560x2560, gate+up 2x9728x2560 (one "
                                "launch), down 2560x9728; weights N(0,0.02) bf16, x N(0,1) "
                                "fp32, fp32 accumulate; one HIP graph per pass"),
                   "weights": "bf16", "batch": 1, "layers": dense_layers,
                   "frac_of_peak": head["frac_of_peak"],
                   "tokens_per_s_equiv": head["tokens_per_s_equiv"]},
        "roofline": roof,
        "cpu_baseline": cpu,
        "stats": head["us_per_layer_stats"],
        "manifest": manifest(torch, dev),
        "contention": gate,
        "sections": sections,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
