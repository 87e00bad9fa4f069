#!/usr/bin/env python3
"""Benchmark of the decode matrix-vector path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--quick] [--no-cpu]
                    [--only dense,q4,w4a16,lmhead,moe256,moe512,moe512v] [--profile-kernel]

The headline step is one pass over the dense BF16 decode matvec set: 36 layer
copies (5.85 GB, far past the 256 MB Infinity Cache) of attn-out 2560x2560,
fused gate+up 2 x 9728x2560 and down 2560x9728, batch 1, each matrix with
its own synthetic N(0,1) activation row, captured in one HIP graph and
replayed K times.  `value` is algorithmic bytes / time in GB/s.  The same
JSON line carries the other workloads (B = 8 dense, Q4_0 x Q8_1 GEMV, the
W4A16 Q4_0 GEMV, the 248320 x 2560 LM head with its on-device argmax, the
256- and 512-expert MoE layers) under "sections", the roofline of the
dominant kernel and the CPU oracle's throughput on a bounded sample.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0
METRIC = ("achieved HBM GB/s (% of MI355X peak) for batch-1 GEMV; MoE layer µs/token")


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


def time_graph(g, steps, warmup):
    """Seconds per replay over `steps` replays, bracketed by synchronize and
    events on the replaying stream."""
    import torch
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    st = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(st)
    for _ in range(steps):
        g.replay()
    e1.record(st)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / 1e3 / steps


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


def dense_section(mm, dev, W, layers, B, steps, warmup):
    import torch
    import synth
    X = {n: synth.activations(layers * B, K, 0, "dense-x", n, B, device=dev).view(layers, B, K)
         for n, (N, K) in DENSE_SHAPES.items()}
    Y = {n: torch.empty((layers, B, N), device=dev) for n, (N, K) in DENSE_SHAPES.items()}

    def step():
        for l in range(layers):
            for n in DENSE_SHAPES:
                mm.gemv_bf16(W[n][l], X[n][l], out=Y[n][l])
    g = capture(step)
    t = time_graph(g, steps, warmup)
    nbytes = layers * dense_bytes(B)
    return dict(B=B, layers=layers, launches_per_layer=3, s_per_step=t,
                us_per_layer=t / layers * 1e6, GBps=nbytes / t / 1e9,
                frac_of_peak=nbytes / t / 1e9 / PEAK_HBM_GBPS, bytes_per_step=nbytes)


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
    t = time_graph(g, steps, warmup) / layers
    per_launch = 2 * N * K + 4 * K + 4 * N
    return dict(kernel="k_gemv_bf16_xl<1, 5, 8, 1, 5> (gate+up 19456x2560, B=1)", s_per_launch=t,
                bytes_per_launch=per_launch, GBps=per_launch / t / 1e9)


# ---------------------------------------------------------------------------
# Q4_0 x Q8_1
# ---------------------------------------------------------------------------

Q4_SHAPES = [(4096, 4096), (11008, 4096)]


def q4_bytes(B):
    return sum(N * K // 32 * 18 + 4 * B * K + 4 * B * N for N, K in Q4_SHAPES)


def q4_section(mm, dev, copies, B, steps, warmup):
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
    t = time_graph(g, steps, warmup)
    nbytes = copies * q4_bytes(B)
    del mats, Ws
    return dict(B=B, copies=copies, act_quant="in-kernel" if B == 1 else "separate pass",
                launches_per_copy=len(Q4_SHAPES) * (1 if B == 1 else 2),
                stored_GB=copies * sum(N * K // 32 * 18 for N, K in Q4_SHAPES) / 1e9,
                s_per_step=t, us_per_copy=t / copies * 1e6, GBps=nbytes / t / 1e9,
                frac_of_peak=nbytes / t / 1e9 / PEAK_HBM_GBPS)


def w4a16_section(mm, dev, copies, B, steps, warmup):
    """The Q4_0 shapes with fp32 activations (no Q8_1 step): one launch per
    product at every B."""
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
    K = Q4_SHAPES[0][1]
    X = synth.activations(copies * B, K, 0, "w4a16bench-x", B, device=dev).view(copies, B, K)
    Ys = [[torch.empty((B, N), device=dev) for N, _ in Q4_SHAPES] for _ in range(copies)]

    def step():
        for c in range(copies):
            for i, W in enumerate(Ws[c]):
                mm.gemv_q4_0_f32(W, X[c], out=Ys[c][i])
    g = capture(step)
    t = time_graph(g, steps, warmup)
    nbytes = copies * q4_bytes(B)
    del mats, Ws
    return dict(B=B, copies=copies, launches_per_copy=len(Q4_SHAPES), s_per_step=t,
                us_per_copy=t / copies * 1e6, GBps=nbytes / t / 1e9,
                frac_of_peak=nbytes / t / 1e9 / PEAK_HBM_GBPS)


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
        t_g = time_graph(capture(gemv), steps, warmup)
        t_a = time_graph(capture(amax), steps, warmup) / reps
        t_b = time_graph(capture(both), steps, warmup)
        gbytes = 2 * LM_VOCAB * LM_HID + 4 * B * LM_HID + 4 * B * LM_VOCAB
        res[f"B{B}"] = dict(us_gemv=t_g * 1e6, us_argmax=t_a * 1e6, us_gemv_argmax=t_b * 1e6,
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

def moe_section(mm, dev, E, k, layers, Bs, steps, warmup, H=2048, I=512):
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
    expert_bytes = lay[0].expert_bytes()
    stored = layers * (E * H * 4 + (E + 1) * expert_bytes)
    res = dict(E=E, k=k, shared=1, H=H, I=I, layers=layers, stored_GB=stored / 1e9)
    for B in Bs:
        X = synth.activations(layers * B, H, 0, "moebench-x", E, B, device=dev).view(layers, B, H)
        Y = torch.empty((layers, B, H), device=dev)
        ids = torch.empty((layers, B, k), dtype=torch.int32, device=dev)
        ws = torch.empty((layers, mm.moe_workspace_bytes(lay[0], B)), dtype=torch.uint8,
                         device=dev)

        def step():
            for l in range(layers):
                mm.moe_layer_decode(lay[l], X[l], out=Y[l], workspace=ws[l], ids=ids[l])
        g = capture(step)
        t = time_graph(g, steps, warmup)
        idn = ids.cpu().numpy()
        uniq = [len(set(idn[l].ravel().tolist())) for l in range(layers)]
        nbytes = sum(E * H * 4 + 4 * B * H * 2 + (u + 1) * expert_bytes for u in uniq)
        res[f"B{B}"] = dict(us_per_layer=t / layers * 1e6,
                            us_per_layer_per_token=t / layers / B * 1e6,
                            mean_unique_experts=sum(uniq) / layers,
                            MB_per_layer=nbytes / layers / 1e6, GBps=nbytes / t / 1e9,
                            frac_of_peak=nbytes / t / 1e9 / PEAK_HBM_GBPS,
                            launches_per_layer=(3 if B <= 2 else 5) if B <= 8
                            else (6 if H in (1024, 2048) else 5 + (B + 7) // 8))
        del X, Y, ids, ws, g
    if len(Bs) > 1 and 1 in Bs:
        res["ratio_Bmax_B1_time"] = res[f"B{max(Bs)}"]["us_per_layer"] / res["B1"]["us_per_layer"]
    del lay, big, sh
    torch.cuda.empty_cache()
    return res


def bw_probe(mm, dev, gb=8.0):
    """Achievable streaming-read bandwidth: the library's read probe over a
    large buffer (128-bit non-temporal loads, grid-stride)."""
    import torch
    n = int(gb * 1e9) // 16 * 4
    a = torch.ones(n, dtype=torch.int32, device=dev)
    out = torch.empty(mm.lib().mmv_probe_slots(), dtype=torch.int32, device=dev)
    g = capture(lambda: mm.stream_read(a, out=out))
    t = time_graph(g, 5, 2)
    del a, g
    torch.cuda.empty_cache()
    return dict(kind="mmv_stream_read over one buffer", GB=n * 4 / 1e9, GBps=n * 4 / t / 1e9)


CAL_BYTES = 1 << 30


def profile_kernel(mm, dev, W, layers):
    """For rocprofv3 counter runs: the dominant kernel's launches, then two
    calibration kernels of known traffic: the read probe over 1 GiB (reads
    only) and an int16 fill of 1 GiB (writes only)."""
    import torch
    dom = dominant_kernel(mm, dev, W, layers, 3, 1)
    buf = torch.ones(CAL_BYTES // 4, dtype=torch.int32, device=dev)
    out = torch.empty(mm.lib().mmv_probe_slots(), dtype=torch.int32, device=dev)
    for _ in range(3):
        mm.stream_read(buf, out=out)
    del buf
    fillbuf = torch.empty(CAL_BYTES // 2, dtype=torch.int16, device=dev)
    for _ in range(3):
        fillbuf.fill_(7)
    torch.cuda.synchronize()
    log(f"profile run: dominant {dom['s_per_launch'] * 1e6:.2f} us/launch; "
        f"calibration read and fill of {CAL_BYTES} bytes")
    return dom


# ---------------------------------------------------------------------------
# CPU baseline: the oracle on a bounded sample of the headline workload
# ---------------------------------------------------------------------------

def cpu_baseline(budget_s=12.0):
    import numpy as np
    import torch

    import oracle
    import synth
    W = {n: synth.bf16_weights(N, K, 0, "dense", n).view(torch.int16).numpy().view(np.uint16)
         for n, (N, K) in DENSE_SHAPES.items()}
    X = {n: synth.activations(1, K, 0, "cpu-x", n).numpy() for n, (N, K) in DENSE_SHAPES.items()}
    oracle.lib()
    nbytes, t0, passes = 0, time.perf_counter(), 0
    while True:
        for n in DENSE_SHAPES:
            oracle.gemv_bf16(W[n], X[n])
        passes += 1
        nbytes += dense_bytes(1)
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    return dict(value=nbytes / el / 1e9, unit="GB/s", cores=1, kind="oracle",
                sample=f"{passes} pass(es) of one dense BF16 layer copy (attn-out, gate+up, "
                       f"down; 162.5 MB of weights), batch 1, single-threaded C oracle, "
                       f"{el:.1f} s")


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

def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--only", default="dense,q4,w4a16,lmhead,moe256,moe512,moe512v")
    ap.add_argument("--quick", action="store_true", help="fewer layer copies (smoke timing)")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--profile-kernel", action="store_true",
                    help="run only the dominant kernel's graph (for rocprofv3 counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs on one GPU only: this library has no multi-GPU path "
              "(the matvec would shard by output rows or by experts, with no exchange "
              "inside a layer)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import moe_matvec_amd as mm
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    only = set(args.only.split(","))
    steps, warmup = args.steps, args.warmup
    dense_layers = 4 if args.quick else 36

    log(f"device {torch.cuda.get_device_name(dev)}; building dense BF16 workload "
        f"({dense_layers} layer copies)")
    W = build_dense(dev, dense_layers)
    if args.profile_kernel:
        profile_kernel(mm, dev, W, dense_layers)
        return
    sections = {}
    head = dense_section(mm, dev, W, dense_layers, 1, steps, warmup)
    log(f"dense B=1: {head['GBps']:.0f} GB/s, {head['us_per_layer']:.2f} us/layer")
    dom = dominant_kernel(mm, dev, W, dense_layers, steps, warmup)
    log(f"dominant kernel: {dom['GBps']:.0f} GB/s, {dom['s_per_launch']*1e6:.2f} us/launch")
    sections["dense_bf16"] = {"B1": head}
    if "dense" in only:
        b8 = dense_section(mm, dev, W, dense_layers, 8, steps, warmup)
        sections["dense_bf16"]["B8"] = b8
        sections["dense_bf16"]["ratio_B8_B1_time"] = b8["s_per_step"] / head["s_per_step"]
        log(f"dense B=8: {b8['GBps']:.0f} GB/s, ratio {sections['dense_bf16']['ratio_B8_B1_time']:.2f}")
    del W
    torch.cuda.empty_cache()

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
        r = moe_section(mm, dev, 512, 10, 4 if args.quick else 48, [1, 4, 8], steps, warmup)
        sections["moe_e512_top10"] = r
        log("moe E=512: " + ", ".join(f"B{b} {r[f'B{b}']['us_per_layer']:.2f} us"
                                      for b in (1, 4, 8)))
    if "moe512v" in only:  # verify / prefill batches: the row-list path (B > 8)
        r = moe_section(mm, dev, 512, 10, 4 if args.quick else 48, [16, 32, 64], steps, warmup)
        sections["moe_e512_top10_verify"] = r
        log("moe E=512 verify: " + ", ".join(
            f"B{b} {r[f'B{b}']['us_per_layer']:.1f} us ({r[f'B{b}']['us_per_layer_per_token']:.2f}"
            f" us/token, {r[f'B{b}']['GBps']:.0f} GB/s)" for b in (16, 32, 64)))
    sections["bw_probe"] = bw_probe(mm, dev)

    cpu = None if args.no_cpu else cpu_baseline()
    traffic = traffic_from_profiles()
    roof = {"bound": "hbm", "achieved": dom["GBps"], "peak": PEAK_HBM_GBPS, "unit": "GB/s",
            "frac": dom["GBps"] / PEAK_HBM_GBPS, "traffic": traffic,
            "frac_of_probe": dom["GBps"] / sections["bw_probe"]["GBps"],
            "kernel": dom["kernel"], "bytes_per_launch": dom["bytes_per_launch"],
            "us_per_launch": dom["s_per_launch"] * 1e6}
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
                   "frac_of_peak": head["frac_of_peak"]},
        "roofline": roof,
        "cpu_baseline": cpu,
        "sections": sections,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
