"""Throughput of the fused attention forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--no-legs] [--extra]

A step is one fa_fwd over the whole causal bf16 workload B=8, H=32,
N=8192, d=128 (scale 1/sqrt(d)), inputs resident in HBM before timing.
Prints one JSON line with the throughput in TFLOP/s (2*N^2*d FLOP per head
for the causal mask, i.e. 4*N^2*d halved), the roofline of the kernel
against the dense bf16 MFMA peak, and the fp64 CPU oracle timed on a
bounded sample of the same workload.

--profile-run: the run used under rocprofv3 counters: one 1 GiB device
copy (the byte-count calibration kernel) followed by --steps launches.
--profile-decode: --steps split-K decode calls on B=8 H=32 N=32768 d=128.
--profile-bwd: --steps backward calls on B=2 H=16 N=4096 d=128 causal (the
forward-plus-backward workload), printed as one JSON line.
--profile-decode-gqa: --steps decode calls on B8 H64 Hkv8 N32768 d128
(8 query heads per key/value head, the MFMA decode kernel).
--profile-fp8: --steps fa_fwd_fp8 calls on B8 H32 N8192 and B2 H16 N4096
d=128 causal (e4m3 inputs).

Next to the timed launches the line carries: the median, min and max
launch time; a cold-cache timing (1 GiB written between launches, more
than the 256 MB Infinity Cache); the shader clock read from sysfs while
the kernel runs, the power cap and the CU count; the rate of a
matrix-core-only kernel (fa_mfma_ceiling) as the sustained MFMA ceiling;
and the oracle's per-core rate and extrapolated full-workload time.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import statistics
import subprocess
import sys
import threading
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6  # MI355X dense bf16 MFMA: 256 CU x 4096 FLOP/clk x 2.4 GHz
PEAK_FP32_TFLOPS = 157.3  # MI355X fp32 (matrix and vector alike): 256 CU x 256 FLOP/clk x 2.4 GHz
PEAK_HBM_GBS = 8000.0
KERNEL_SOURCE = os.path.join(ROOT, "aware_softmax_amd", "csrc", "fa_fwd_mfma.hip")
COUNTERS_FILE = os.path.join(ROOT, "profiles", "fa_fwd_bf16_B8H32N8192d128_counters.txt")
METRIC = "causal bf16 attention fwd TFLOPS at N=8k,d=128; % of MI355X MFMA peak"


def attention_flops(B, H, N, d, causal):
    """Algorithmic FLOPs: 4*N^2*d per head (two N x N x d products), halved
    for the causal mask."""
    f = 4.0 * N * N * d * B * H
    return f / 2 if causal else f


def causal_row_flops(rows, d):
    """FLOPs of the causal rows actually visible: row i sees i + 1 keys."""
    return float(sum(4.0 * d * (int(i) + 1) for i in rows))


def kernel_source_hash(path=KERNEL_SOURCE):
    """sha256 of the kernel source with comments and blank space removed, so
    that only a change of the code itself invalidates stored counters."""
    with open(path) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    text = " ".join(text.split())
    return hashlib.sha256(text.encode()).hexdigest()


def traffic_models(w, bq, lds_bytes=160 * 1024):
    """HBM bytes per launch under three models, next to the measured
    traffic: compulsory (read Q, K, V, write O and L once); the pages'
    Theta(N^2 d^2 / M) bound with M = one CU's 160 KB of LDS in elements;
    and re-reading every visible K/V tile once per query block of bq rows
    with no cache reuse."""
    s = 2  # bytes per element
    heads = w.B * w.H
    compulsory = heads * (4 * w.N * w.d * s + 4 * w.N)
    theta = heads * w.N * w.N * w.d * w.d * s / (lds_bytes / s)
    nqb = -(-w.N // bq)
    tiles = sum(min(w.N, (i + 1) * bq) for i in range(nqb)) if w.causal else nqb * w.N
    no_reuse = heads * (2 * s * w.d * tiles + 2 * w.N * w.d * s + 4 * w.N)
    return {"compulsory": compulsory, "theta_N2d2_over_M": round(theta), "no_reuse_per_query_block": no_reuse,
            "M_bytes": lds_bytes, "block_q": bq}


def read_traffic():
    """HBM bytes per launch from the committed counter summary, or None if
    the summary is missing or the kernel source changed since."""
    if not os.path.exists(COUNTERS_FILE):
        return None
    kv = {}
    with open(COUNTERS_FILE) as f:
        for line in f:
            if ":" in line:
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    if kv.get("kernel_code_sha256 (source without comments or blank space)") != kernel_source_hash():
        return None
    try:
        return float(kv["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def make_inputs(w, threads=16):
    import numpy as np
    import torch

    import synthetic

    dev = torch.device("cuda:0")
    out = []
    for t in ("q", "k", "v"):
        st = synthetic.full_storage(w.config_id, t, w.B, w.H, w.N, w.d, w.dtype, threads=threads)
        out.append(torch.from_numpy(st.view(np.int16)).view(torch.bfloat16).to(dev))
        del st
    return out


def prewarm(fn, ms=200.0):
    """Calls fn() back to back until about `ms` of GPU time has passed
    (untimed).  After an idle spell the first tens of milliseconds of
    launches run 3-6 % slower than the steady state (clock and memory
    system ramping up); every timed region below starts after such a
    stretch of the same launches."""
    import torch

    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    done, n = 0.0, 1
    while done < ms and n < 100000:
        a.record()
        for _ in range(n):
            fn()
        b.record()
        torch.cuda.synchronize()
        done += a.elapsed_time(b)
        n = min(2 * n, 1000)


def time_launches(fa, q, k, v, o, lse, causal, scale, steps, warmup):
    import torch

    for _ in range(warmup):
        fa.fwd(q, k, v, causal=causal, scale=scale, out=o, lse=lse)
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    t_begin = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_begin.record()
    for i in range(steps):
        starts[i].record()
        fa.fwd(q, k, v, causal=causal, scale=scale, out=o, lse=lse)
        ends[i].record()
    t_end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    per = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    time_launches.last_per_launch = per
    return t_begin.elapsed_time(t_end) / steps, sum(per) / len(per), min(per), max(per), wall


def graph_ms(fn, reps, check=None):
    """Mean GPU time of fn() with launch overhead removed: `reps` calls
    captured into one HIP graph (stream capture through torch), replayed
    twice, the second replay timed.  For kernels shorter than the host's
    cost of a Python-wrapped launch (tens of microseconds), whose eager
    timing would measure the host.  check(), if given, runs after the
    timed replay (e.g. the outputs against an eager call)."""
    import torch

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(reps):
            fn()
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    g.replay()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    if check is not None:
        check()
    del g
    return ms


def time_backward(fa, w, q, k, v, o, lse, steps, warmup):
    """fa_bwd (its three kernels) on one workload, inputs and the forward's
    outputs resident; FLOPs 2.5x the forward's (five N x N x d products
    instead of two), halved for the causal mask like the forward."""
    import numpy as np
    import torch

    import synthetic

    st = synthetic.full_storage(w.config_id, "do", w.B, w.H, w.N, w.d, w.dtype)
    do = torch.from_numpy(st.view(np.int16)).view(torch.bfloat16).to(q.device)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    ws = torch.empty(fa.bwd_workspace_bytes(w.B, w.H, w.N, w.d), dtype=torch.uint8, device=q.device)
    fa.fwd(q, k, v, causal=w.causal, scale=w.scale, out=o, lse=lse)

    def step():
        fa.bwd(q, k, v, o, lse, do, causal=w.causal, scale=w.scale, dq=dq, dk=dk, dv=dv, workspace=ws)

    prewarm(step)
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(steps):
        step()
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / steps
    f = 2.5 * attention_flops(w.B, w.H, w.N, w.d, w.causal)
    return {"ms": round(ms, 4), "TFLOP/s": round(f / (ms * 1e-3) / 1e12, 2),
            "flops_per_call": f, "kernels": "bwd_pre + bwd_dkdv + bwd_dq"}


def time_gqa(fa, steps=10, warmup=2):
    """Grouped key/value heads: causal forward B8 H32 Hkv8 N8192 d128 and
    forward + backward B2 H16 Hkv4 N4096 d128 (FLOPs as for H heads)."""
    import numpy as np
    import torch

    import synthetic

    out = {}
    dev = torch.device("cuda:0")

    def tens(cid, t, B, H, N, d):
        st = synthetic.full_storage(cid, t, B, H, N, d, "bf16", threads=16)
        return torch.from_numpy(st.view(np.int16)).view(torch.bfloat16).to(dev)

    for (B, H, Hkv, N, d, with_bwd) in ((8, 32, 8, 8192, 128, False), (2, 16, 4, 4096, 128, True)):
        q, do = tens(3, "q", B, H, N, d), tens(3, "do", B, H, N, d)
        k, v = tens(3, "k", B, Hkv, N, d), tens(3, "v", B, Hkv, N, d)
        o = torch.empty_like(q)
        lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
        scale = 1.0 / math.sqrt(d)
        f = attention_flops(B, H, N, d, True)
        label = f"causal bf16 B{B} H{H} Hkv{Hkv} N{N} d{d}"

        def timed(fn):
            prewarm(fn)
            for _ in range(warmup):
                fn()
            torch.cuda.synchronize()
            t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            t0.record()
            for _ in range(steps):
                fn()
            t1.record()
            torch.cuda.synchronize()
            return t0.elapsed_time(t1) / steps

        ms = timed(lambda: fa.fwd(q, k, v, causal=True, scale=scale, out=o, lse=lse))
        out[f"{label} fwd"] = {"ms": round(ms, 4), "TFLOP/s": round(f / (ms * 1e-3) / 1e12, 2)}
        if with_bwd:
            dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(k)
            ws = torch.empty(fa.bwd_gqa_workspace_bytes(B, H, Hkv, N, d), dtype=torch.uint8, device=dev)
            ms = timed(lambda: fa.bwd(q, k, v, o, lse, do, causal=True, scale=scale, dq=dq, dk=dk, dv=dv,
                                      workspace=ws))
            out[f"{label} bwd"] = {"ms": round(ms, 4), "TFLOP/s": round(2.5 * f / (ms * 1e-3) / 1e12, 2)}
        del q, k, v, do, o, lse
        torch.cuda.empty_cache()
    return out


def time_f32(fa, steps=10, warmup=2):
    """float32 legs: the single-head workload B1 H1 N256 d64 non-causal
    (the small-grid VALU kernel), graph-timed (a launch-latency case), and
    B2 H16 N4096 d64 non-causal (the fp32 matrix-core kernel) for
    throughput, against the fp32 peak."""
    import torch

    import synthetic

    out = {}
    dev = torch.device("cuda:0")
    for (B, H, N, d, graph) in ((1, 1, 256, 64, True), (2, 16, 4096, 64, False)):
        q, k, v = (torch.from_numpy(synthetic.full_storage(1, t, B, H, N, d, "f32", threads=16)).to(dev)
                   for t in ("q", "k", "v"))
        o = torch.empty_like(q)
        lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
        scale = 1.0 / math.sqrt(d)
        call = lambda: fa.fwd(q, k, v, causal=False, scale=scale, out=o, lse=lse)
        f = attention_flops(B, H, N, d, False)
        prewarm(call)
        if graph:
            ms = graph_ms(call, 100)
        else:
            for _ in range(warmup):
                call()
            torch.cuda.synchronize()
            t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            t0.record()
            for _ in range(steps):
                call()
            t1.record()
            torch.cuda.synchronize()
            ms = t0.elapsed_time(t1) / steps
        tf = f / (ms * 1e-3) / 1e12
        out[f"non-causal fp32 fwd B{B} H{H} N{N} d{d}"] = {
            "ms": round(ms, 4), "TFLOP/s": round(tf, 2), "frac_of_fp32_peak": round(tf / PEAK_FP32_TFLOPS, 4),
            "timing": "HIP graph of 100 launches" if graph else "events around 10 launches"}
        del q, k, v, o, lse
        torch.cuda.empty_cache()
    return out


def time_f16(fa, steps=10, warmup=2):
    """float16 legs: causal forward B8 H32 N8192 d128, backward B2 H16 N4096
    d128 and decode B8 H32 N32768 d128 (inputs seeded like the bf16
    workloads, rounded to fp16)."""
    import numpy as np
    import torch

    import synthetic

    out = {}
    dev = torch.device("cuda:0")

    def timed(fn):
        prewarm(fn)
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record()
        for _ in range(steps):
            fn()
        t1.record()
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / steps

    def tens(cid, t, B, H, N, d):
        return torch.from_numpy(synthetic.full_storage(cid, t, B, H, N, d, "f16", threads=16)).to(dev)

    for (B, H, N, d, with_bwd) in ((8, 32, 8192, 128, False), (2, 16, 4096, 128, True)):
        q, k, v = (tens(3, t, B, H, N, d) for t in ("q", "k", "v"))
        o = torch.empty_like(q)
        lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
        scale = 1.0 / math.sqrt(d)
        f = attention_flops(B, H, N, d, True)
        ms = timed(lambda: fa.fwd(q, k, v, causal=True, scale=scale, out=o, lse=lse))
        out[f"causal fp16 fwd B{B} H{H} N{N} d{d}"] = {"ms": round(ms, 4), "TFLOP/s": round(f / (ms * 1e-3) / 1e12, 2)}
        if with_bwd:
            do = tens(3, "do", B, H, N, d)
            dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
            ws = torch.empty(fa.bwd_workspace_bytes(B, H, N, d), dtype=torch.uint8, device=dev)
            ms = timed(lambda: fa.bwd(q, k, v, o, lse, do, causal=True, scale=scale, dq=dq, dk=dk, dv=dv,
                                      workspace=ws))
            out[f"causal fp16 bwd B{B} H{H} N{N} d{d}"] = {"ms": round(ms, 4),
                                                          "TFLOP/s": round(2.5 * f / (ms * 1e-3) / 1e12, 2)}
            del do, dq, dk, dv
        del q, k, v, o, lse
        torch.cuda.empty_cache()
    w = synthetic.DECODE_WORKLOADS[6]
    st = synthetic.decode_storage(w.config_id, w.B, w.H, w.Hkv, w.N, w.d, 16, dtype="f16")
    q, k, v = (torch.from_numpy(st[t]).to(dev) for t in ("q", "k", "v"))
    del st
    r = time_decode(fa, w, q, k, v, 0, steps, warmup)
    out["decode fp16 B8 H32 N32768 d128 split-K"] = r
    del q, k, v
    torch.cuda.empty_cache()
    return out


def time_fp8(fa, steps=10, warmup=3, shapes=((8, 32, 8192, 128), (2, 16, 4096, 128))):
    """fa_fwd_fp8 (e4m3 inputs, bf16 output) on B8 H32 N8192 d128 and
    B2 H16 N4096 d128 causal; FLOPs counted as for the bf16 forward."""
    import numpy as np
    import torch

    import synthetic

    out = {}
    for (B, H, N, d) in shapes:
        w = synthetic.Workload(3, "", B, H, N, d, "e4m3", True)
        q, k, v = (torch.from_numpy(synthetic.full_storage(w.config_id, t, B, H, N, d, "e4m3", threads=16)).cuda()
                   for t in ("q", "k", "v"))
        o = torch.empty((B, H, N, d), dtype=torch.bfloat16, device=q.device)
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
        ds = synthetic.E4M3_DESCALE

        def step():
            fa.fwd_fp8(q, k, v, ds, ds, ds, causal=True, scale=w.scale, out=o, lse=lse)

        prewarm(step)
        for _ in range(warmup):
            step()
        torch.cuda.synchronize()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record()
        for _ in range(steps):
            step()
        t1.record()
        torch.cuda.synchronize()
        ms = t0.elapsed_time(t1) / steps
        out[f"causal fp8 (e4m3) fwd B{B} H{H} N{N} d{d}"] = {
            "ms": round(ms, 4), "TFLOP/s": round(attention_flops(B, H, N, d, True) / (ms * 1e-3) / 1e12, 2)}
        del q, k, v, o, lse
        torch.cuda.empty_cache()
    return out


def varlen_lengths(seed=0xFA0, B=16, lo=256, hi=8192):
    """Seeded sequence lengths of a packed batch: log-uniform in [lo, hi]."""
    import numpy as np

    rng = np.random.Generator(np.random.PCG64([0xFA, 50, seed]))
    return np.exp(rng.uniform(np.log(lo), np.log(hi), size=B)).astype(np.int64)


def time_varlen(fa, steps=10, warmup=2):
    """Packed variable-length causal forward (16 sequences of seeded
    log-uniform lengths in 256..8192, H32 d128 bf16) against the same
    sequences padded to the longest one (fixed-length call on B16 Nmax);
    TFLOP/s count only the sequences' own causal FLOPs in both."""
    import numpy as np
    import torch

    lens = varlen_lengths()
    total, nmax, B, H, d = int(lens.sum()), int(lens.max()), len(lens), 32, 128
    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev).manual_seed(0xFA51)
    q, k, v = (torch.randn(H, total, d, generator=gen, device=dev).to(torch.bfloat16) for _ in range(3))
    cu = torch.from_numpy(np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)).to(dev)
    o = torch.empty_like(q)
    lse = torch.empty((H, total), dtype=torch.float32, device=dev)
    f = sum(attention_flops(1, H, int(n), d, True) for n in lens)

    def timed(fn):
        prewarm(fn)
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record()
        for _ in range(steps):
            fn()
        t1.record()
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / steps

    ms_v = timed(lambda: fa.fwd_varlen(q, k, v, cu, nmax, causal=True, out=o, lse=lse))
    do = torch.randn(H, total, d, generator=gen, device=dev).to(torch.bfloat16)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(fa.bwd_varlen_workspace_bytes(H, total, d), dtype=torch.uint8, device=dev)
    ms_b = timed(lambda: fa.bwd_varlen(q, k, v, o, lse, do, cu, nmax, causal=True, dq=dq, dk=dk, dv=dv,
                                       workspace=ws))
    del q, k, v, o, lse, do, dq, dk, dv, ws
    torch.cuda.empty_cache()
    qp, kp, vp = (torch.randn(B, H, nmax, d, generator=gen, device=dev).to(torch.bfloat16) for _ in range(3))
    op = torch.empty_like(qp)
    lp = torch.empty((B, H, nmax), dtype=torch.float32, device=dev)
    ms_p = timed(lambda: fa.fwd(qp, kp, vp, causal=True, out=op, lse=lp))
    del qp, kp, vp, op, lp
    torch.cuda.empty_cache()
    label = f"causal bf16 varlen fwd B{B} H{H} d{d} total {total} (max {nmax})"
    return {label: {"ms": round(ms_v, 4), "TFLOP/s": round(f / (ms_v * 1e-3) / 1e12, 2),
                    "padded_ms": round(ms_p, 4), "padded_useful_TFLOP/s": round(f / (ms_p * 1e-3) / 1e12, 2),
                    "inputs": "torch.randn seeded on the device (values do not affect the timing)"},
            label.replace("fwd", "bwd"): {"ms": round(ms_b, 4), "TFLOP/s": round(2.5 * f / (ms_b * 1e-3) / 1e12, 2)}}


def decode_inputs(w, threads=16):
    import numpy as np
    import torch

    import synthetic

    st = synthetic.decode_storage(w.config_id, w.B, w.H, w.Hkv, w.N, w.d, threads)
    return [torch.from_numpy(st[t].view(np.int16)).view(torch.bfloat16).cuda() for t in ("q", "k", "v")]


def decode_bytes(w):
    """Compulsory HBM bytes of one decode call: read K, V and q, write o
    and lse."""
    return 2 * w.B * w.Hkv * w.N * w.d * 2 + 2 * w.B * w.H * w.d * 2 + 4 * w.B * w.H


def time_decode(fa, w, q, k, v, num_splits, steps, warmup):
    """fa_decode (split kernel + combine kernel) on one decode workload with
    inputs resident; GB/s of compulsory bytes against the 8 TB/s HBM peak."""
    import torch

    splits, chunk, need = fa.decode_plan(w.B, w.H, w.Hkv, w.N, w.d, num_splits)
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H), dtype=torch.float32, device=q.device)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)

    def step():
        fa.decode(q, k, v, scale=w.scale, num_splits=num_splits, out=o, lse=lse, workspace=ws)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(steps):
        step()
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / steps
    gbs = decode_bytes(w) / (ms * 1e-3) / 1e9
    return {"ms": round(ms, 4), "GB/s": round(gbs, 1), "frac_of_hbm_peak": round(gbs / PEAK_HBM_GBS, 3),
            "splits": splits, "keys_per_split": chunk, "bytes_per_call": decode_bytes(w),
            "kernels": "decode_split + decode_combine"}


def time_default_legs(fa):
    """The other measured workloads, in every default run (after the headline
    leg, outside its timed region): causal bf16 forward on B1 H16 N2048 d64,
    B8 H32 N8192 d64, B1 H16 N32768 d128 (batch-1 long context) and B2 H16
    N4096 d128, the
    backward of the last and of B2 H8 N4096 d256, split-K decode on B8
    H32 N32768 d128, and the e4m3 forward on B8 H32 N8192 d128.  Inputs are the seeded workloads of the parity tests
    (the d256 one drawn the same way); each leg frees its tensors."""
    import dataclasses

    import torch

    import synthetic

    legs = {}
    w256 = dataclasses.replace(synthetic.WORKLOADS[5], config_id=9400, name="causal bf16 backward B2 H8 N4096 d256",
                               H=8, d=256)
    w64 = dataclasses.replace(synthetic.WORKLOADS[3], config_id=4500, name="causal bf16 B8 H32 N8192 d64", d=64)
    for cid in (2, 64, 4, 5, 256):
        ww = {256: w256, 64: w64}.get(cid) or synthetic.WORKLOADS[cid]
        qq, kk, vv = make_inputs(ww)
        oo = torch.empty_like(qq)
        ll = torch.empty((ww.B, ww.H, ww.N), dtype=torch.float32, device=qq.device)
        steps = 50 if cid == 2 else 20
        if cid != 256:
            prewarm(lambda: fa.fwd(qq, kk, vv, causal=True, scale=ww.scale, out=oo, lse=ll))
            _, msk, mn, mx, _ = time_launches(fa, qq, kk, vv, oo, ll, True, ww.scale, steps, 3)
            f = attention_flops(ww.B, ww.H, ww.N, ww.d, True)
            leg = {"ms": round(msk, 4), "min_ms": round(mn, 4), "max_ms": round(mx, 4)}
            if msk < 0.5:
                # short kernel: the eager per-launch events include the host's
                # launch cost; time a graph of back-to-back launches instead,
                # and check its output against the eager call's bits
                ref = oo.clone()

                def same():
                    assert torch.equal(oo.view(torch.int16), ref.view(torch.int16)), "graph replay output differs"

                msk = graph_ms(lambda: fa.fwd(qq, kk, vv, causal=True, scale=ww.scale, out=oo, lse=ll), 100, same)
                leg = {"ms": round(msk, 4), "eager_ms": leg["ms"], "timing": "HIP graph of 100 launches"}
            tf = f / (msk * 1e-3) / 1e12
            leg.update({"TFLOP/s": round(tf, 2), "frac_of_peak": round(tf / PEAK_BF16_TFLOPS, 4), "flops_per_call": f})
            legs[f"causal bf16 fwd B{ww.B} H{ww.H} N{ww.N} d{ww.d}"] = leg
        if cid in (5, 256):
            r = time_backward(fa, ww, qq, kk, vv, oo, ll, 20, 3)
            r["frac_of_peak"] = round(r["TFLOP/s"] / PEAK_BF16_TFLOPS, 4)
            legs[f"causal bf16 bwd B{ww.B} H{ww.H} N{ww.N} d{ww.d}"] = r
        del qq, kk, vv, oo, ll
        torch.cuda.empty_cache()
    dw = synthetic.DECODE_WORKLOADS[6]
    dq_, dk_, dv_ = decode_inputs(dw)
    # 200 untimed calls: the first ~100 calls after the inputs are copied in
    # run up to 10 % slower
    legs[f"{dw.name} split-K"] = time_decode(fa, dw, dq_, dk_, dv_, 0, 50, 200)
    del dq_, dk_, dv_
    torch.cuda.empty_cache()
    # the e4m3 forward on the headline shape (its B2 H16 N4096 leg and the
    # fp32 legs run under --extra)
    legs.update(time_fp8(fa, shapes=((8, 32, 8192, 128),)))
    return legs


def device_sysfs(torch):
    """sysfs directory of the GPU torch calls cuda:0 (from its PCI address),
    or None where it is not readable."""
    p = torch.cuda.get_device_properties(0)
    bus = getattr(p, "pci_bus_id", None)
    if bus is None:
        return None
    path = "/sys/bus/pci/devices/%04x:%02x:%02x.0" % (getattr(p, "pci_domain_id", 0), bus,
                                                      getattr(p, "pci_device_id", 0))
    return path if os.path.exists(os.path.join(path, "pp_dpm_sclk")) else None


def read_sclk_mhz(path):
    """Current shader clock: pp_dpm_sclk lists the levels and marks the
    running one (or the actual frequency, on an 'S:' line) with '*'."""
    try:
        with open(os.path.join(path, "pp_dpm_sclk")) as f:
            for line in f:
                if "*" in line:
                    m = re.search(r"(\d+)\s*mhz", line, re.I)
                    return int(m.group(1)) if m else None
    except OSError:
        return None
    return None


def read_hwmon(path, name):
    """A hwmon value of the device (power in microwatts), or None."""
    import glob

    for f in glob.glob(os.path.join(path, "hwmon", "hwmon*", name)):
        try:
            with open(f) as fh:
                return int(fh.read().strip())
        except (OSError, ValueError):
            return None
    return None


class ClockSampler:
    """Reads the shader clock and the average power from sysfs every
    `period` seconds on a host thread while GPU work runs."""

    def __init__(self, path, period=0.005):
        self.path, self.period = path, period
        self.sclk, self.power = [], []
        self._stop = threading.Event()
        self._thread = threading.Thread(target=self._run, daemon=True)

    def _run(self):
        while not self._stop.is_set():
            c = read_sclk_mhz(self.path)
            if c is not None:
                self.sclk.append(c)
            pw = read_hwmon(self.path, "power1_average")
            if pw is None:
                pw = read_hwmon(self.path, "power1_input")
            if pw is not None:
                self.power.append(pw / 1e6)
            time.sleep(self.period)

    def __enter__(self):
        if self.path:
            self._thread.start()
        return self

    def __exit__(self, *exc):
        if self.path:
            self._stop.set()
            self._thread.join()

    def summary(self):
        if not self.sclk:
            return None
        out = {"median": statistics.median(self.sclk), "min": min(self.sclk), "max": max(self.sclk),
               "samples": len(self.sclk)}
        if self.power:
            out["power_w_median"] = round(statistics.median(self.power), 1)
        return out


def sustained_clock(fa, torch, path, q, k, v, o, lse, scale, seconds=1.0):
    """Shader clock sampled while fa_fwd launches run back to back for about
    `seconds` (outside the timed region)."""
    if path is None:
        return None
    fa.fwd(q, k, v, causal=True, scale=scale, out=o, lse=lse)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    with ClockSampler(path) as cs:
        while time.perf_counter() - t0 < seconds:
            for _ in range(25):
                fa.fwd(q, k, v, causal=True, scale=scale, out=o, lse=lse)
            torch.cuda.synchronize()
    return cs.summary()


def mfma_ceiling(fa, torch, path, iters=1000, blocks=2048, seconds=1.0):
    """Rate of the matrix-core-only kernel (dense bf16 MFMA, no memory
    traffic) run back to back for about `seconds`, with the shader clock
    sampled meanwhile."""
    sink = torch.empty(blocks * 256, dtype=torch.float32, device="cuda:0")
    for _ in range(2):
        fa.mfma_ceiling(sink, iters, blocks)
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    total_ms, calls = 0.0, 0
    t0 = time.perf_counter()
    with ClockSampler(path) as cs:
        while time.perf_counter() - t0 < seconds:
            a.record()
            for _ in range(20):
                fa.mfma_ceiling(sink, iters, blocks)
            b.record()
            torch.cuda.synchronize()
            total_ms += a.elapsed_time(b)
            calls += 20
    ms = total_ms / calls
    flops = fa.MFMA_CEILING_FLOP_PER_ITER_BLOCK * iters * blocks
    out = {"TFLOP/s": round(flops / (ms * 1e-3) / 1e12, 1), "ms": round(ms, 3), "calls": calls,
           "kernel": f"fa_mfma_ceiling: {blocks} workgroups x 4 waves x {iters} x 4 v_mfma_f32_32x32x16_bf16"}
    clk = cs.summary()
    if clk:
        out["sclk_mhz"] = clk
    return out


def cold_cache(fa, torch, q, k, v, o, lse, scale, launches=10):
    """fa_fwd time with 1 GiB written between launches (flushes the 256 MB
    Infinity Cache and the L2s); only the forward is inside the events."""
    scratch = torch.empty(1 << 28, dtype=torch.float32, device=q.device)
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(launches)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(launches)]
    for i in range(launches):
        scratch.fill_(float(i))
        starts[i].record()
        fa.fwd(q, k, v, causal=True, scale=scale, out=o, lse=lse)
        ends[i].record()
    torch.cuda.synchronize()
    per = [s_.elapsed_time(e) for s_, e in zip(starts, ends)]
    del scratch
    return statistics.median(per)


def cpu_per_core(w_id, budget_s=4.0):
    """The oracle on one host thread, in a child process whose BLAS pools
    are limited to one thread before NumPy loads (no GPU use)."""
    env = dict(os.environ, OMP_NUM_THREADS="1", OPENBLAS_NUM_THREADS="1", MKL_NUM_THREADS="1",
               BLIS_NUM_THREADS="1")
    try:
        r = subprocess.run([sys.executable, os.path.abspath(__file__), "--cpu-per-core", str(w_id),
                            str(budget_s)], env=env, capture_output=True, text=True, timeout=120)
        return json.loads(r.stdout.strip().splitlines()[-1])
    except Exception as e:  # reported, never fatal for the GPU measurement
        return {"error": repr(e)[:200]}


def cpu_baseline(w, budget_s=12.0, rows_per_head=512):
    """The fp64 oracle on the host cores over a bounded sample of the same
    workload: seeded (b, h) heads, 512 seeded query rows each, until the
    time budget is spent (at least one head)."""
    import numpy as np

    import oracle
    import synthetic

    try:
        from threadpoolctl import threadpool_info

        threads = max((p.get("num_threads", 1) for p in threadpool_info()), default=1)
    except Exception:
        threads = len(os.sched_getaffinity(0))
    heads = synthetic.sample_heads(w.config_id, w.B, w.H, w.B * w.H)
    rows = synthetic.sample_rows(w.config_id, w.N, rows_per_head)
    flops = 0.0
    spent = 0.0
    done = 0
    for b, h in heads:
        q, k, v = (synthetic.head_values(w.config_id, t, b, h, w.N, w.d, w.dtype) for t in ("q", "k", "v"))
        t0 = time.perf_counter()
        oracle.naive_attention(q, k, v, w.causal, w.scale, rows=rows)
        spent += time.perf_counter() - t0
        flops += causal_row_flops(rows, w.d) if w.causal else 4.0 * w.d * w.N * len(rows)
        done += 1
        if spent >= budget_s:
            break
    return {
        "value": flops / spent / 1e12,
        "unit": "TFLOP/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": f"{done} seeded heads x {len(rows)} seeded query rows of B={w.B} H={w.H} N={w.N} "
                  f"d={w.d} causal (naive fp64 NumPy, materialised score rows); {spent:.1f} s",
        "seconds": spent,
        "extrapolated_full_workload_s": round(
            attention_flops(w.B, w.H, w.N, w.d, w.causal) / (flops / spent), 1),
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-legs", action="store_true",
                    help="skip the other workloads' legs (profiling runs: some legs launch the headline kernel)")
    ap.add_argument("--extra", action="store_true", help="also time the other workloads and non-causal")
    ap.add_argument("--profile-run", action="store_true")
    ap.add_argument("--profile-decode", action="store_true",
                    help="run --steps fa_decode calls on B=8 H=32 N=32768 d=128 (for rocprofv3)")
    ap.add_argument("--profile-decode-gqa", action="store_true",
                    help="run --steps fa_decode calls on B=8 H=64 Hkv=8 N=32768 d=128 (the MFMA decode)")
    ap.add_argument("--profile-fp8", action="store_true",
                    help="run the fp8 legs (B8 H32 N8192 and B2 H16 N4096 d=128 causal, for rocprofv3)")
    ap.add_argument("--profile-bwd", action="store_true",
                    help="run --steps fa_bwd calls on B=2 H=16 N=4096 d=128 causal (for rocprofv3)")
    ap.add_argument("--cpu-per-core", nargs=2, metavar=("WORKLOAD", "SECONDS"), help=argparse.SUPPRESS)
    args = ap.parse_args()
    if args.cpu_per_core:
        import synthetic

        r = cpu_baseline(synthetic.WORKLOADS[int(args.cpu_per_core[0])], budget_s=float(args.cpu_per_core[1]))
        print(json.dumps({"value": r["value"], "unit": r["unit"], "cores": r["cores"], "sample": r["sample"]}), flush=True)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the attention forward is sharded over heads with no "
              f"communication, and the benchmark runs on a single MI355X; --gpus {args.gpus} is not "
              f"supported.", file=sys.stderr)
        sys.exit(2)

    import torch

    import aware_softmax_amd as fa
    import synthetic

    if args.profile_decode:
        dw = synthetic.DECODE_WORKLOADS[6]
        dq_, dk_, dv_ = decode_inputs(dw)
        r = time_decode(fa, dw, dq_, dk_, dv_, 0, args.steps, 2)
        print(json.dumps({"profile-decode": dw.name, **r}), flush=True)
        return

    if args.profile_decode_gqa:
        dw = synthetic.DecodeWorkload(8, "decode bf16 B8 H64 Hkv8 N32768 d128", 8, 64, 8, 32768, 128)
        dq_, dk_, dv_ = decode_inputs(dw)
        r = time_decode(fa, dw, dq_, dk_, dv_, 0, args.steps, 2)
        print(json.dumps({"profile-decode-gqa": dw.name, **r}), flush=True)
        return

    if args.profile_fp8:
        print(json.dumps({"profile-fp8": time_fp8(fa, steps=args.steps, warmup=2)}), flush=True)
        return

    if args.profile_bwd:
        wb = synthetic.WORKLOADS[5]
        qq, kk, vv = make_inputs(wb)
        oo = torch.empty_like(qq)
        ll = torch.empty((wb.B, wb.H, wb.N), dtype=torch.float32, device=qq.device)
        r = time_backward(fa, wb, qq, kk, vv, oo, ll, args.steps, 2)
        print(json.dumps({"profile-bwd": wb.name, **r}), flush=True)
        return

    w = synthetic.WORKLOADS[3]
    q, k, v = make_inputs(w)
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=q.device)

    if args.profile_run:
        src = torch.empty(1 << 29, dtype=torch.int16, device=q.device)  # 1 GiB
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        for _ in range(args.steps):
            fa.fwd(q, k, v, causal=True, scale=w.scale, out=o, lse=lse)
        torch.cuda.synchronize()
        print(f"profile-run: 1 GiB copy + {args.steps} fa_fwd launches done", flush=True)
        return

    # the device's clock under the forward, sampled over 1 s of back-to-back
    # launches; it also brings the device to its steady state before the
    # timed steps (see prewarm)
    path = device_sysfs(torch)
    clock = sustained_clock(fa, torch, path, q, k, v, o, lse, w.scale)
    if path is None:
        prewarm(lambda: fa.fwd(q, k, v, causal=True, scale=w.scale, out=o, lse=lse), 1000.0)
    ms_step, ms_kernel, ms_min, ms_max, wall = time_launches(
        fa, q, k, v, o, lse, True, w.scale, args.steps, args.warmup)
    flops = attention_flops(w.B, w.H, w.N, w.d, True)
    tflops = flops / (ms_step * 1e-3) / 1e12
    achieved = flops / (ms_kernel * 1e-3) / 1e12
    per_launch = time_launches.last_per_launch
    bq, bk, waves = fa.tile_config(w.d, fa.DTYPE_BF16)
    traffic = read_traffic()
    props = torch.cuda.get_device_properties(0)
    ceiling = mfma_ceiling(fa, torch, path)
    cold_ms = cold_cache(fa, torch, q, k, v, o, lse, w.scale)
    power_cap = read_hwmon(path, "power1_cap") if path else None
    result = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "causal bf16 attention forward B=8 H=32 N=8192 d=128 scale=1/sqrt(d)",
            "B": w.B, "H": w.H, "N": w.N, "d": w.d, "causal": True,
            "tile": {"block_q": bq, "block_k": bk, "waves": waves},
            "inputs": "i.i.d. N(0,1) fp32 rounded to bf16, seeded per head",
        },
        "frac_of_peak": round(tflops / PEAK_BF16_TFLOPS, 4),
        "roofline": {
            "bound": "mfma",
            "achieved": round(achieved, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
            "traffic": traffic,
            "kernel_ms": {"mean": round(ms_kernel, 4), "median": round(statistics.median(per_launch), 4),
                          "min": round(ms_min, 4), "max": round(ms_max, 4)},
            "flops_per_launch": flops,
            "mfma_ceiling": dict(ceiling, frac=round(achieved / ceiling["TFLOP/s"], 4)),
            "traffic_models": traffic_models(w, bq),
        },
        "cold_cache": {"ms": round(cold_ms, 4), "TFLOP/s": round(flops / (cold_ms * 1e-3) / 1e12, 2),
                       "how": "1 GiB device write between launches, median of 10"},
        "device": {
            "name": props.name, "arch": getattr(props, "gcnArchName", None),
            "cu_count": props.multi_processor_count,
            "sclk_mhz_under_fwd": clock,
            "power_cap_w": round(power_cap / 1e6, 1) if power_cap else None,
        },
    }
    del q, k, v, o, lse
    torch.cuda.empty_cache()
    if not args.no_legs:
        result["workloads"] = time_default_legs(fa)
    if args.extra:
        extra = {}
        for cid in (2, 4, 5):
            ww = synthetic.WORKLOADS[cid]
            qq, kk, vv = make_inputs(ww)
            oo = torch.empty_like(qq)
            ll = torch.empty((ww.B, ww.H, ww.N), dtype=torch.float32, device=qq.device)
            prewarm(lambda: fa.fwd(qq, kk, vv, causal=True, scale=ww.scale, out=oo, lse=ll))
            ms, msk, _, _, _ = time_launches(fa, qq, kk, vv, oo, ll, True, ww.scale, 20, 3)
            f = attention_flops(ww.B, ww.H, ww.N, ww.d, True)
            label = f"causal bf16 fwd B{ww.B} H{ww.H} N{ww.N} d{ww.d}"
            extra[label] = {"ms": round(msk, 4), "TFLOP/s": round(f / (msk * 1e-3) / 1e12, 2)}
            if cid == 5:
                extra[f"causal bf16 bwd B{ww.B} H{ww.H} N{ww.N} d{ww.d}"] = time_backward(
                    fa, ww, qq, kk, vv, oo, ll, 20, 3)
                for d in (32, 64, 96):  # the other backward head dims, same shape otherwise
                    hw = synthetic.Workload(5, "", ww.B, ww.H, ww.N, d, "bf16", True)
                    q2, k2, v2 = make_inputs(hw)
                    o2 = torch.empty_like(q2)
                    l2 = torch.empty((hw.B, hw.H, hw.N), dtype=torch.float32, device=q2.device)
                    extra[f"causal bf16 bwd B{hw.B} H{hw.H} N{hw.N} d{d}"] = time_backward(
                        fa, hw, q2, k2, v2, o2, l2, 20, 3)
                    del q2, k2, v2, o2, l2
            del qq, kk, vv, oo, ll
            torch.cuda.empty_cache()
        qq, kk, vv = make_inputs(w)
        oo = torch.empty_like(qq)
        ll = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=qq.device)
        prewarm(lambda: fa.fwd(qq, kk, vv, causal=False, scale=w.scale, out=oo, lse=ll))
        ms, msk, _, _, _ = time_launches(fa, qq, kk, vv, oo, ll, False, w.scale, 10, 2)
        f = attention_flops(w.B, w.H, w.N, w.d, False)
        extra["non-causal bf16 B8 H32 N8192 d128"] = {
            "ms": round(msk, 4), "TFLOP/s": round(f / (msk * 1e-3) / 1e12, 2),
            "causal_speedup_time_ratio": round(msk / ms_kernel, 3)}
        del qq, kk, vv, oo, ll
        torch.cuda.empty_cache()
        # other head dims and grouped key/value heads (seeded like workload 3)
        for d in (32, 64, 96, 256):
            hw = synthetic.Workload(3, "", 8, 32, 8192, d, "bf16", True)
            qq, kk, vv = make_inputs(hw)
            oo = torch.empty_like(qq)
            ll = torch.empty((hw.B, hw.H, hw.N), dtype=torch.float32, device=qq.device)
            prewarm(lambda: fa.fwd(qq, kk, vv, causal=True, scale=hw.scale, out=oo, lse=ll))
            ms, msk, _, _, _ = time_launches(fa, qq, kk, vv, oo, ll, True, hw.scale, 10, 2)
            f = attention_flops(hw.B, hw.H, hw.N, hw.d, True)
            extra[f"causal bf16 fwd B8 H32 N8192 d{d}"] = {"ms": round(msk, 4),
                                                           "TFLOP/s": round(f / (msk * 1e-3) / 1e12, 2)}
            del qq, kk, vv, oo, ll
            torch.cuda.empty_cache()
        extra.update(time_gqa(fa))
        extra.update(time_f16(fa))
        extra.update(time_f32(fa))
        extra.update(time_fp8(fa))
        extra.update(time_varlen(fa))
        gqa8 = synthetic.DecodeWorkload(8, "decode bf16 B8 H64 Hkv8 N32768 d128", 8, 64, 8, 32768, 128)
        for dw in [synthetic.DECODE_WORKLOADS[cid] for cid in (6, 7, 8)] + [gqa8]:
            dq_, dk_, dv_ = decode_inputs(dw)
            for ns, tag in ((0, "split-K"), (1, "unsplit")):
                # 200 untimed calls: the first ~100 calls after the inputs
                # are copied in run up to 10 % slower
                extra[f"{dw.name} {tag}"] = time_decode(fa, dw, dq_, dk_, dv_, ns, 20, 200)
            del dq_, dk_, dv_
            torch.cuda.empty_cache()
        result["other_workloads"] = extra
    if not args.no_cpu:
        result["cpu_baseline"] = cpu_baseline(w)
        result["cpu_baseline"]["per_core"] = cpu_per_core(w.config_id)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
