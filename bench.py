#!/usr/bin/env python3
"""Benchmark of the retention operator on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--no-secondary]
                    [--only NAME] [--calib-copy] [--calib-mfma]

Headline workload (one "step" = one chunkwise forward over one batch, i.e. every stage
of the chunkwise hot path: tile staging, decay generation, intra-chunk scores and
P V, the cross-chunk term, the state carry, and the output store):
    train_bf16: B=4 H=8 N=2048 d_k=256 d_v=512 chunk=64, bf16 in / fp32 accumulate,
    gamma_h = 1 - 2^(-5-h).
Throughput is tokens/s = B*N / step time, with inputs resident in HBM.  Several
input sets are rotated so a step never finds its inputs in the 256 MB MALL left
over from the previous step.

Secondary lines (same JSON object, "secondary"): the recurrent decode step, per head and
gated (batch 128, H=32, d=128, 1024 consecutive steps, GB/s of the fp32 state stream), the
long-sequence workload at chunk 128/256/512, the gated workload, the backward of the
train and gated workloads (with an initial state and a final-state gradient; GB/s
counts Q, K, V, dO read and dQ, dK, dV written once), the parallel form on short
sequences (with the chunkwise form on the same inputs beside it), and the gated
retention layer around the operator (B=4 N=2048 D=1024 H=8 d=128; TFLOP/s of its six
projections over the layer's time).

"roofline" describes the dominant kernel of the headline step, the single-block
matrix-core chunkwise pass (the headline's one launch per step): algorithmic bytes (Q,
K, V read once, O written once) per launch / its average launch time, measured with
HIP events the library records around each of its launches on the launch stream
(retention_profile_enable / retention_profile_read) over a second timed run of the
same steps, against 8 TB/s.  "traffic" is HBM bytes per launch from the committed
rocprofv3 FETCH_SIZE / WRITE_SIZE summary, scaled by the copy-kernel calibration
factor, and "mfma_busy_counter" the matrix-core busy fraction from the committed
rocprofv3 counters (SQ_VALU_MFMA_BUSY_CYCLES over GRBM_GUI_ACTIVE x SIMDs); both are
null when the kernel source changed since they were taken.
Every timed run is preceded by SETTLE_S (0.3 s) of untimed steps of the same workload and
then the W warmup steps: the GPU's first few hundred milliseconds of sustained work run
10-25% slower than its steady state.  The K timed steps are whole steps, unchanged.
"timing" adds per-call HIP-event times of the headline (median, minimum, mean, p90 over
at least 100 calls), back to back and with a 1 GiB write before each call that evicts
the inputs from the MALL and L2; the decode lines add the per-step distribution.
"achievable" is measured context: the library's matrix-core loop (no memory traffic)
and a plain device copy, against the spec peaks.
"cpu_baseline" times the fp64 oracle (recurrent form, numpy) on a bounded sample of
the same workload on the host.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "chunkwise retention fwd tokens/s & % MFMA peak; decode-step HBM GB/s"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2516.6
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "train_bf16_traffic.json")
# source of the headline's dominant kernel (the single-block chunkwise pass)
KERNEL_SRC = os.path.join(ROOT, "retnet_retention_fwd_amd", "csrc", "chunk64.hip")
HEADLINE_KERNEL = "chunk1_kernel<256, false, false, 0> (single-block matrix-core chunkwise pass)"


def kernel_hash() -> str:
    with open(KERNEL_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def alg_bytes(B, H, N, dk, dv, gated=False, elem=2):
    """Q, K, V read once and O written once (plus g for the gated form)."""
    return B * H * N * ((2 * dk + 2 * dv) * elem + (4 if gated else 0))


def alg_flops(B, H, N, dk, dv, C):
    """Causal chunkwise flops: (C+1)(dk+dv) + 4 dk dv per token-head."""
    return B * H * N * ((C + 1) * (dk + dv) + 4 * dk * dv)


# Untimed steps run for this long before a workload's warmup steps.  The GPU runs its
# first few hundred milliseconds of sustained work 10-25% slower than its steady state
# (measured on the headline: 79-97 us per step over the first 80 steps of a process,
# 73-75 us after 0.3 s of steps), so a short run would time that transient instead of
# the operator.
SETTLE_S = 0.3


def settle(fn, torch, seconds=SETTLE_S):
    """Run fn(0), fn(1), ... untimed until `seconds` of wall time have passed."""
    t0 = time.perf_counter()
    i = 0
    while time.perf_counter() - t0 < seconds:
        fn(i)
        i += 1
        if i % 16 == 0:
            torch.cuda.synchronize()   # keep the queue short, so the wall clock tracks the GPU
    torch.cuda.synchronize()
    return i


def time_steps(fn, steps, warmup, torch, settle_s=SETTLE_S):
    if settle_s > 0:
        settle(fn, torch, settle_s)
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    t0.record(stream)
    for i in range(steps):
        fn(i)
    t1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    return t0.elapsed_time(t1) / 1e3, wall     # seconds (events), seconds (host clock)


def stats(ms_list):
    """Median, minimum, mean and 90th percentile of per-call times (microseconds)."""
    xs = sorted(1e3 * x for x in ms_list)
    n = len(xs)
    return {"calls": n, "median_us": round(xs[n // 2], 3), "min_us": round(xs[0], 3),
            "mean_us": round(sum(xs) / n, 3), "p90_us": round(xs[min(n - 1, int(0.9 * n))], 3)}


def per_call_times(step, n, torch, flush_buf=None):
    """HIP-event time of each of n calls on the current stream (milliseconds).  With
    flush_buf, a write of that buffer (1 GiB) before each call, outside its events,
    evicts the inputs from the MALL and the L2."""
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for i in range(n):
        if flush_buf is not None:
            flush_buf.fill_(i & 0x7F)
        ev[i][0].record()
        step(i)
        ev[i][1].record()
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in ev]


def achievable(torch, R):
    """Achievable-peak context measured in this run: the library's matrix-core loop
    (bf16, no memory traffic) and a plain 1 GiB device copy (read + write)."""
    out = torch.empty(256 * 8, dtype=torch.float32, device="cuda")
    iters = 2000
    R.calib_mfma(256, 8, 50, out=out)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    flops = 0.0
    for _ in range(5):
        flops += R.calib_mfma(256, 8, iters, out=out)
    e1.record()
    torch.cuda.synchronize()
    mfma_tflops = flops / (e0.elapsed_time(e1) * 1e-3) / 1e12
    a = torch.empty(1 << 28, device="cuda")
    b = torch.empty_like(a)
    b.copy_(a)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(5):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    copy_gbps = 5 * 2 * a.numel() * 4 / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del a, b
    return {"mfma_loop_TFLOPs": round(mfma_tflops, 1), "mfma_loop_frac_of_spec": round(mfma_tflops / BF16_PEAK_TFLOPS, 4),
            "copy_GBps": round(copy_gbps, 1), "copy_frac_of_spec": round(copy_gbps / HBM_PEAK_GBS, 4),
            "what": "bf16 16x16x32 matrix-core loop (256 workgroups x 8 waves, 16 independent accumulators per "
                    "wave, no memory traffic); torch copy_ of 1 GiB fp32 (read + write bytes)"}


def chunk_inputs(torch, B, H, N, dk, dv, gated, sets, seed):
    """Seeded synthetic inputs on the GPU: Q,K,V ~ N(0,1)/sqrt(dk) in bf16; per-head
    gammas or g = logsigmoid(x)/16.  `sets` independent copies to rotate through."""
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    out = []
    s = 1.0 / math.sqrt(dk)
    for _ in range(sets):
        q = (torch.randn(B, H, N, dk, device="cuda", generator=g) * s).to(torch.bfloat16)
        k = (torch.randn(B, H, N, dk, device="cuda", generator=g) * s).to(torch.bfloat16)
        v = (torch.randn(B, H, N, dv, device="cuda", generator=g) * s).to(torch.bfloat16)
        if gated:
            d = torch.nn.functional.logsigmoid(torch.randn(B, H, N, device="cuda", generator=g)) / 16
        else:
            d = None
        o = torch.empty(B, H, N, dv, device="cuda", dtype=torch.bfloat16)
        out.append((q, k, v, d, o))
    return out


def run_chunk_workload(torch, R, name, B, H, N, dk, dv, C, gammas, gated, steps, warmup, seed,
                       kernel_times=False, dist_calls=0):
    per_set = alg_bytes(B, H, N, dk, dv, gated)
    sets = max(2, min(8, int(math.ceil(768e6 / per_set))))
    data = chunk_inputs(torch, B, H, N, dk, dv, gated, sets, seed)
    gm = torch.tensor(gammas, device="cuda", dtype=torch.float32) if not gated else None
    code = 1
    ws_bytes = R.workspace_bytes(B, H, N, dk, dv, C, code, gated)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device="cuda")

    def step(i):
        q, k, v, d, o = data[i % sets]
        if gated:
            R.gated_retention_chunkwise_fwd(q, k, v, d, C, out=o, workspace=ws)
        else:
            R.retention_chunkwise_fwd(q, k, v, gm, C, out=o, workspace=ws)

    t, wall = time_steps(step, steps, warmup, torch)
    kernels = None
    if kernel_times:
        # same steps again, each library launch bracketed by HIP events on its stream
        R.profile_enable(True)
        time_steps(step, steps, 0, torch, settle_s=0)
        prof = R.profile_read()
        R.profile_enable(False)
        kernels = {k: {"launches": v["launches"], "avg_us": round(1e3 * v["ms"] / v["launches"], 3)}
                   for k, v in prof.items() if k != "dropped" and v["launches"] > 0}
        kernels["dropped"] = prof["dropped"]
    dist = None
    if dist_calls > 0:
        # per-call times: back to back (inputs rotated as in the timed steps), and with
        # the MALL and L2 flushed by a 1 GiB write before each call
        flush = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        dist = {"unflushed": stats(per_call_times(step, dist_calls, torch)),
                "flushed": stats(per_call_times(step, dist_calls, torch, flush))}
        del flush
    per = t / steps
    nb = alg_bytes(B, H, N, dk, dv, gated)
    fl = alg_flops(B, H, N, dk, dv, C)
    return {
        "workload": name, "B": B, "H": H, "N": N, "dk": dk, "dv": dv, "chunk": C,
        "us_per_step": per * 1e6, "tokens_per_s": B * N / per,
        "alg_GBps": nb / per / 1e9, "hbm_frac": nb / per / 1e9 / HBM_PEAK_GBS,
        "alg_TFLOPs": fl / per / 1e12, "mfma_frac": fl / per / 1e12 / BF16_PEAK_TFLOPS,
        "input_sets": sets, "workspace_bytes": ws_bytes, "wall_s": wall, "kernels": kernels,
        "per_call": dist,
    }


def alg_bytes_bwd(B, H, N, dk, dv, gated=False, elem=2):
    """Backward: Q, K, V, dO read once; dQ, dK, dV written once (plus g read, dg written)."""
    return B * H * N * ((4 * dk + 3 * dv) * elem + (8 if gated else 0))


def run_bwd_workload(torch, R, name, B, H, N, dk, dv, C, gammas, gated, steps, warmup, seed):
    """Backward of a chunkwise workload with an initial state and a final-state gradient."""
    data = chunk_inputs(torch, B, H, N, dk, dv, gated, 2, seed)
    g = torch.Generator(device="cuda")
    g.manual_seed(seed + 100)
    grads = [torch.randn(B, H, N, dv, device="cuda", generator=g).to(torch.bfloat16) for _ in range(2)]
    s0 = torch.randn(B, H, dk, dv, device="cuda", generator=g) * 0.1
    ds = torch.randn(B, H, dk, dv, device="cuda", generator=g) * 0.1
    gm = torch.tensor(gammas, device="cuda", dtype=torch.float32) if not gated else None
    ws = torch.empty(max(R.bwd_workspace_bytes(B, H, N, dk, dv, C, 1, gated), 1), dtype=torch.uint8, device="cuda")

    def step(i):
        q, k, v, d, _ = data[i % 2]
        if gated:
            R.gated_retention_chunkwise_bwd(q, k, v, d, grads[i % 2], C, state_in=s0, grad_state_out=ds,
                                            return_grad_state_in=True, workspace=ws)
        else:
            R.retention_chunkwise_bwd(q, k, v, gm, grads[i % 2], C, state_in=s0, grad_state_out=ds,
                                      return_grad_state_in=True, workspace=ws)

    t, wall = time_steps(step, steps, warmup, torch)
    per = t / steps
    nb = alg_bytes_bwd(B, H, N, dk, dv, gated)
    fl = 3 * alg_flops(B, H, N, dk, dv, C)
    return {
        "workload": name + " backward", "B": B, "H": H, "N": N, "dk": dk, "dv": dv, "chunk": C,
        "us_per_step": per * 1e6, "tokens_per_s": B * N / per,
        "alg_GBps": nb / per / 1e9, "hbm_frac": nb / per / 1e9 / HBM_PEAK_GBS,
        "pass_TFLOPs": fl / per / 1e12, "wall_s": wall,
    }


def run_parallel_workload(torch, R, B, H, N, dk, dv, steps, warmup, seed):
    """Parallel form on a short sequence, per-head decays; the chunkwise form (chunk 64)
    on the same inputs is timed beside it."""
    data = chunk_inputs(torch, B, H, N, dk, dv, False, 2, seed)
    gm = torch.tensor([1.0 - 2.0 ** (-5.0 - i) for i in range(H)], device="cuda", dtype=torch.float32)
    outs = [torch.empty(B, H, N, dv, device="cuda", dtype=torch.bfloat16) for _ in range(2)]

    def par(i):
        q, k, v, _, _ = data[i % 2]
        R.retention_parallel_fwd(q, k, v, gm, out=outs[i % 2])

    def chk(i):
        q, k, v, _, _ = data[i % 2]
        R.retention_chunkwise_fwd(q, k, v, gm, 64, out=outs[i % 2])

    tp, _ = time_steps(par, steps, warmup, torch)
    tc, _ = time_steps(chk, steps, warmup, torch)
    nb = alg_bytes(B, H, N, dk, dv)
    return {"workload": "parallel form", "B": B, "H": H, "N": N, "dk": dk, "dv": dv,
            "us_per_step": tp / steps * 1e6, "tokens_per_s": B * N / (tp / steps),
            "alg_GBps": nb / (tp / steps) / 1e9, "chunkwise_c64_us": tc / steps * 1e6}


def run_msr_workload(torch, R, B, N, D, H, dk, dv, steps, warmup, seed):
    """Gated retention layer (projections, rotation, decays, retention, norm and gate,
    output projection) on bf16 activations and random weights."""
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    x = torch.randn(B, N, D, device="cuda", generator=g).to(torch.bfloat16)
    s = D ** -0.5
    shapes = ((H * dk, D), (H * dk, D), (H * dv, D), (H * dv, D), (H, D), (D, H * dv))
    w = [(torch.randn(*sh, device="cuda", generator=g) * s).to(torch.bfloat16) for sh in shapes]
    ws = torch.empty(R.msr_workspace_bytes(B, N, D, H, dk, dv, 64), dtype=torch.uint8, device="cuda")
    y = torch.empty(B, N, D, dtype=torch.bfloat16, device="cuda")

    def step(i):
        R.gated_msr_fwd(x, *w, H, dk, dv, chunk=64, out=y, workspace=ws)

    t, _ = time_steps(step, steps, warmup, torch)
    per = t / steps
    fl = 2 * B * N * D * (2 * H * dk + 2 * H * dv + H) + 2 * B * N * H * dv * D
    return {"workload": "gated retention layer", "B": B, "N": N, "D": D, "H": H, "dk": dk, "dv": dv, "chunk": 64,
            "us_per_step": per * 1e6, "tokens_per_s": B * N / per, "projection_TFLOPs": fl / per / 1e12}


def run_decode(torch, R, steps_per_call=1024, warm_calls=1, seed=4, gated=False):
    """Recurrent decode: batch 128, H=32, d=128; S0 ~ N(0, 0.1^2) fp32; fresh bf16
    q,k,v per step (pre-generated on the GPU); gamma_h = 1 - 2^(-5 - 7h/31), or (gated) a
    fresh g = logsigmoid(x)/16 [B,H] fp32 per step."""
    B, H, d = 128, 32, 128
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    S = torch.randn(B, H, d, d, device="cuda", generator=g) * 0.1
    s = 1.0 / math.sqrt(d)
    q = (torch.randn(steps_per_call, B, H, d, device="cuda", generator=g) * s).to(torch.bfloat16)
    k = (torch.randn(steps_per_call, B, H, d, device="cuda", generator=g) * s).to(torch.bfloat16)
    v = (torch.randn(steps_per_call, B, H, d, device="cuda", generator=g) * s).to(torch.bfloat16)
    gm = torch.tensor([1.0 - 2.0 ** (-5.0 - h * 7.0 / 31.0) for h in range(H)], device="cuda")
    gs = (torch.nn.functional.logsigmoid(torch.randn(steps_per_call, B, H, device="cuda", generator=g)) / 16
          if gated else None)
    o = torch.empty(B, H, d, device="cuda", dtype=torch.bfloat16)

    def step(i):
        j = i % steps_per_call
        if gated:
            R.gated_retention_decode_step(q[j], k[j], v[j], gs[j], S, out=o)
        else:
            R.retention_decode_step(q[j], k[j], v[j], gm, S, out=o)

    t, _ = time_steps(step, steps_per_call, warm_calls * 16, torch)
    per = t / steps_per_call
    nb = B * H * (2 * d * d * 4 + 4 * d * 2 + (4 if gated else 0))
    # the same 1024 steps again, each bracketed by its own events
    dist = stats(per_call_times(step, steps_per_call, torch))
    return {"workload": "gated_decode_bf16" if gated else "decode_bf16", "batch": B, "H": H, "dk": d, "dv": d,
            "steps": steps_per_call,
            "us_per_step": per * 1e6, "tokens_per_s": B / per,
            "hbm_GBps": nb / per / 1e9, "hbm_frac": nb / per / 1e9 / HBM_PEAK_GBS, "per_step": dist}


def cpu_baseline(max_seconds=15.0):
    """fp64 oracle (recurrent form) on the headline workload's first T tokens of every
    (b,h), T chosen so the run takes about `max_seconds`."""
    import numpy as np
    from oracle import retention_recurrent
    from retnet_retention_fwd_amd import inputs as I
    w = I.WORKLOADS["train_bf16"]
    rng = np.random.default_rng(w.seed)
    probe_T = 32
    shp = (w.B, w.H)

    def mk(T):
        s = 1.0 / math.sqrt(w.dk)
        q = rng.standard_normal(shp + (T, w.dk)) * s
        k = rng.standard_normal(shp + (T, w.dk)) * s
        v = rng.standard_normal(shp + (T, w.dv)) * s
        return q, k, v

    gm = I.gammas("train_bf16", w.H).astype(np.float64)
    t0 = os.times()
    w0 = time.perf_counter()
    retention_recurrent(*mk(probe_T), gm)
    probe = time.perf_counter() - w0
    T = int(max(probe_T, min(w.N, probe_T * max_seconds / max(probe, 1e-6))))
    t1 = os.times()
    w1 = time.perf_counter()
    retention_recurrent(*mk(T), gm)
    wall = time.perf_counter() - w1
    t2 = os.times()
    cpu = (t2.user - t1.user) + (t2.system - t1.system)
    threads = max(1, int(round(cpu / max(wall, 1e-9))))
    del t0
    try:
        affinity = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        affinity = os.cpu_count()
    try:   # numpy's BLAS pool (the recurrence's elementwise loop does not use it)
        from threadpoolctl import threadpool_info
        blas = ",".join(f"{p.get('internal_api')}:{p.get('num_threads')}" for p in threadpool_info()
                        if p.get("user_api") == "blas") or "none"
    except Exception:   # threadpoolctl missing or unable to inspect: report unknown
        blas = "unknown"
    return {"value": w.B * T / wall, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"train_bf16 workload, all {w.B}x{w.H} (b,h), first {T} of {w.N} tokens, "
                      f"fp64 numpy recurrence; {wall:.1f} s wall, {cpu:.1f} s CPU; "
                      f"host has {os.cpu_count()} logical CPUs, {affinity} in this process's affinity; "
                      f"BLAS threads {blas}"}


def counter_summary():
    """The committed rocprofv3 counter summary of the headline kernel, or None if it was
    taken on another version of the kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    return t if t.get("kernel_sha256_16") == kernel_hash() else None


def traffic_per_launch():
    """HBM bytes per launch from the committed counter summary, or None if stale."""
    t = counter_summary()
    return None if t is None else t.get("hbm_bytes_per_launch")


SECONDARY_NAMES = ("decode_bf16", "gated_decode_bf16", "long_bf16_C512", "long_bf16_C256", "long_bf16_C128", "gated_bf16",
                   "train_bf16_backward", "gated_bf16_backward", "parallel_bf16_N256", "parallel_bf16_N512",
                   "msr_layer_bf16")


def secondary_line(torch, R, name):
    h = [1.0 - 2.0 ** (-5.0 - i) for i in range(8)]
    g3 = [1.0 - 2.0 ** (-5.0 - i * 7.0 / 15.0) for i in range(16)]
    if name == "decode_bf16":
        return run_decode(torch, R)
    if name == "gated_decode_bf16":
        return run_decode(torch, R, seed=11, gated=True)
    if name.startswith("long_bf16_C"):
        return run_chunk_workload(torch, R, "long_bf16", 1, 16, 16384, 128, 128, int(name[11:]), g3, False, 50, 5,
                                  seed=3, kernel_times=True)
    if name == "gated_bf16":
        return run_chunk_workload(torch, R, "gated_bf16", 2, 16, 8192, 128, 128, 64, None, True, 50, 5, seed=5,
                                  kernel_times=True)
    if name == "train_bf16_backward":
        return run_bwd_workload(torch, R, "train_bf16", 4, 8, 2048, 256, 512, 64, h, False, 20, 3, seed=6)
    if name == "gated_bf16_backward":
        return run_bwd_workload(torch, R, "gated_bf16", 2, 16, 8192, 128, 128, 64, None, True, 20, 3, seed=7)
    if name == "parallel_bf16_N256":
        return run_parallel_workload(torch, R, 2, 16, 256, 128, 128, 50, 5, seed=8)
    if name == "parallel_bf16_N512":
        return run_parallel_workload(torch, R, 16, 8, 512, 128, 128, 50, 5, seed=9)
    if name == "msr_layer_bf16":
        return run_msr_workload(torch, R, 4, 2048, 1024, 8, 128, 128, 30, 5, seed=10)
    raise ValueError(name)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-secondary", action="store_true", help="skip decode/long/gated lines")
    ap.add_argument("--calib-copy", action="store_true",
                    help="run only a plain 1 GiB device copy (counter calibration for rocprofv3)")
    ap.add_argument("--calib-mfma", action="store_true",
                    help="run only the achievable-peak references (matrix-core loop, device copy)")
    ap.add_argument("--only", choices=SECONDARY_NAMES,
                    help="run only this secondary line and print it (for profiling one workload)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the operator runs on a single MI355X and there is no "
              "multi-GPU path (--gpus must be 1).", file=sys.stderr)
        sys.exit(2)

    import torch
    import retnet_retention_fwd_amd as R
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    R.lib()   # fail loudly if the HIP library is missing

    if args.calib_copy:
        n = 1 << 28   # 1 GiB of fp32
        a = torch.ones(n, device="cuda")
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"calib_copy_bytes": n * 4}))
        return

    if args.calib_mfma:
        print(json.dumps({"achievable": achievable(torch, R)}))
        return

    if args.only:
        print(json.dumps({args.only: secondary_line(torch, R, args.only)}))
        return

    h = [1.0 - 2.0 ** (-5.0 - i) for i in range(8)]
    head = run_chunk_workload(torch, R, "train_bf16", 4, 8, 2048, 256, 512, 64, h, False,
                              args.steps, args.warmup, seed=2, kernel_times=True, dist_calls=max(100, args.steps))

    secondary = {}
    if not args.no_secondary:
        for name in SECONDARY_NAMES:
            secondary[name] = secondary_line(torch, R, name)

    main_us = head["kernels"]["chunk_main"]["avg_us"]
    nb = alg_bytes(4, 8, 2048, 256, 512)
    fl = alg_flops(4, 8, 2048, 256, 512, 64)
    achieved = nb / (main_us * 1e-6) / 1e9
    cs = counter_summary()
    roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic_per_launch(),
            "kernel": HEADLINE_KERNEL,
            "alg_bytes_per_launch": nb, "avg_launch_us": main_us,
            "mfma_tflops": round(fl / (main_us * 1e-6) / 1e12, 1),
            "mfma_frac": round(fl / (main_us * 1e-6) / 1e12 / BF16_PEAK_TFLOPS, 4),
            # matrix-core busy cycles / (GPU busy cycles x SIMDs), from the committed
            # rocprofv3 counters of this kernel source (null once the kernel changed)
            "mfma_busy_counter": None if cs is None else cs.get("mfma_busy_frac"),
            "step_kernels": head["kernels"]}

    line = {
        "metric": METRIC,
        "value": round(head["tokens_per_s"], 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head["us_per_step"] / 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded normal inputs at the workload's shapes, resident in HBM)",
        "config": {"workload": "train_bf16 chunkwise retention forward", "B": 4, "H": 8, "N": 2048,
                   "dk": 256, "dv": 512, "chunk": 64, "global_batch": 4, "seq_len": 2048,
                   "parallelism": "single GPU"},
        "roofline": roof,
        "timing": {"protocol": "value and ms_per_step: HIP events around the timed steps back to back, after "
                               f"{SETTLE_S} s of untimed steps and the warmup steps; per_call: events around each "
                               "of the calls, unflushed and with a 1 GiB write before each",
                   "per_call": head["per_call"]},
    }
    line["achievable"] = achievable(torch, R)
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline()
    if secondary:
        line["secondary"] = {k: {kk: (round(vv, 4) if isinstance(vv, float) else vv) for kk, vv in v.items()}
                             for k, v in secondary.items()}
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
