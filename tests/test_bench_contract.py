"""Host-side checks of bench.py's contract (no GPU: nothing here launches a kernel)."""
import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "single" in r.stderr and "--gpus must be 1" in r.stderr
    assert r.stdout == ""


def brute_force_flops(N, C, dk, dv):
    """Multiply-adds (2 flops each) of the chunkwise form of one head, counted term by term:
    causal scores and score-times-value products inside each chunk, the cross-chunk query
    term and the state update of every token."""
    fl = 0
    for c0 in range(0, N, C):
        L = min(C, N - c0)
        for j in range(L):
            for l in range(j + 1):
                fl += 2 * dk + 2 * dv          # q_j . k_l and p_jl v_l
            fl += 2 * dk * dv                  # q_j S
            fl += 2 * dk * dv                  # k_j^T v_j into S
    return fl


def test_flop_and_byte_counts():
    # whole chunks: the per-token closed form equals the term-by-term count
    for N, C, dk, dv in [(8, 4, 2, 3), (16, 16, 5, 1), (12, 1, 3, 3)]:
        assert bench.alg_flops(1, 1, N, dk, dv, C) == brute_force_flops(N, C, dk, dv)
    assert bench.alg_flops(2, 3, 8, 2, 3, 4) == 6 * brute_force_flops(8, 4, 2, 3)
    # the train workload: Q, K, V read and O written once, bf16
    assert bench.alg_bytes(4, 8, 2048, 256, 512) == 4 * 8 * 2048 * (256 + 256 + 512 + 512) * 2 == 201326592
    assert bench.alg_bytes(1, 1, 10, 4, 4, gated=True) == 10 * (16 * 2 + 4)


def test_traffic_figure_follows_the_kernel_source(monkeypatch):
    with open(bench.TRAFFIC_FILE) as f:
        t = json.load(f)
    monkeypatch.setattr(bench, "kernel_hash", lambda: t["kernel_sha256_16"])
    assert bench.traffic_per_launch() == t["hbm_bytes_per_launch"]
    monkeypatch.setattr(bench, "kernel_hash", lambda: "0" * 16)
    assert bench.traffic_per_launch() is None
    # the stored figure is the scaled sum of the two counters
    cal = t["copy_calibration"]
    expect = (t["fetch_kib_per_dispatch"] * cal["fetch_scale"] + t["write_kib_per_dispatch"] * cal["write_scale"]) * 1024
    assert abs(t["hbm_bytes_per_launch"] - expect) <= 1e-3 * expect
