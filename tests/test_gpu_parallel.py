"""GPU parity of the parallel-form entry points (through the C ABI) against the fp64
oracle's parallel form, which the oracle tests pin to the recurrence.

Tolerance (max|err| / max|ref| over the output): 1e-4 for fp32 inputs, 1e-2 for bf16.
Inputs: retnet_retention_fwd_amd.inputs.random_case (Q, K, V ~ N(0,1)/sqrt(dk); gamma
~ U(0.8, 1) per head, or g = logsigmoid(x)/16 per token).
"""
import numpy as np
import pytest

import oracle as O
from retnet_retention_fwd_amd import inputs as I

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 1e-2}


def R():
    import retnet_retention_fwd_amd as R_
    return R_


def rel(gpu, ref):
    g = gpu.detach().float().cpu().double().numpy()
    assert np.all(np.isfinite(g)), "non-finite GPU output"
    return float(np.max(np.abs(g - ref)) / max(np.max(np.abs(ref)), 1e-30))


def run(x, gated):
    d = lambda t: t[0].cuda()  # noqa: E731
    if gated:
        o = R().gated_retention_parallel_fwd(d(x["q"]), d(x["k"]), d(x["v"]), d(x["g"]))
    else:
        o = R().retention_parallel_fwd(d(x["q"]), d(x["k"]), d(x["v"]), d(x["gamma"]))
    torch.cuda.synchronize()
    return o


def ref(x, gated):
    if gated:
        return O.gated_retention_parallel(x["q"][1], x["k"][1], x["v"][1], x["g"][1])[0]
    return O.retention_parallel(x["q"][1], x["k"][1], x["v"][1], x["gamma"][1])[0]


CASES = [
    # (B, H, N, dk, dv, dtype, gated): several query blocks, ragged tails, every tile shape
    (2, 3, 200, 64, 64, "bf16", False),
    (1, 2, 333, 128, 128, "bf16", False),
    (1, 2, 130, 256, 512, "bf16", False),
    (2, 2, 64, 64, 128, "bf16", False),
    (1, 1, 1, 128, 64, "bf16", False),          # one token
    (2, 2, 300, 128, 128, "bf16", True),
    (1, 2, 512, 64, 192, "bf16", True),         # the longest gated sequence on the matrix cores
    (1, 2, 77, 256, 256, "bf16", True),
    (1, 2, 700, 128, 128, "bf16", True),        # longer gated: generic kernel
    (1, 1, 1500, 64, 64, "bf16", False),        # per head: any length on the matrix cores
    (1, 1, 130, 128, 1024, "bf16", False),      # the widest d_v
    (1, 2, 70, 32, 48, "f32", False),           # fp32: generic kernel
    (1, 2, 70, 32, 48, "f32", True),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "x".join(map(str, c)))
def test_parallel_matches_oracle(case):
    B, H, N, dk, dv, dt, gated = case
    print(f"\n[case] parallel {case}", flush=True)
    x = I.random_case(sum(case[:5]), B, H, N, dk, dv, dtype=dt, gated=gated)
    assert rel(run(x, gated), ref(x, gated)) <= TOL[dt]


def test_parallel_equals_chunkwise_without_state():
    """The two GPU forms compute the same function: the parallel form against the
    chunkwise one on the same inputs (bf16, ragged)."""
    print("\n[case] parallel vs chunkwise", flush=True)
    x = I.random_case(9, 2, 4, 450, 128, 128, dtype="bf16")
    d = lambda t: t[0].cuda()  # noqa: E731
    a = R().retention_parallel_fwd(d(x["q"]), d(x["k"]), d(x["v"]), d(x["gamma"]))
    b = R().retention_chunkwise_fwd(d(x["q"]), d(x["k"]), d(x["v"]), d(x["gamma"]), 64)
    torch.cuda.synchronize()
    r = ref(x, False)
    assert rel(a, r) <= TOL["bf16"] and rel(b, r) <= TOL["bf16"]
    assert rel(a, b.float().cpu().double().numpy()) <= TOL["bf16"]


def test_parallel_short_workload_sampled_heads():
    """The short-sequence workload the benchmark times (B=16 H=8 N=512 dk=dv=128), with
    the oracle on two sampled heads."""
    print("\n[case] parallel short workload", flush=True)
    B, H, N, dk, dv = 16, 8, 512, 128, 128
    x = I.random_case(11, B, H, N, dk, dv, dtype="bf16")
    o = run(x, False)
    for b, h in ((0, 0), (15, 7)):
        q, k, v = (x[n][1][b:b + 1, h:h + 1] for n in ("q", "k", "v"))
        r = O.retention_parallel(q, k, v, x["gamma"][1][h:h + 1])[0]
        assert rel(o[b:b + 1, h:h + 1], r) <= TOL["bf16"], (b, h)
