"""GPU parity: the HIP library (through its C ABI) against the fp64 oracle.

Tolerance (max|err| / max|ref| over the compared tensor): 1e-4 for fp32 inputs, 1e-2 for
bf16 inputs.  Inputs are seeded and synthetic (retnet_retention_fwd_amd.inputs); the
oracle reads the very values uploaded to the GPU, promoted to fp64.
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
    g = gpu.detach().float().cpu().double().numpy() if hasattr(gpu, "detach") else np.asarray(gpu)
    ref = np.asarray(ref, dtype=np.float64)
    assert np.all(np.isfinite(g)), "non-finite GPU output"
    return float(np.max(np.abs(g - ref)) / max(np.max(np.abs(ref)), 1e-30))


def dev(x):
    return x[0].cuda()


def say(msg):
    print(f"\n[case] {msg}", flush=True)


def run_chunk(x, chunk, gated, state_in=False, return_state=True):
    args = [dev(x["q"]), dev(x["k"]), dev(x["v"]), dev(x["g"] if gated else x["gamma"]), chunk]
    si = dev(x["state_in"]) if state_in else None
    fn = R().gated_retention_chunkwise_fwd if gated else R().retention_chunkwise_fwd
    out = fn(*args, state_in=si, return_state=return_state)
    torch.cuda.synchronize()
    return out


def oracle_chunk(x, gated, state_in=False, heads=None):
    q, k, v = x["q"][1], x["k"][1], x["v"][1]
    d = x["g"][1] if gated else x["gamma"][1]
    si = x["state_in"][1] if state_in else None
    if heads is not None:
        b, h = heads
        q, k, v = q[b][:, h], k[b][:, h], v[b][:, h]
        si = None if si is None else si[b][:, h]
        d = d[b][:, h] if gated else d[h]
    if gated:
        return O.gated_retention_recurrent(q, k, v, d, si)
    return O.retention_recurrent(q, k, v, d, si)


def test_native_library_is_loaded():
    L = R().lib()
    assert L.retention_abi_version() == 1
    assert L._name.endswith("libretention_fwd.so")


# ------------------------------------------------------------------ tiny fp32 workload
def test_tiny_f32_workload():
    w = I.WORKLOADS["tiny_f32"]
    say(f"{w}")
    x = I.make_chunkwise(w)
    o, S = run_chunk(x, w.chunk, gated=False)
    ro, rS = oracle_chunk(x, gated=False)
    assert rel(o, ro) <= TOL["f32"]
    assert rel(S, rS) <= TOL["f32"]


# ------------------------------------------------------------------ small shapes, both paths
SMALL = [
    # (B, H, N, dk, dv, chunk, dtype, gated, state_in)
    (1, 2, 64, 16, 16, 16, "f32", False, False),
    (2, 3, 77, 24, 40, 16, "f32", False, True),
    (1, 2, 130, 64, 64, 7, "f32", True, True),
    (1, 1, 300, 128, 96, 100, "f32", False, True),
    (1, 2, 200, 48, 40, 33, "bf16", False, True),        # bf16 on the generic kernel
    (1, 2, 190, 32, 64, 64, "bf16", True, False),        # dk 32: generic kernel
    (1, 2, 64, 64, 64, 64, "bf16", False, False),        # matrix-core path from here on
    (2, 2, 300, 64, 128, 64, "bf16", False, True),
    (1, 3, 257, 128, 128, 128, "bf16", False, True),
    (1, 2, 600, 128, 128, 256, "bf16", True, True),
    (1, 2, 1100, 128, 64, 512, "bf16", False, True),
    (1, 2, 1100, 128, 128, 512, "bf16", True, False),
    (2, 1, 333, 256, 128, 64, "bf16", False, True),
    (1, 2, 200, 256, 192, 128, "bf16", True, True),
    (1, 1, 129, 64, 64, 100, "bf16", False, True),       # chunk not a multiple of 64
    (1, 1, 90, 128, 128, 37, "bf16", True, True),
    (1, 2, 1, 128, 128, 64, "bf16", False, True),        # N = 1
    (1, 2, 40, 128, 128, 512, "bf16", False, True),      # chunk > N
    (1, 2, 250, 256, 256, 48, "bf16", False, True),      # dk 256, 128-column tiles, short chunk
    (1, 2, 150, 256, 64, 64, "bf16", True, True),        # dk 256 gated, one block per chunk
    (1, 1, 170, 64, 192, 40, "bf16", False, False),
    (1, 1, 200, 128, 1024, 64, "bf16", False, True),     # the widest d_v: eight column tiles
    (1, 1, 150, 64, 1024, 64, "bf16", True, False),
    (1, 1, 130, 256, 1024, 64, "bf16", False, True),     # the largest state, 256 x 1024
    # two segments where the second walks the first state-only (prefix split)
    (1, 16, 600, 128, 1024, 64, "bf16", False, True),
    (2, 8, 450, 128, 1024, 64, "bf16", True, True),
    (1, 32, 300, 256, 512, 64, "bf16", False, True),     # ragged last chunk
    # per head, the state-only prefix runs over three stages; prefixes of 2 to 5 chunks
    # enter it at each of them (d_k 256 and 128), and short sequences of one chunk, a
    # one-token last chunk, 384 columns and a grid that is not a multiple of 8
    (1, 32, 256, 256, 512, 64, "bf16", False, True),
    (1, 32, 320, 256, 512, 64, "bf16", False, False),
    (1, 16, 384, 128, 1024, 64, "bf16", False, True),
    (1, 32, 448, 256, 512, 64, "bf16", False, True),
    (1, 16, 256, 128, 1024, 64, "bf16", False, False),
    (1, 32, 64, 256, 512, 64, "bf16", False, True),
    (1, 32, 65, 256, 512, 64, "bf16", False, True),
    (2, 22, 150, 256, 384, 64, "bf16", False, True),
    (1, 43, 100, 256, 384, 64, "bf16", False, False),
    # chunks of 128/256/512 with d_k = 128 (query-row parallel main pass): two column
    # tiles, ragged last chunks (one that ends inside the second pass of a 512-token
    # chunk, one of 8 tokens), several segments, and a chunk of one block
    (1, 2, 700, 128, 256, 256, "bf16", False, True),
    (2, 2, 1600, 128, 128, 512, "bf16", False, False),
    (1, 1, 777, 128, 128, 512, "bf16", False, True),
    (1, 2, 520, 128, 128, 256, "bf16", False, True),
    (1, 4, 2700, 128, 128, 128, "bf16", False, True),
    (1, 2, 5000, 128, 128, 512, "bf16", False, True),
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: "B{}H{}N{}dk{}dv{}C{}{}{}{}".format(*c[:7], "g" if c[7] else "", "s" if c[8] else ""))
def test_small_shapes(case):
    B, H, N, dk, dv, C, dt, gated, si = case
    say(case)
    x = I.random_case(sum(case[:6]), B, H, N, dk, dv, dtype=dt, gated=gated, state_in=si)
    o, S = run_chunk(x, C, gated, state_in=si)
    ro, rS = oracle_chunk(x, gated, state_in=si)
    assert rel(o, ro) <= TOL[dt]
    assert rel(S, rS) <= TOL[dt]


@pytest.mark.parametrize("gated", [False, True])
def test_segmented_sequence(gated):
    """Few (b,h) and a long sequence: the matrix-core path splits the sequence into
    segments (state pre-pass + scan); results must not depend on it."""
    B, H, N, dk, dv, C = 1, 2, 4000, 128, 128, 64
    say(("segmented", gated))
    assert R().workspace_bytes(B, H, N, dk, dv, C, 1, gated) > 0
    x = I.random_case(42, B, H, N, dk, dv, dtype="bf16", gated=gated, state_in=True)
    o, S = run_chunk(x, C, gated, state_in=True)
    ro, rS = oracle_chunk(x, gated, state_in=True)
    assert rel(o, ro) <= TOL["bf16"]
    assert rel(S, rS) <= TOL["bf16"]


STRONG = [
    # (B, H, N, dk, dv, chunk, gated): decays strong enough that the kernels' state
    # scale is reset often and many decay factors underflow to zero
    (1, 2, 300, 256, 256, 64, False),
    (1, 2, 300, 256, 128, 64, True),
    (1, 2, 300, 128, 128, 128, True),
    (1, 2, 200, 64, 64, 40, True),
    (1, 2, 260, 128, 64, 64, False),
    (1, 2, 1300, 128, 128, 512, False),
    (1, 2, 700, 128, 128, 128, False),
]


@pytest.mark.parametrize("case", STRONG, ids=lambda c: "B{}H{}N{}dk{}dv{}C{}{}".format(*c[:6], "g" if c[6] else ""))
def test_strong_decay(case):
    B, H, N, dk, dv, C, gated = case
    say(("strong", case))
    x = I.random_case(sum(case[:6]) + 7, B, H, N, dk, dv, dtype="bf16", gated=gated, state_in=True,
                      gamma_lo=0.05)
    if gated:
        rng = np.random.default_rng(N + dk)
        x["g"] = I.to_dtype(I.logsigmoid(rng.standard_normal((B, H, N)) * 4.0), "f32")
    o, S = run_chunk(x, C, gated, state_in=True)
    ro, rS = oracle_chunk(x, gated, state_in=True)
    assert rel(o, ro) <= TOL["bf16"]
    assert rel(S, rS) <= TOL["bf16"]


@pytest.mark.parametrize("case", [(1, 2, 200, 256, 256, 64), (1, 2, 200, 128, 128, 100), (1, 2, 130, 64, 64, 64),
                                  (1, 2, 150, 128, 64, 40), (1, 2, 600, 128, 128, 256), (1, 2, 1100, 128, 128, 512)],
                         ids=lambda c: "N{}dk{}dv{}C{}".format(*c[2:]))
def test_tiny_gamma(case):
    """Per-head decays far below the usual range: the decay factors the kernels split
    into per-lane and per-tile parts must not overflow."""
    B, H, N, dk, dv, C = case
    say(("tiny gamma", case))
    x = I.random_case(N + dk + dv, B, H, N, dk, dv, dtype="bf16", state_in=True)
    x["gamma"] = I.to_dtype(np.array([0.001, 0.04]), "f32")
    o, S = run_chunk(x, C, False, state_in=True)
    ro, rS = oracle_chunk(x, False, state_in=True)
    assert rel(o, ro) <= TOL["bf16"]
    assert rel(S, rS) <= TOL["bf16"]


def test_kernel_timing_records_every_launch():
    """The library's event timing sees each launch of a split-sequence call once."""
    say("kernel timing")
    x = I.random_case(77, 1, 2, 4000, 128, 128, dtype="bf16")
    R().profile_enable(True)
    try:
        o, _ = run_chunk(x, 64, False)
        p = R().profile_read()
    finally:
        R().profile_enable(False)
    assert p["dropped"] == 0
    for kind in ("chunk_main", "chunk_prepass", "chunk_scan"):
        assert p[kind]["launches"] == 1, (kind, p)
        assert p[kind]["ms"] > 0.0
    assert p["decode"]["launches"] == 0
    ro, _ = oracle_chunk(x, False)
    assert rel(o, ro) <= TOL["bf16"]


# ------------------------------------------------------------------ edge cases
def test_empty_sequence_passes_state_through():
    say("N=0")
    q = torch.zeros(1, 2, 0, 64, dtype=torch.bfloat16, device="cuda")
    v = torch.zeros(1, 2, 0, 64, dtype=torch.bfloat16, device="cuda")
    gm = torch.tensor([0.5, 0.9], device="cuda")
    si = torch.randn(1, 2, 64, 64, device="cuda")
    o, S = R().retention_chunkwise_fwd(q, q, v, gm, 64, state_in=si, return_state=True)
    torch.cuda.synchronize()
    assert o.shape == (1, 2, 0, 64)
    assert torch.equal(S, si)
    o, S = R().retention_chunkwise_fwd(q, q, v, gm, 64, return_state=True)
    torch.cuda.synchronize()
    assert torch.count_nonzero(S) == 0


def test_gamma_one_is_linear_attention():
    """gamma = 1: causal linear attention; on all-ones inputs o_n = dk (n+1)."""
    say("gamma=1")
    B, H, N, d = 1, 1, 200, 64
    one = torch.ones(B, H, N, d, dtype=torch.float32, device="cuda")
    o = R().retention_chunkwise_fwd(one, one, one, torch.ones(1, device="cuda"), 64)
    torch.cuda.synchronize()
    exp = d * (torch.arange(N, device="cuda", dtype=torch.float64) + 1)
    assert torch.allclose(o[0, 0, :, 0].double(), exp, rtol=1e-5)


@pytest.mark.parametrize("N,C", [(200, 64), (4000, 64), (1100, 512)])
def test_gamma_one_bf16_matrix_cores(N, C):
    """gamma = 1 on the bf16 matrix-core path (the tutorial's quiz: retention with no
    decay is causal linear attention).  All-ones inputs give o_n = dk (n+1) and
    S_N = N in every entry; random inputs match the oracle.  N = 4000 with two heads
    splits the sequence into segments."""
    say(("gamma=1 bf16", N, C))
    B, H, d = 1, 2, 128
    gm = torch.ones(H, device="cuda")
    one = torch.ones(B, H, N, d, dtype=torch.bfloat16, device="cuda")
    o, S = R().retention_chunkwise_fwd(one, one, one, gm, C, return_state=True)
    torch.cuda.synchronize()
    exp = d * (np.arange(N, dtype=np.float64) + 1)
    assert rel(o[0, :, :, :], np.broadcast_to(exp[None, :, None], (H, N, d))) <= TOL["bf16"]
    assert torch.all(S == float(N))
    x = I.random_case(N + C, B, H, N, d, d, dtype="bf16", state_in=True)
    x["gamma"] = I.to_dtype(np.ones(H), "f32")
    o, S = run_chunk(x, C, False, state_in=True)
    ro, rS = oracle_chunk(x, False, state_in=True)
    assert rel(o, ro) <= TOL["bf16"]
    assert rel(S, rS) <= TOL["bf16"]


@pytest.mark.parametrize("dk,dv,N", [(128, 128, 1500), (256, 128, 700), (64, 64, 300)])
def test_gated_constant_g_matches_per_head(dk, dv, N):
    """A gated call whose log-decays are constant per head, g = log(gamma_h), is the
    per-head form with that gamma (the pwwt.cn guide's gated decay reduces to RetNet's
    fixed per-head decay).  Both kernels are checked against the oracle and against each
    other; gamma = 1 (g = 0) is one of the heads."""
    say(("constant g", dk, dv, N))
    B, H, C = 1, 4, 64
    x = I.random_case(dk + N, B, H, N, dk, dv, dtype="bf16", state_in=True)
    lg = np.log(np.array([0.9, 0.97, 0.999, 1.0]))
    g = I.to_dtype(np.broadcast_to(lg[None, :, None], (B, H, N)).copy(), "f32")
    # the per-head decay is exp of the very fp32 log-decay the gated call takes
    x["gamma"] = I.to_dtype(np.exp(g[1][0, :, 0]), "f32")
    og, Sg = run_chunk(dict(x, g=g), C, True, state_in=True)
    op, Sp = run_chunk(x, C, False, state_in=True)
    rog, rSg = oracle_chunk(dict(x, g=g), True, state_in=True)
    rop, rSp = oracle_chunk(x, False, state_in=True)
    assert rel(og, rog) <= TOL["bf16"] and rel(Sg, rSg) <= TOL["bf16"]
    assert rel(op, rop) <= TOL["bf16"] and rel(Sp, rSp) <= TOL["bf16"]
    assert rel(og, op.float().cpu().double().numpy()) <= TOL["bf16"]
    # the oracle's two forms differ only through the fp32 rounding of gamma = exp(g)
    # (about 1e-7 relative per step, compounded over N steps)
    assert float(np.max(np.abs(rog - rop))) <= 1e-3 * float(np.max(np.abs(rop)))


def test_closed_form_all_ones_bf16():
    """All-ones inputs: o_n = dk (1 - gamma^(n+1)) / (1 - gamma) (geometric series)."""
    say("all-ones closed form bf16")
    B, H, N, d = 1, 2, 700, 128
    one = torch.ones(B, H, N, d, dtype=torch.bfloat16, device="cuda")
    gm = torch.tensor([0.9, 0.99], device="cuda")
    for C in (64, 256, 512):
        o, S = R().retention_chunkwise_fwd(one, one, one, gm, C, return_state=True)
        torch.cuda.synchronize()
        n = np.arange(N)
        g = np.array([0.9, 0.99], dtype=np.float32).astype(np.float64)
        exp = d * (1 - g[:, None] ** (n[None] + 1)) / (1 - g[:, None])
        assert rel(o[0, :, :, 0], exp) <= 1e-2
        expS = (1 - g ** N) / (1 - g)
        assert rel(S[0, :, 0, 0], expS) <= 1e-2


def test_split_resume_and_decode_handoff():
    """chunkwise(N1) -> state_out -> chunkwise(N2, state_in) -> decode steps equals the
    recurrence over the whole sequence (the prefill state seeds the next call)."""
    say("split/resume + decode handoff")
    B, H, N1, N2, M, d = 2, 2, 320, 200, 16, 128
    x = I.random_case(7, B, H, N1 + N2 + M, d, d, dtype="bf16", state_in=False)
    q, k, v = (x[n][0].cuda() for n in ("q", "k", "v"))
    gm = x["gamma"][0].cuda()
    o1, S1 = R().retention_chunkwise_fwd(q[:, :, :N1].contiguous(), k[:, :, :N1].contiguous(),
                                         v[:, :, :N1].contiguous(), gm, 64, return_state=True)
    sl = slice(N1, N1 + N2)
    o2, S2 = R().retention_chunkwise_fwd(q[:, :, sl].contiguous(), k[:, :, sl].contiguous(),
                                         v[:, :, sl].contiguous(), gm, 128, state_in=S1, return_state=True)
    outs = []
    S = S2.clone()
    for t in range(N1 + N2, N1 + N2 + M):
        outs.append(R().retention_decode_step(q[:, :, t].contiguous(), k[:, :, t].contiguous(),
                                              v[:, :, t].contiguous(), gm, S))
    torch.cuda.synchronize()
    ro, rS = O.retention_recurrent(x["q"][1], x["k"][1], x["v"][1], x["gamma"][1])
    got = torch.cat([o1, o2, torch.stack(outs, dim=2)], dim=2)
    assert rel(got, ro) <= TOL["bf16"]
    assert rel(S, rS) <= TOL["bf16"]


def test_in_place_state():
    """state_out may be the same buffer as state_in."""
    say("in-place state")
    x = I.random_case(9, 1, 2, 150, 128, 128, dtype="bf16", state_in=True)
    S = dev(x["state_in"]).clone()
    o = R().retention_chunkwise_fwd(dev(x["q"]), dev(x["k"]), dev(x["v"]), dev(x["gamma"]), 64,
                                    state_in=S, state_out=S)
    torch.cuda.synchronize()
    ro, rS = oracle_chunk(x, False, state_in=True)
    assert rel(o[0], ro) <= TOL["bf16"] and rel(S, rS) <= TOL["bf16"]


def test_chunk_size_changes_rounding_only():
    say("chunk invariance")
    x = I.random_case(10, 1, 4, 1024, 128, 128, dtype="bf16")
    outs = [run_chunk(x, C, False)[0].float() for C in (64, 128, 256, 512)]
    for o in outs[1:]:
        assert rel(o, outs[0].cpu().double().numpy()) <= 1e-2


def test_deterministic_and_no_out_of_bounds_writes():
    """Two runs are bitwise identical; guard bands around o and state_out stay intact."""
    say("determinism + guard bands")
    B, H, N, dk, dv = 1, 2, 1000, 128, 128
    x = I.random_case(11, B, H, N, dk, dv, dtype="bf16", state_in=True)
    pad = 4096
    res = []
    for _ in range(2):
        obuf = torch.full((pad + B * H * N * dv + pad,), 7.0, dtype=torch.bfloat16, device="cuda")
        sbuf = torch.full((pad + B * H * dk * dv + pad,), 3.0, dtype=torch.float32, device="cuda")
        o = obuf[pad:pad + B * H * N * dv].view(B, H, N, dv)
        S = sbuf[pad:pad + B * H * dk * dv].view(B, H, dk, dv)
        R().retention_chunkwise_fwd(dev(x["q"]), dev(x["k"]), dev(x["v"]), dev(x["gamma"]), 256,
                                    state_in=dev(x["state_in"]), out=o, state_out=S)
        torch.cuda.synchronize()
        assert torch.all(obuf[:pad] == 7.0) and torch.all(obuf[-pad:] == 7.0)
        assert torch.all(sbuf[:pad] == 3.0) and torch.all(sbuf[-pad:] == 3.0)
        res.append((o.clone(), S.clone()))
    assert torch.equal(res[0][0], res[1][0]) and torch.equal(res[0][1], res[1][1])


# ------------------------------------------------------------------ decode
@pytest.mark.parametrize("dk,dv,dt,gated", [(128, 128, "bf16", False), (128, 128, "f32", False),
                                            (64, 64, "bf16", True), (96, 256, "bf16", False),
                                            (40, 24, "f32", True), (128, 128, "bf16", True)])
def test_decode_steps(dk, dv, dt, gated):
    say(("decode", dk, dv, dt, gated))
    B, H, steps = 3, 4, 40
    rng = np.random.default_rng(dk + dv)
    S0 = I.to_dtype(rng.standard_normal((B, H, dk, dv)) * 0.1, "f32")
    qs = I.to_dtype(rng.standard_normal((steps, B, H, dk)) / np.sqrt(dk), dt)
    ks = I.to_dtype(rng.standard_normal((steps, B, H, dk)) / np.sqrt(dk), dt)
    vs = I.to_dtype(rng.standard_normal((steps, B, H, dv)) / np.sqrt(dk), dt)
    if gated:
        dec = I.to_dtype(I.logsigmoid(rng.standard_normal((steps, B, H))) / 16, "f32")
    else:
        dec = I.to_dtype(rng.uniform(0.8, 1.0, size=H), "f32")
    S = S0[0].cuda().clone()
    Sref = S0[1]
    worst = 0.0
    for t in range(steps):
        d_t = dec[0][t].cuda().contiguous() if gated else dec[0].cuda()
        fn = R().gated_retention_decode_step if gated else R().retention_decode_step
        o = fn(qs[0][t].cuda(), ks[0][t].cuda(), vs[0][t].cuda(), d_t, S)
        f = O.gated_retention_decode_step if gated else O.retention_decode_step
        ro, Sref = f(qs[1][t], ks[1][t], vs[1][t], dec[1][t] if gated else dec[1], Sref)
        torch.cuda.synchronize()
        worst = max(worst, rel(o, ro))
    assert worst <= TOL[dt]
    assert rel(S, Sref) <= TOL[dt]


# ------------------------------------------------------------------ full-size workloads
@pytest.fixture(scope="module")
def train_case():
    w = I.WORKLOADS["train_bf16"]
    return w, I.make_chunkwise(w)


def oracle_pairs(x, pairs, gated=False):
    """The oracle on the listed (b,h) pairs only, run as one batch of len(pairs) heads."""
    bs, hs = [p[0] for p in pairs], [p[1] for p in pairs]
    q, k, v = (x[n][1][bs, hs][None] for n in ("q", "k", "v"))
    if gated:
        return O.gated_retention_recurrent(q, k, v, x["g"][1][bs, hs][None])
    return O.retention_recurrent(q, k, v, x["gamma"][1][hs])


def test_train_workload_full_size(train_case):
    """B=4 H=8 N=2048 dk=256 dv=512 C=64 on the GPU at full size; the oracle checks one
    (b,h) pair per head, (h mod 4, h), so every one of the eight decays is compared over
    the whole sequence."""
    w, x = train_case
    say(w)
    o, S = run_chunk(x, w.chunk, False)
    pairs = [(h % 4, h) for h in range(w.H)]
    ro, rS = oracle_pairs(x, pairs)
    for i, (b, h) in enumerate(pairs):
        assert rel(o[b, h], ro[0, i]) <= TOL["bf16"], (b, h)
        assert rel(S[b, h], rS[0, i]) <= TOL["bf16"], (b, h)


@pytest.fixture(scope="module")
def long_case():
    w = I.WORKLOADS["long_bf16"]
    x = I.make_chunkwise(w)
    heads = ([0], [0, 5, 10, 15])
    return w, x, heads, oracle_chunk(x, False, heads=heads)


@pytest.mark.parametrize("chunk", [128, 256, 512])
def test_long_workload_full_size(long_case, chunk):
    """B=1 H=16 N=16384 d=128 at each chunk size; the oracle checks heads 0,5,10,15."""
    w, x, heads, (ro, rS) = long_case
    say((w.name, chunk))
    o, S = run_chunk(x, chunk, False)
    sel = (slice(0, 1), heads[1])
    assert rel(o[sel], ro) <= TOL["bf16"]
    assert rel(S[sel], rS) <= TOL["bf16"]


def test_gated_workload_full_size():
    w = I.WORKLOADS["gated_bf16"]
    say(w)
    x = I.make_chunkwise(w)
    o, S = run_chunk(x, w.chunk, True)
    heads = ([0, 1], [0, 7, 15])
    ro, rS = oracle_chunk(x, True, heads=heads)
    sel = (slice(0, 2), heads[1])
    assert rel(o[:, heads[1]], ro) <= TOL["bf16"]
    assert rel(S[:, heads[1]], rS) <= TOL["bf16"]


@pytest.fixture(scope="module")
def decode_case():
    w = I.WORKLOADS["decode_bf16"]
    return w, I.make_decode(w)


def test_decode_workload_full_size(decode_case):
    """batch 128, H=32, d=128, 1024 consecutive steps on the full state; the oracle
    follows batch rows {0, 63, 127} (all 32 heads, every gamma) through every step."""
    w, x = decode_case
    say(w)
    rows = [0, 63, 127]
    S = x["state0"][0].cuda()
    gm = x["gamma"][0].cuda()
    q, k, v = (x[n].cuda() for n in ("q", "k", "v"))
    o_all = torch.empty(w.N, w.B, w.H, w.dv, dtype=torch.bfloat16, device="cuda")
    for t in range(w.N):
        R().retention_decode_step(q[t], k[t], v[t], gm, S, out=o_all[t])
    torch.cuda.synchronize()
    Sref = x["state0"][1][rows]
    qr, kr, vr = (x[n][:, rows].to(torch.float64).numpy() for n in ("q", "k", "v"))
    worst = 0.0
    o_np = o_all[:, rows].float().cpu().double().numpy()
    for t in range(w.N):
        ro, Sref = O.retention_decode_step(qr[t], kr[t], vr[t], x["gamma"][1], Sref)
        worst = max(worst, float(np.max(np.abs(o_np[t] - ro)) / np.max(np.abs(ro))))
    assert worst <= TOL["bf16"], worst
    assert rel(S[rows], Sref) <= TOL["bf16"]


def test_gated_decode_workload_full_size(decode_case):
    """The gated decode step at the decode workload's full shape (batch 128, H=32,
    d=128, the same S0 and q, k, v over 1024 steps) with per-step log-decays
    g_t = logsigmoid(x)/16; the oracle follows batch rows {0, 63, 127} through every step."""
    w, x = decode_case
    say(("gated", w))
    g = I.decode_log_decays(44, w.N, w.B, w.H)
    rows = [0, 63, 127]
    S = x["state0"][0].cuda()
    gd = g[0].cuda()
    q, k, v = (x[n].cuda() for n in ("q", "k", "v"))
    o_all = torch.empty(w.N, w.B, w.H, w.dv, dtype=torch.bfloat16, device="cuda")
    for t in range(w.N):
        R().gated_retention_decode_step(q[t], k[t], v[t], gd[t], S, out=o_all[t])
    torch.cuda.synchronize()
    Sref = x["state0"][1][rows]
    qr, kr, vr = (x[n][:, rows].to(torch.float64).numpy() for n in ("q", "k", "v"))
    gr = g[1][:, rows]
    worst = 0.0
    o_np = o_all[:, rows].float().cpu().double().numpy()
    for t in range(w.N):
        ro, Sref = O.gated_retention_decode_step(qr[t], kr[t], vr[t], gr[t], Sref)
        worst = max(worst, float(np.max(np.abs(o_np[t] - ro)) / np.max(np.abs(ro))))
    assert worst <= TOL["bf16"], worst
    assert rel(S[rows], Sref) <= TOL["bf16"]
