"""GPU parity of the backward entry points (through the C ABI) against the fp64 oracle's
backward (the adjoint recurrence, pinned to finite differences in test_oracle.py).

Tolerance (max|err| / max|ref| per gradient tensor): 1e-4 for fp32 inputs, 1e-2 for bf16
inputs, as for the forward.  Inputs: retnet_retention_fwd_amd.inputs (random_case for
q, k, v and the decays, backward_grads for the upstream gradients).
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


def say(msg):
    print(f"\n[case] {msg}", flush=True)


def gpu_bwd(x, gr, chunk, gated, state_in, dstate):
    d = lambda t: t[0].cuda()  # noqa: E731
    fn = R().gated_retention_chunkwise_bwd if gated else R().retention_chunkwise_bwd
    out = fn(d(x["q"]), d(x["k"]), d(x["v"]), d(x["g"] if gated else x["gamma"]), d(gr["grad_o"]), chunk,
             state_in=d(x["state_in"]) if state_in else None,
             grad_state_out=d(gr["grad_state_out"]) if dstate else None, return_grad_state_in=True)
    torch.cuda.synchronize()
    return out


def oracle_bwd(x, gr, gated, state_in, dstate, heads=None):
    q, k, v = x["q"][1], x["k"][1], x["v"][1]
    d = x["g"][1] if gated else x["gamma"][1]
    si = x["state_in"][1] if state_in else None
    do = gr["grad_o"][1]
    ds = gr["grad_state_out"][1] if dstate else None
    if heads is not None:
        b, h = heads
        q, k, v, do = q[b][:, h], k[b][:, h], v[b][:, h], do[b][:, h]
        si = None if si is None else si[b][:, h]
        ds = None if ds is None else ds[b][:, h]
        d = d[b][:, h] if gated else d[h]
    if gated:
        dq, dk, dv, dg, dS0 = O.gated_retention_recurrent_bwd(q, k, v, d, do, si, ds)
        return dict(dq=dq, dk=dk, dv=dv, dg=dg, dS0=dS0)
    dq, dk, dv, dS0 = O.retention_recurrent_bwd(q, k, v, d, do, si, ds)
    return dict(dq=dq, dk=dk, dv=dv, dS0=dS0)


def as_dict(out, gated):
    if gated:
        return dict(dq=out[0], dk=out[1], dv=out[2], dg=out[3], dS0=out[4])
    return dict(dq=out[0], dk=out[1], dv=out[2], dS0=out[3])


CASES = [
    # (B, H, N, dk, dv, chunk, dtype, gated, state_in, dstate): several tiles, ragged tails
    (1, 2, 100, 64, 64, 64, "bf16", False, True, True),
    (2, 2, 150, 128, 128, 64, "bf16", True, True, True),
    (1, 2, 77, 128, 128, 128, "bf16", False, False, False),
    (1, 1, 130, 64, 128, 64, "bf16", True, False, True),
    (1, 2, 90, 256, 512, 64, "bf16", False, True, True),     # d_v split into two score slices
    (1, 1, 70, 128, 384, 32, "bf16", True, True, True),      # three slices, gated
    (1, 2, 70, 32, 48, 16, "f32", False, True, True),        # generic kernels
    (1, 2, 66, 32, 48, 16, "f32", True, True, True),
    (1, 1, 50, 96, 80, 32, "f32", False, True, True),       # state transposes: partial 64x64 tiles
    (1, 2, 45, 21, 30, 16, "f32", True, True, True),        # sizes off multiples of 4: scalar transposes
    (1, 1, 17000, 16, 16, 64, "f32", True, False, True),    # gate scan: more than 16 tokens a thread
    (2, 1, 1, 64, 64, 64, "bf16", True, True, True),         # one token
    # few chains and long sequences: 32 segments, so the reversed per-head walk composes
    # its entry states in the separate scan (state_in divided by gamma there)
    (1, 2, 2000, 128, 128, 64, "bf16", False, True, True),
    # d_v slices as extra chains with 16 segments (scan with slice offsets), reversed dk pass
    (1, 1, 1000, 256, 512, 64, "bf16", False, True, True),
    (1, 1, 90, 128, 1024, 64, "bf16", False, True, True),     # the widest d_v: four slices
    (1, 1, 90, 128, 1024, 64, "bf16", True, True, True),
    # 128 chains x column tiles: two segments, so the reversed d_v pass walks the first
    # segment state-only in its second segment's workgroups (prefix split)
    (2, 32, 300, 128, 256, 64, "bf16", False, True, True),
    (2, 32, 300, 128, 256, 64, "bf16", True, True, True),
    (1, 2, 150, 256, 256, 64, "bf16", True, True, True),      # gated d_k = 256, fp32 dq and dk
    # row dots (gated, d_k = d_v = 128) in passes split in two segments: the reversed and the
    # forward walks with a state-only prefix
    (2, 64, 300, 128, 128, 64, "bf16", True, True, True),
    (1, 2, 1, 128, 128, 64, "bf16", True, True, True),        # one token: a single partial chunk
    (1, 1, 5, 256, 256, 64, "bf16", False, True, True),       # reversed d_k = 256 walk, five tokens
    # the dk pass reads the dv pass's segment states transposed: scanned entry states (19 and
    # 11 segments; gated row dots, and a per-head d_k = d_v = 256 walk), composed in the pass
    # (3 segments) as above at (2, 2, 150) and (1, 2, 150)
    (1, 1, 1200, 128, 128, 64, "bf16", True, True, True),
    (1, 1, 700, 256, 256, 64, "bf16", False, True, True),
    (1, 1, 700, 256, 256, 64, "bf16", False, False, False),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "x".join(map(str, c)))
def test_small_backward(case):
    B, H, N, dk, dv, C, dt, gated, si, ds = case
    say(("bwd", case))
    seed = sum(case[:6])
    x = I.random_case(seed, B, H, N, dk, dv, dtype=dt, gated=gated, state_in=si)
    gr = I.backward_grads(seed + 1, B, H, N, dk, dv, dtype=dt, state=ds)
    got = as_dict(gpu_bwd(x, gr, C, gated, si, ds), gated)
    ref = oracle_bwd(x, gr, gated, si, ds)
    for name, r in ref.items():
        assert rel(got[name], r) <= TOL[dt], (name, rel(got[name], r))


def test_empty_sequence_backward():
    """N = 0: no tokens, so S_N = S0 and grad_state_in = grad_state_out."""
    say("bwd empty")
    x = I.random_case(5, 1, 2, 0, 64, 64, dtype="bf16", state_in=True)
    gr = I.backward_grads(6, 1, 2, 0, 64, 64, dtype="bf16", state=True)
    out = gpu_bwd(x, gr, 64, False, True, True)
    assert out[0].numel() == 0
    assert torch.equal(out[3].cpu(), gr["grad_state_out"][0])


def test_train_shape_backward_sampled_heads():
    """Full train size (B=4 H=8 N=2048 dk=256 dv=512 chunk=64), in the configuration the
    benchmark times; the oracle checks two sampled (b,h) heads."""
    w = I.WORKLOADS["train_bf16"]
    say("bwd train full size")
    x = I.make_chunkwise(w, state_in=True)
    gr = I.backward_grads(101, w.B, w.H, w.N, w.dk, w.dv, dtype="bf16", state=True)
    got = as_dict(gpu_bwd(x, gr, w.chunk, False, True, True), False)
    for b, h in ((0, 0), (3, 7)):
        ref = oracle_bwd(x, gr, False, True, True, heads=(slice(b, b + 1), slice(h, h + 1)))
        for name, r in ref.items():
            g = got[name][b:b + 1, h:h + 1]
            assert rel(g, r) <= TOL["bf16"], (b, h, name, rel(g, r))


def test_gated_shape_backward_sampled_head():
    """Gated workload size (B=2 H=16 N=8192 dk=dv=128 chunk=64); one sampled head."""
    w = I.WORKLOADS["gated_bf16"]
    say("bwd gated full size")
    x = I.make_chunkwise(w, state_in=True)
    gr = I.backward_grads(102, w.B, w.H, w.N, w.dk, w.dv, dtype="bf16", state=True)
    got = as_dict(gpu_bwd(x, gr, w.chunk, True, True, True), True)
    b, h = 1, 9
    ref = oracle_bwd(x, gr, True, True, True, heads=(slice(b, b + 1), slice(h, h + 1)))
    for name, r in ref.items():
        g = got[name][b:b + 1, h:h + 1]
        assert rel(g, r) <= TOL["bf16"], (name, rel(g, r))


def test_backward_matches_autograd_reference():
    """A different route to the same gradients: torch autograd through a float64 PyTorch
    recurrence on the CPU (no oracle code), on a small case."""
    say("bwd vs autograd")
    B, H, N, dk, dv = 1, 2, 40, 64, 64
    x = I.random_case(77, B, H, N, dk, dv, dtype="bf16", gated=True, state_in=True)
    gr = I.backward_grads(78, B, H, N, dk, dv, dtype="bf16", state=True)
    got = as_dict(gpu_bwd(x, gr, 16, True, True, True), True)
    t = {n: torch.tensor(x[n][1], requires_grad=True) for n in ("q", "k", "v", "g", "state_in")}
    S = t["state_in"]
    outs = []
    for n in range(N):
        S = torch.exp(t["g"][:, :, n])[..., None, None] * S + t["k"][:, :, n, :, None] * t["v"][:, :, n, None, :]
        outs.append(torch.einsum("bhi,bhij->bhj", t["q"][:, :, n], S))
    o = torch.stack(outs, dim=2)
    L = (o * torch.tensor(gr["grad_o"][1])).sum() + (S * torch.tensor(gr["grad_state_out"][1])).sum()
    L.backward()
    for name, key in (("dq", "q"), ("dk", "k"), ("dv", "v"), ("dg", "g"), ("dS0", "state_in")):
        assert rel(got[name], t[key].grad.numpy()) <= TOL["bf16"], name
