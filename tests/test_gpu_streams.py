"""The library on a caller's stream and inside a captured HIP graph.

Every entry point enqueues on the stream it is given and allocates nothing, so its
launches can be captured.  The graph test replays a captured forward (with the segment
pre-pass), a gated backward and a run of decode steps several times, with eager work
between replays, and compares every replay bit for bit with the eager result (the
kernels are deterministic).
"""
import pytest

from retnet_retention_fwd_amd import inputs as I

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def R():
    import retnet_retention_fwd_amd as R_
    return R_


def _case():
    x = I.random_case(21, 1, 4, 1500, 128, 128, dtype="bf16", gated=True, state_in=True)
    return {n: t[0].cuda() for n, t in x.items()}


def test_side_stream_matches_default_stream():
    print("\n[case] side stream", flush=True)
    x = _case()
    ws = torch.empty(max(R().workspace_bytes(1, 4, 1500, 128, 128, 64, 1, True), 1), dtype=torch.uint8, device="cuda")
    ref = R().gated_retention_chunkwise_fwd(x["q"], x["k"], x["v"], x["g"], 64, state_in=x["state_in"], workspace=ws)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        ws2 = torch.empty_like(ws)
        out = R().gated_retention_chunkwise_fwd(x["q"], x["k"], x["v"], x["g"], 64, state_in=x["state_in"],
                                                workspace=ws2)
    side.synchronize()
    assert torch.equal(out, ref)


def test_explicit_stream_without_workspace():
    """stream= names a side stream and the wrapper allocates the workspace and the output
    itself: both must belong to that stream, so that memory freed after the call is not
    handed to the current stream's work while the side stream's kernels still use it."""
    print("\n[case] explicit stream, wrapper-allocated workspace", flush=True)
    x = _case()
    ref = R().gated_retention_chunkwise_fwd(x["q"], x["k"], x["v"], x["g"], 64, state_in=x["state_in"])
    torch.cuda.synchronize()
    nbytes = R().workspace_bytes(1, 4, 1500, 128, 128, 64, 1, True)
    assert nbytes > 0
    side = torch.cuda.Stream()
    outs = []
    for rep in range(4):
        side.wait_stream(torch.cuda.current_stream())
        outs.append(R().gated_retention_chunkwise_fwd(x["q"], x["k"], x["v"], x["g"], 64, state_in=x["state_in"],
                                                      stream=side))
        # the current stream allocates blocks of the workspace's size and overwrites them
        # at once, while the side stream may still be running
        junk = [torch.full((nbytes,), 255, dtype=torch.uint8, device="cuda") for _ in range(2)]
        junk += [torch.full(tuple(ref.shape), 7.0, dtype=ref.dtype, device="cuda")]
        del junk
    side.synchronize()
    torch.cuda.synchronize()
    for rep, out in enumerate(outs):
        assert torch.equal(out, ref), rep


def test_graph_capture_and_replay():
    print("\n[case] graph capture", flush=True)
    x = _case()
    B, H, N, d = 1, 4, 1500, 128
    gm = torch.tensor([0.9, 0.95, 0.99, 0.999], device="cuda")
    grad_o = torch.randn(B, H, N, d, device="cuda").to(torch.bfloat16)
    S_dec = torch.randn(2, H, d, d, device="cuda") * 0.1
    qd, kd, vd = (torch.randn(8, 2, H, d, device="cuda").to(torch.bfloat16) for _ in range(3))
    # static buffers the graph reads and writes
    o = torch.empty(B, H, N, d, dtype=torch.bfloat16, device="cuda")
    fws = torch.empty(max(R().workspace_bytes(B, H, N, d, d, 64, 1, False), 1), dtype=torch.uint8, device="cuda")
    bws = torch.empty(max(R().bwd_workspace_bytes(B, H, N, d, d, 64, 1, True), 1), dtype=torch.uint8, device="cuda")
    od = torch.empty(2, H, d, dtype=torch.bfloat16, device="cuda")
    S_work = torch.empty_like(S_dec)

    def work():
        R().retention_chunkwise_fwd(x["q"], x["k"], x["v"], gm, 64, out=o, workspace=fws)
        grads = R().gated_retention_chunkwise_bwd(x["q"], x["k"], x["v"], x["g"], grad_o, 64, state_in=x["state_in"],
                                                  workspace=bws)
        S_work.copy_(S_dec)
        for t in range(8):
            R().retention_decode_step(qd[t], kd[t], vd[t], gm, S_work, out=od)
        return grads

    # eager reference (also sets every kernel attribute before the capture)
    g_eager = [t.clone() for t in work()]
    o_eager, od_eager, S_eager = o.clone(), od.clone(), S_work.clone()
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            g_static = work()
    torch.cuda.current_stream().wait_stream(side)
    for rep in range(3):
        o.zero_()
        od.zero_()
        for t in g_static:
            t.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, o_eager), rep
        assert torch.equal(od, od_eager), rep
        assert torch.equal(S_work, S_eager), rep
        for a, b in zip(g_static, g_eager):
            assert torch.equal(a, b), rep
        # eager work between replays
        R().retention_chunkwise_fwd(x["q"], x["k"], x["v"], gm, 64)
        torch.cuda.synchronize()


def test_calibration_loop_runs():
    """The matrix-core loop reference runs and reports its flop count."""
    print("\n[case] matrix-core loop reference", flush=True)
    out = torch.empty(4 * 8, dtype=torch.float32, device="cuda")
    flops = R().calib_mfma(4, 8, 10, out=out)
    torch.cuda.synchronize()
    assert flops == 4 * 8 * 10 * 16 * 16384
    assert torch.all(torch.isfinite(out))
