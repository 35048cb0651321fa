"""GPU check of the entry point that allocates nothing (retention_chunkwise_fwd_noalloc),
called through the C ABI, against retention_chunkwise_fwd with a caller workspace: two
calls in a row, the second on a smaller input, each compared bit for bit (both run the
same kernels on the same inputs)."""
import ctypes

import pytest

from retnet_retention_fwd_amd import inputs as I

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def R():
    import retnet_retention_fwd_amd as R_
    return R_


@pytest.mark.parametrize("order", ["large_then_small"])
def test_noalloc_matches_workspace_entry_point(order):
    L = R().lib()
    vp = ctypes.c_void_p
    # (B, H, N, d, chunk): segmented sequences that need scratch; the second is smaller
    cases = [(1, 4, 3000, 128, 64), (1, 2, 900, 128, 100)]
    for i, (B, H, N, d, C) in enumerate(cases):
        print(f"\n[case] noalloc {order} #{i}: B{B} H{H} N{N} d{d} C{C}", flush=True)
        need = R().workspace_bytes(B, H, N, d, d, C, 1, False)
        assert 0 < need <= 32 << 20
        x = I.random_case(100 + i, B, H, N, d, d, dtype="bf16", state_in=True)
        q, k, v, gm, si = (x[n][0].cuda() for n in ("q", "k", "v", "gamma", "state_in"))
        ref, S_ref = R().retention_chunkwise_fwd(q, k, v, gm, C, state_in=si, return_state=True)
        o = torch.full_like(ref, 7.0)
        S = torch.full_like(S_ref, 3.0)
        stream = torch.cuda.current_stream()
        st = L.retention_chunkwise_fwd_noalloc(vp(q.data_ptr()), vp(k.data_ptr()), vp(v.data_ptr()),
                                               vp(gm.data_ptr()), vp(o.data_ptr()), vp(si.data_ptr()),
                                               vp(S.data_ptr()), B, H, N, d, d, C, 1, vp(stream.cuda_stream))
        assert st == 0, R().lib().retention_status_string(st)
        torch.cuda.synchronize()
        assert torch.equal(o, ref), i
        assert torch.equal(S, S_ref), i
