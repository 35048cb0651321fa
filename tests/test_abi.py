"""Host-side checks of the C ABI (no GPU needed: every call here fails validation and so
returns before anything is enqueued)."""
import ctypes
import os
import re

import pytest

from retnet_retention_fwd_amd import _lib

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "retention.h")

OK, ERR_NULL, ERR_SHAPE, ERR_DTYPE, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_ALIAS, ERR_HIP = range(8)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b([a-z_][a-z0-9_]*)\s*\(", text)) - {"defined"})


@pytest.fixture(scope="module")
def L():
    return _lib.lib()


def test_every_declared_symbol_is_exported(L):
    names = declared_functions()
    assert set(names) == set(_lib.EXPORTED), names
    for n in names:
        assert hasattr(L, n), n


def test_abi_version_and_status_strings(L):
    assert L.retention_abi_version() == 1
    for s in range(8):
        assert _lib.status_string(s)
    assert _lib.status_string(99) == "unknown status"


FAKE = 1 << 40          # never dereferenced: validation fails before any launch
MB = 1 << 20


def chunk(L, q=FAKE, k=FAKE + 64 * MB, v=FAKE + 128 * MB, d=FAKE + 192 * MB, o=FAKE + 256 * MB,
          si=None, so=None, B=1, H=2, N=64, dk=16, dv=16, C=16, dt=0, ws=None, wsb=0, gated=False):
    f = L.gated_retention_chunkwise_fwd if gated else L.retention_chunkwise_fwd
    return f(q, k, v, d, o, si, so, B, H, N, dk, dv, C, dt, ws, wsb, None)


@pytest.mark.parametrize("gated", [False, True])
def test_chunk_validation(L, gated):
    c = lambda **kw: chunk(L, gated=gated, **kw)  # noqa: E731
    assert c(dt=7) == ERR_DTYPE
    assert c(B=-1) == ERR_SHAPE
    assert c(N=-3) == ERR_SHAPE
    assert c(dk=0) == ERR_SHAPE
    assert c(C=0) == ERR_SHAPE
    assert c(dk=257) == ERR_UNSUPPORTED
    assert c(dv=2000) == ERR_UNSUPPORTED
    assert c(q=None) == ERR_NULL
    assert c(o=None) == ERR_NULL
    assert c(d=None) == ERR_NULL
    # output overlapping an input
    assert c(o=FAKE + 100) == ERR_ALIAS
    assert c(so=FAKE + 64 * MB) == ERR_ALIAS                 # state_out over k
    assert c(si=FAKE + 300 * MB, so=FAKE + 300 * MB + 16) == ERR_ALIAS   # partial overlap
    # gated long chunks on the generic (fp32) path need their cumsum in LDS
    if gated:
        assert c(N=4096, C=2048) == ERR_UNSUPPORTED
    # bf16 matrix-core path with a split sequence needs workspace
    need = L.retention_workspace_bytes(1, 2, 65536, 128, 128, 64, 1, int(gated))
    assert need > 0
    assert c(N=65536, dk=128, dv=128, C=64, dt=1) == ERR_WORKSPACE
    assert c(N=65536, dk=128, dv=128, C=64, dt=1, ws=FAKE + 400 * MB, wsb=need - 1) == ERR_WORKSPACE
    # the segment states are written in 16-byte units: a misaligned workspace is refused
    assert c(N=65536, dk=128, dv=128, C=64, dt=1, ws=FAKE + 400 * MB + 4, wsb=need) == ERR_WORKSPACE


def test_decode_validation(L):
    f = L.retention_decode_step
    args = dict(q=FAKE, k=FAKE + MB, v=FAKE + 2 * MB, d=FAKE + 3 * MB, s=FAKE + 4 * MB, o=FAKE + 8 * MB)

    def call(B=2, H=2, dk=16, dv=16, dt=1, **kw):
        a = dict(args, **kw)
        return f(a["q"], a["k"], a["v"], a["d"], a["s"], a["o"], B, H, dk, dv, dt, None)

    assert call(dt=5) == ERR_DTYPE
    assert call(B=-1) == ERR_SHAPE
    assert call(dk=0) == ERR_SHAPE
    assert call(dk=300) == ERR_UNSUPPORTED
    assert call(s=None) == ERR_NULL
    assert call(o=FAKE + 4 * MB + 8) == ERR_ALIAS       # o inside the state
    assert call(s=FAKE + 2 * MB) == ERR_ALIAS            # state over v
    assert call(B=0) == OK                               # empty: nothing to do, nothing launched
    g = L.gated_retention_decode_step
    assert g(FAKE, FAKE + MB, FAKE + 2 * MB, None, FAKE + 4 * MB, FAKE + 8 * MB, 2, 2, 16, 16, 1, None) == ERR_NULL


def test_workspace_query(L):
    # fp32 and generic shapes never need workspace
    assert L.retention_workspace_bytes(1, 2, 64, 16, 16, 16, 0, 0) == 0
    # a short sequence with enough (b,h) x column tiles runs unsplit
    assert L.retention_workspace_bytes(16, 16, 2048, 128, 128, 64, 1, 0) == 0
    # two segments of 64-token chunks: the second walks the first state-only, no workspace
    assert L.retention_workspace_bytes(4, 8, 2048, 256, 512, 64, 1, 0) == 0
    assert L.retention_workspace_bytes(2, 8, 2048, 128, 1024, 64, 1, 1) == 0
    # long sequences with few heads are split; workspace holds one fp32 state per segment
    ws = L.retention_workspace_bytes(1, 16, 16384, 128, 128, 512, 1, 0)
    assert ws >= 2 * 16 * 128 * 128 * 4
    assert L.retention_workspace_bytes(2, 16, 8192, 128, 128, 64, 1, 1) >= 2 * 2 * 16 * 128 * 128 * 4
    assert L.retention_workspace_bytes(-1, 2, 64, 16, 16, 16, 0, 0) == 0


def test_long_heads_leave_the_matrix_core_path(L):
    # The matrix-core kernels address one head's rows with 32-bit byte offsets: a head
    # whose rows span 2^31 bytes or more runs on the generic kernel (no workspace), its
    # backward with d_v > 256 and the gated layer are reported unsupported.
    n_fit = (1 << 30) // 1024 - 64 - 1          # (N + 64) * 1024 * 2 < 2^31
    n_over = n_fit + 1
    assert L.retention_workspace_bytes(1, 1, n_fit, 256, 1024, 64, 1, 0) > 0
    assert L.retention_workspace_bytes(1, 1, n_over, 256, 1024, 64, 1, 0) == 0
    assert L.retention_workspace_bytes(1, 1, n_over, 256, 1024, 64, 1, 1) == 0
    assert L.retention_bwd_workspace_bytes(1, 1, n_fit, 256, 1024, 64, 1, 0) > 0
    assert L.retention_bwd_workspace_bytes(1, 1, n_over, 256, 1024, 64, 1, 0) == 0
    n_fit = (1 << 30) // 128 - 64 - 1
    assert L.gated_msr_workspace_bytes(1, n_fit, 128, 1, 128, 128, 64) > 0
    assert L.gated_msr_workspace_bytes(1, n_fit + 1, 128, 1, 128, 128, 64) == 0


def bwd(L, gated=False, q=FAKE, k=FAKE + 64 * MB, v=FAKE + 128 * MB, d=FAKE + 192 * MB, si=None,
        go=FAKE + 256 * MB, gso=None, gq=FAKE + 320 * MB, gk=FAKE + 384 * MB, gv=FAKE + 448 * MB,
        gg=FAKE + 512 * MB, gsi=None, B=1, H=2, N=64, dk=16, dv=16, C=16, dt=0, ws=None, wsb=0):
    if gated:
        return L.gated_retention_chunkwise_bwd(q, k, v, d, si, go, gso, gq, gk, gv, gg, gsi, B, H, N, dk, dv, C, dt,
                                               ws, wsb, None)
    return L.retention_chunkwise_bwd(q, k, v, d, si, go, gso, gq, gk, gv, gsi, B, H, N, dk, dv, C, dt, ws, wsb,
                                     None)


@pytest.mark.parametrize("gated", [False, True])
def test_backward_validation(L, gated):
    c = lambda **kw: bwd(L, gated=gated, **kw)  # noqa: E731
    assert c(dt=9) == ERR_DTYPE
    assert c(N=-1) == ERR_SHAPE
    assert c(dk=300) == ERR_UNSUPPORTED
    assert c(go=None) == ERR_NULL
    assert c(gq=None) == ERR_NULL
    if gated:
        assert c(gg=None) == ERR_NULL
    assert c(gq=FAKE + 100) == ERR_ALIAS                     # grad_q over q
    assert c(gv=FAKE + 320 * MB) == ERR_ALIAS                # grad_v over grad_q
    assert c(gsi=FAKE + 256 * MB) == ERR_ALIAS               # grad_state_in over grad_o
    # fp32 with d_v above the score width of the kernels
    assert c(dv=512) == ERR_UNSUPPORTED
    # an initial state needs workspace (its transposed copy)
    need = L.retention_bwd_workspace_bytes(1, 2, 64, 16, 16, 16, 1, int(gated))
    assert need > 0
    si = FAKE + 700 * MB
    assert c(dt=1, si=si) == ERR_WORKSPACE
    assert c(dt=1, si=si, ws=FAKE + 600 * MB, wsb=16) == ERR_WORKSPACE
    assert c(dt=1, si=si, ws=FAKE + 600 * MB + 4, wsb=need) == ERR_WORKSPACE   # 16-byte alignment
    assert c(B=0) == OK                                                   # nothing to do


def test_backward_workspace_query(L):
    # the d_v split needs a partial-sum buffer; every size is positive for a real shape
    a = L.retention_bwd_workspace_bytes(4, 8, 2048, 256, 512, 64, 1, 0)
    b = L.retention_bwd_workspace_bytes(4, 8, 2048, 256, 256, 64, 1, 0)
    assert a > b > 0
    assert L.retention_bwd_workspace_bytes(1, 1, 64, 16, 512, 16, 0, 0) == 0   # fp32, d_v > 256
    assert L.retention_bwd_workspace_bytes(-1, 1, 64, 16, 16, 16, 0, 0) == 0
    assert L.retention_bwd_workspace_bytes(1, 1, 0, 16, 16, 16, 1, 1) == 0     # no tokens


@pytest.mark.parametrize("gated", [False, True])
def test_parallel_validation(L, gated):
    f = L.gated_retention_parallel_fwd if gated else L.retention_parallel_fwd

    def c(q=FAKE, k=FAKE + 64 * MB, v=FAKE + 128 * MB, d=FAKE + 192 * MB, o=FAKE + 256 * MB, B=1, H=2, N=64,
          dk=16, dv=16, dt=1):
        return f(q, k, v, d, o, B, H, N, dk, dv, dt, None)

    assert c(dt=4) == ERR_DTYPE
    assert c(N=-1) == ERR_SHAPE
    assert c(dk=512) == ERR_UNSUPPORTED
    assert c(d=None) == ERR_NULL
    assert c(o=None) == ERR_NULL
    assert c(o=FAKE + 64 * MB) == ERR_ALIAS      # o over k
    assert c(B=0) == OK and c(N=0) == OK          # nothing to do


def test_msr_validation(L):
    def c(x=FAKE, y=FAKE + 700 * MB, B=1, N=64, D=128, H=8, dk=64, dv=64, C=64, base=10000.0, eps=1e-5, ws=None,
          wsb=0):
        w = [FAKE + (64 + 32 * i) * MB for i in range(6)]
        return L.gated_msr_fwd(x, *w, y, B, N, D, H, dk, dv, C, base, eps, ws, wsb, None)

    assert c(D=0) == ERR_SHAPE
    assert c(base=1.0) == ERR_SHAPE
    assert c(eps=-1.0) == ERR_SHAPE
    assert c(dk=48) == ERR_UNSUPPORTED          # head size off the matrix-core shapes
    assert c(D=100) == ERR_UNSUPPORTED          # reduction not a multiple of 64
    assert c(x=None) == ERR_NULL
    assert c(y=FAKE + 64 * MB) == ERR_ALIAS     # y over wq
    need = L.gated_msr_workspace_bytes(1, 64, 128, 8, 64, 64, 64)
    assert need > 0
    assert c() == ERR_WORKSPACE
    assert c(ws=FAKE + 900 * MB, wsb=need - 1) == ERR_WORKSPACE
    assert c(B=0) == OK and c(N=0) == OK
    assert L.gated_msr_workspace_bytes(1, 64, 100, 8, 64, 64, 64) == 0


def test_profile_read_validation(L):
    assert L.retention_profile_read(None, None, -1, None) == ERR_SHAPE
    assert L.retention_profile_read(None, None, 2, None) == ERR_NULL
    assert L.retention_profile_read(None, None, 0, None) == OK     # nothing recorded


def test_python_binding_rejects_cpu_tensors():
    import torch
    from retnet_retention_fwd_amd import retention_chunkwise_fwd
    q = torch.zeros(1, 1, 4, 16)
    with pytest.raises(ValueError):
        retention_chunkwise_fwd(q, q, q, torch.ones(1), 4)


def test_decode_wrapper_rejects_wrong_out_shape(monkeypatch):
    """The C entry point sees only pointers, so the binding checks the shape of a
    caller's `out`; a smaller one would let the kernel write past it."""
    torch = pytest.importorskip("torch")

    def lenient(t, name, dtype=None, device=None):   # host tensors stand in for device ones
        if dtype is not None and t.dtype != dtype:
            raise TypeError(name)

    monkeypatch.setattr(_lib, "_require", lenient)
    B, H, d = 2, 3, 16
    q = torch.zeros(B, H, d, dtype=torch.bfloat16)
    gamma = torch.full((H,), 0.9)
    state = torch.zeros(B, H, d, d)
    for bad in ((B, H, d // 2), (B, H - 1, d), (B * H * d,)):
        out = torch.zeros(bad, dtype=torch.bfloat16)
        with pytest.raises(ValueError, match="out must be"):
            _lib.retention_decode_step(q, q, q, gamma, state, out=out)
        with pytest.raises(ValueError, match="out must be"):
            _lib.gated_retention_decode_step(q, q, q, torch.zeros(B, H), state, out=out)


def test_calibration_loop_validation(L):
    """The matrix-core loop reference validates its arguments before launching."""
    assert L.retention_calib_mfma(None, 1, 1, 1, None) == ERR_NULL
    assert L.retention_calib_mfma(FAKE, 0, 1, 1, None) == ERR_SHAPE
    assert L.retention_calib_mfma(FAKE, 1, 9, 1, None) == ERR_SHAPE
    assert L.retention_calib_mfma(FAKE, 1, 1, 0, None) == ERR_SHAPE
    # 256 workgroups x 8 waves x 10 rounds x 16 products of 2*16*16*32 flops
    assert L.retention_calib_mfma_flops(256, 8, 10) == 256 * 8 * 10 * 16 * 16384


def test_noalloc_rejects_calls_beyond_its_scratch(L):
    """The entry point without workspace refuses a call that would need more scratch
    than its fixed array holds, before anything touches the GPU."""
    cap = 32 << 20
    need = L.retention_workspace_bytes(1, 255, 200, 256, 128, 48, 1, 0)
    assert need > cap
    f = L.retention_chunkwise_fwd_noalloc
    st = f(FAKE, FAKE + 64 * MB, FAKE + 128 * MB, FAKE + 192 * MB, FAKE + 256 * MB, None, None,
           1, 255, 200, 256, 128, 48, 1, None)
    assert st == ERR_WORKSPACE
    # invalid arguments are still reported as such (nothing is launched)
    assert f(FAKE, FAKE, FAKE, FAKE, FAKE, None, None, 1, 2, 64, 16, 16, 16, 7, None) == ERR_DTYPE
    assert f(None, FAKE, FAKE, FAKE, FAKE, None, None, 1, 2, 64, 16, 16, 16, 0, None) == ERR_NULL
