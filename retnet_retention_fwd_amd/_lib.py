"""ctypes binding of libretention_fwd.so (the C ABI declared in include/retention.h).

Argument marshalling only: every step of the operator runs in the library's HIP
kernels.  torch provides device memory (outputs, workspace) and the current stream.
If the library is missing or cannot be loaded, every call raises; there is no other
code path.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libretention_fwd.so")

RETN_F32 = 0
RETN_BF16 = 1

STATUS_NAMES = {
    0: "RETN_OK", 1: "RETN_ERR_NULL", 2: "RETN_ERR_SHAPE", 3: "RETN_ERR_DTYPE",
    4: "RETN_ERR_UNSUPPORTED", 5: "RETN_ERR_WORKSPACE", 6: "RETN_ERR_ALIAS", 7: "RETN_ERR_HIP",
}

# Every symbol include/retention.h declares.
EXPORTED = (
    "retention_chunkwise_fwd",
    "gated_retention_chunkwise_fwd",
    "retention_decode_step",
    "gated_retention_decode_step",
    "retention_workspace_bytes",
    "retention_status_string",
    "retention_abi_version",
    "retention_profile_enable",
    "retention_profile_read",
    "retention_chunkwise_bwd",
    "gated_retention_chunkwise_bwd",
    "retention_bwd_workspace_bytes",
    "retention_parallel_fwd",
    "gated_retention_parallel_fwd",
    "gated_msr_fwd",
    "gated_msr_workspace_bytes",
    "retention_calib_mfma",
    "retention_calib_mfma_flops",
    "retention_chunkwise_fwd_noalloc",
)

# Kernel kinds reported by retention_profile_read.
PROFILE_KINDS = ("chunk_main", "chunk_prepass", "chunk_scan", "chunk_generic", "decode", "state_copy")


class RetentionError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        super().__init__(f"{where}: {STATUS_NAMES.get(status, status)} ({detail})")
        self.status = status


_lib = None

_vp = ctypes.c_void_p
_i = ctypes.c_int
_sz = ctypes.c_size_t


def lib() -> ctypes.CDLL:
    """Load the library once; raise if it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run `python -m retnet_retention_fwd_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    chunk_sig = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _vp, _sz, _vp]
    for name in ("retention_chunkwise_fwd", "gated_retention_chunkwise_fwd"):
        f = getattr(L, name)
        f.argtypes = chunk_sig
        f.restype = ctypes.c_int
    for name in ("retention_decode_step", "gated_retention_decode_step"):
        f = getattr(L, name)
        f.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _vp]
        f.restype = ctypes.c_int
    L.retention_workspace_bytes.argtypes = [_i, _i, _i, _i, _i, _i, _i, _i]
    L.retention_workspace_bytes.restype = _sz
    L.retention_status_string.argtypes = [_i]
    L.retention_status_string.restype = ctypes.c_char_p
    L.retention_abi_version.argtypes = []
    L.retention_abi_version.restype = ctypes.c_int
    L.retention_profile_enable.argtypes = [_i]
    L.retention_profile_enable.restype = ctypes.c_int
    L.retention_profile_read.argtypes = [_vp, _vp, _i, _vp]
    L.retention_profile_read.restype = ctypes.c_int
    L.retention_chunkwise_bwd.argtypes = [_vp] * 11 + [_i] * 7 + [_vp, _sz, _vp]
    L.retention_chunkwise_bwd.restype = ctypes.c_int
    L.gated_retention_chunkwise_bwd.argtypes = [_vp] * 12 + [_i] * 7 + [_vp, _sz, _vp]
    L.gated_retention_chunkwise_bwd.restype = ctypes.c_int
    L.retention_bwd_workspace_bytes.argtypes = [_i, _i, _i, _i, _i, _i, _i, _i]
    L.retention_bwd_workspace_bytes.restype = _sz
    for name in ("retention_parallel_fwd", "gated_retention_parallel_fwd"):
        f = getattr(L, name)
        f.argtypes = [_vp] * 5 + [_i] * 6 + [_vp]
        f.restype = ctypes.c_int
    L.gated_msr_fwd.argtypes = [_vp] * 8 + [_i] * 7 + [ctypes.c_float, ctypes.c_float, _vp, _sz, _vp]
    L.gated_msr_fwd.restype = ctypes.c_int
    L.gated_msr_workspace_bytes.argtypes = [_i] * 7
    L.gated_msr_workspace_bytes.restype = _sz
    L.retention_calib_mfma.argtypes = [_vp, _i, _i, _i, _vp]
    L.retention_calib_mfma.restype = ctypes.c_int
    L.retention_calib_mfma_flops.argtypes = [_i, _i, _i]
    L.retention_calib_mfma_flops.restype = ctypes.c_double
    L.retention_chunkwise_fwd_noalloc.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _vp]
    L.retention_chunkwise_fwd_noalloc.restype = ctypes.c_int
    _lib = L
    return L


def status_string(status: int) -> str:
    return lib().retention_status_string(status).decode()


def _check(status: int, where: str):
    if status != 0:
        raise RetentionError(status, where, status_string(status))


def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return RETN_BF16
    if t.dtype == torch.float32:
        return RETN_F32
    raise TypeError(f"q/k/v must be bfloat16 or float32, got {t.dtype}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _require(t, name, dtype=None, device=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _stream(stream):
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _on_stream(stream):
    """Context in which the wrapper allocates its outputs and workspace: the stream the
    kernels run on, so that torch's caching allocator hands a freed block out again only
    in that stream's order (a block allocated on another stream could be reused there
    while the kernels still read or write it)."""
    import contextlib
    torch = _torch()
    return contextlib.nullcontext() if stream is None else torch.cuda.stream(stream)


def workspace_bytes(B, H, N, dk, dv, chunk, dtype_code, gated) -> int:
    return int(lib().retention_workspace_bytes(B, H, N, dk, dv, chunk, dtype_code, 1 if gated else 0))


def _chunk_call_impl(fn_name, q, k, v, decay, chunk, state_in, return_state, out, state_out, stream,
                workspace, gated):
    torch = _torch()
    L = lib()
    _require(q, "q")
    dev = q.device
    _require(k, "k", q.dtype, dev)
    _require(v, "v", q.dtype, dev)
    _require(decay, "g" if gated else "gamma", torch.float32, dev)
    if q.dim() != 4 or k.shape != q.shape or v.dim() != 4 or v.shape[:3] != q.shape[:3]:
        raise ValueError(f"expected q,k [B,H,N,dk] and v [B,H,N,dv]; got {tuple(q.shape)} "
                         f"{tuple(k.shape)} {tuple(v.shape)}")
    B, H, N, dk = q.shape
    dv = v.shape[-1]
    exp_decay = (B, H, N) if gated else (H,)
    if tuple(decay.shape) != exp_decay:
        raise ValueError(f"decay must have shape {exp_decay}, got {tuple(decay.shape)}")
    if state_in is not None:
        _require(state_in, "state_in", torch.float32, dev)
        if tuple(state_in.shape) != (B, H, dk, dv):
            raise ValueError("state_in must be [B,H,dk,dv]")
    if out is None:
        out = torch.empty((B, H, N, dv), dtype=q.dtype, device=dev)
    else:
        _require(out, "out", q.dtype, dev)
        if tuple(out.shape) != (B, H, N, dv):
            raise ValueError("out must be [B,H,N,dv]")
    if state_out is None and return_state:
        state_out = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    elif state_out is not None:
        _require(state_out, "state_out", torch.float32, dev)
        if tuple(state_out.shape) != (B, H, dk, dv):
            raise ValueError("state_out must be [B,H,dk,dv]")
    code = _dtype_code(q)
    ws_need = workspace_bytes(B, H, N, dk, dv, chunk, code, gated)
    if workspace is None and ws_need > 0:
        workspace = torch.empty(ws_need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = getattr(L, fn_name)(_ptr(q), _ptr(k), _ptr(v), _ptr(decay), _ptr(out), _ptr(state_in),
                             _ptr(state_out), B, H, N, dk, dv, int(chunk), code, _ptr(workspace),
                             ws_bytes, _stream(stream))
    _check(st, fn_name)
    return (out, state_out) if (return_state or state_out is not None) else out


def _chunk_call(fn_name, q, k, v, decay, chunk, state_in, return_state, out, state_out, stream, workspace, gated):
    with _on_stream(stream):
        return _chunk_call_impl(fn_name, q, k, v, decay, chunk, state_in, return_state, out, state_out, stream,
                                workspace, gated)


def retention_chunkwise_fwd(q, k, v, gamma, chunk, state_in=None, return_state=False, out=None,
                            state_out=None, stream=None, workspace=None):
    """Chunkwise retention forward with per-head decays gamma[H] (fp32).

    q, k: [B,H,N,dk], v: [B,H,N,dv] (bf16 or fp32, contiguous, on the GPU).  Returns o
    [B,H,N,dv] in the input dtype, or (o, state_out) if return_state or state_out is given.
    """
    return _chunk_call("retention_chunkwise_fwd", q, k, v, gamma, chunk, state_in, return_state, out,
                       state_out, stream, workspace, False)


def retention_chunkwise_fwd_noalloc(q, k, v, gamma, chunk, state_in=None, return_state=False, out=None,
                                    state_out=None, stream=None):
    """retention_chunkwise_fwd whose scratch comes from the library's own fixed device array
    (for callers that cannot allocate; pass out and state_out to allocate nothing here
    either).  Calls that overlap on one device race on that array."""
    with _on_stream(stream):
        return _noalloc_impl(q, k, v, gamma, chunk, state_in, return_state, out, state_out, stream)


def _noalloc_impl(q, k, v, gamma, chunk, state_in, return_state, out, state_out, stream):
    torch = _torch()
    L = lib()
    _require(q, "q")
    dev = q.device
    _require(k, "k", q.dtype, dev)
    _require(v, "v", q.dtype, dev)
    _require(gamma, "gamma", torch.float32, dev)
    if q.dim() != 4 or k.shape != q.shape or v.dim() != 4 or v.shape[:3] != q.shape[:3]:
        raise ValueError(f"expected q,k [B,H,N,dk] and v [B,H,N,dv]; got {tuple(q.shape)} "
                         f"{tuple(k.shape)} {tuple(v.shape)}")
    B, H, N, dk = q.shape
    dv = v.shape[-1]
    if tuple(gamma.shape) != (H,):
        raise ValueError(f"gamma must have shape {(H,)}, got {tuple(gamma.shape)}")
    if state_in is not None:
        _require(state_in, "state_in", torch.float32, dev)
        if tuple(state_in.shape) != (B, H, dk, dv):
            raise ValueError("state_in must be [B,H,dk,dv]")
    if out is None:
        out = torch.empty((B, H, N, dv), dtype=q.dtype, device=dev)
    else:
        _require(out, "out", q.dtype, dev)
        if tuple(out.shape) != (B, H, N, dv):
            raise ValueError("out must be [B,H,N,dv]")
    if state_out is None and return_state:
        state_out = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    elif state_out is not None:
        _require(state_out, "state_out", torch.float32, dev)
        if tuple(state_out.shape) != (B, H, dk, dv):
            raise ValueError("state_out must be [B,H,dk,dv]")
    st = L.retention_chunkwise_fwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(gamma), _ptr(out), _ptr(state_in),
                                           _ptr(state_out), B, H, N, dk, dv, int(chunk), _dtype_code(q),
                                           _stream(stream))
    _check(st, "retention_chunkwise_fwd_noalloc")
    return (out, state_out) if (return_state or state_out is not None) else out


def gated_retention_chunkwise_fwd(q, k, v, g, chunk, state_in=None, return_state=False, out=None,
                                  state_out=None, stream=None, workspace=None):
    """Gated chunkwise retention forward with per-token log-decays g[B,H,N] (fp32, <= 0)."""
    return _chunk_call("gated_retention_chunkwise_fwd", q, k, v, g, chunk, state_in, return_state, out,
                       state_out, stream, workspace, True)


def _parallel_call_impl(fn_name, q, k, v, decay, out, stream, gated):
    torch = _torch()
    L = lib()
    _require(q, "q")
    dev = q.device
    _require(k, "k", q.dtype, dev)
    _require(v, "v", q.dtype, dev)
    _require(decay, "g" if gated else "gamma", torch.float32, dev)
    if q.dim() != 4 or k.shape != q.shape or v.dim() != 4 or v.shape[:3] != q.shape[:3]:
        raise ValueError(f"expected q,k [B,H,N,dk] and v [B,H,N,dv]; got {tuple(q.shape)} "
                         f"{tuple(k.shape)} {tuple(v.shape)}")
    B, H, N, dk = q.shape
    dv = v.shape[-1]
    exp_decay = (B, H, N) if gated else (H,)
    if tuple(decay.shape) != exp_decay:
        raise ValueError(f"decay must have shape {exp_decay}, got {tuple(decay.shape)}")
    if out is None:
        out = torch.empty((B, H, N, dv), dtype=q.dtype, device=dev)
    else:
        _require(out, "out", q.dtype, dev)
        if tuple(out.shape) != (B, H, N, dv):
            raise ValueError("out must be [B,H,N,dv]")
    st = getattr(L, fn_name)(_ptr(q), _ptr(k), _ptr(v), _ptr(decay), _ptr(out), B, H, N, dk, dv, _dtype_code(q),
                             _stream(stream))
    _check(st, fn_name)
    return out


def _parallel_call(fn_name, q, k, v, decay, out, stream, gated):
    with _on_stream(stream):
        return _parallel_call_impl(fn_name, q, k, v, decay, out, stream, gated)


def retention_parallel_fwd(q, k, v, gamma, out=None, stream=None):
    """Parallel-form retention forward O = (Q K^T (.) D) V (no state); shapes as the chunkwise form."""
    return _parallel_call("retention_parallel_fwd", q, k, v, gamma, out, stream, False)


def gated_retention_parallel_fwd(q, k, v, g, out=None, stream=None):
    """Gated parallel-form forward with per-token log-decays g[B,H,N] (fp32, <= 0)."""
    return _parallel_call("gated_retention_parallel_fwd", q, k, v, g, out, stream, True)


def msr_workspace_bytes(B, N, D, H, dk, dv, chunk) -> int:
    return int(lib().gated_msr_workspace_bytes(B, N, D, H, dk, dv, chunk))


def gated_msr_fwd(x, wq, wk, wv, wg, wgt, wo, H, dk, dv, chunk=64, rope_base=10000.0, norm_eps=1e-5, out=None,
                  workspace=None, stream=None):
    """Gated multi-scale retention layer on x [B,N,D] (bf16): projections (weights [out, in],
    bf16), interleaved rotary rotation of q and k, k / sqrt(dk), decay logsigmoid(gt)/16,
    gated chunkwise retention, per-head RMSNorm, silu gate, output projection.  Returns y
    [B,N,D] bf16."""
    with _on_stream(stream):
        return _gated_msr_fwd_impl(x, wq, wk, wv, wg, wgt, wo, H, dk, dv, chunk, rope_base, norm_eps, out, workspace,
                                   stream)


def _gated_msr_fwd_impl(x, wq, wk, wv, wg, wgt, wo, H, dk, dv, chunk, rope_base, norm_eps, out, workspace, stream):
    torch = _torch()
    L = lib()
    _require(x, "x", torch.bfloat16)
    dev = x.device
    if x.dim() != 3:
        raise ValueError("x must be [B,N,D]")
    B, N, D = x.shape
    shapes = {"wq": (H * dk, D), "wk": (H * dk, D), "wv": (H * dv, D), "wg": (H * dv, D), "wgt": (H, D),
              "wo": (D, H * dv)}
    ws_ = {"wq": wq, "wk": wk, "wv": wv, "wg": wg, "wgt": wgt, "wo": wo}
    for name, t in ws_.items():
        _require(t, name, torch.bfloat16, dev)
        if tuple(t.shape) != shapes[name]:
            raise ValueError(f"{name} must be {shapes[name]}, got {tuple(t.shape)}")
    if out is None:
        out = torch.empty((B, N, D), dtype=torch.bfloat16, device=dev)
    else:
        _require(out, "out", torch.bfloat16, dev)
        if tuple(out.shape) != (B, N, D):
            raise ValueError("out must be [B,N,D]")
    need = msr_workspace_bytes(B, N, D, H, dk, dv, chunk)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = L.gated_msr_fwd(_ptr(x), _ptr(wq), _ptr(wk), _ptr(wv), _ptr(wg), _ptr(wgt), _ptr(wo), _ptr(out), B, N, D,
                         H, dk, dv, int(chunk), float(rope_base), float(norm_eps), _ptr(workspace), ws_bytes,
                         _stream(stream))
    _check(st, "gated_msr_fwd")
    return out


def bwd_workspace_bytes(B, H, N, dk, dv, chunk, dtype_code, gated) -> int:
    return int(lib().retention_bwd_workspace_bytes(B, H, N, dk, dv, chunk, dtype_code, 1 if gated else 0))


def _bwd_call_impl(q, k, v, decay, grad_o, chunk, state_in, grad_state_out, return_grad_state_in, stream,
              workspace, gated):
    torch = _torch()
    L = lib()
    _require(q, "q")
    dev = q.device
    _require(k, "k", q.dtype, dev)
    _require(v, "v", q.dtype, dev)
    _require(grad_o, "grad_o", q.dtype, dev)
    _require(decay, "g" if gated else "gamma", torch.float32, dev)
    if q.dim() != 4 or k.shape != q.shape or v.dim() != 4 or v.shape[:3] != q.shape[:3]:
        raise ValueError(f"expected q,k [B,H,N,dk] and v [B,H,N,dv]; got {tuple(q.shape)} "
                         f"{tuple(k.shape)} {tuple(v.shape)}")
    B, H, N, dk = q.shape
    dv = v.shape[-1]
    if tuple(grad_o.shape) != (B, H, N, dv):
        raise ValueError("grad_o must be [B,H,N,dv]")
    exp_decay = (B, H, N) if gated else (H,)
    if tuple(decay.shape) != exp_decay:
        raise ValueError(f"decay must have shape {exp_decay}, got {tuple(decay.shape)}")
    for name, t in (("state_in", state_in), ("grad_state_out", grad_state_out)):
        if t is not None:
            _require(t, name, torch.float32, dev)
            if tuple(t.shape) != (B, H, dk, dv):
                raise ValueError(f"{name} must be [B,H,dk,dv]")
    gq = torch.empty_like(q)
    gk = torch.empty_like(k)
    gv = torch.empty_like(v)
    gg = torch.empty((B, H, N), dtype=torch.float32, device=dev) if gated else None
    gs = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev) if return_grad_state_in else None
    code = _dtype_code(q)
    ws_need = bwd_workspace_bytes(B, H, N, dk, dv, chunk, code, gated)
    if workspace is None and ws_need > 0:
        workspace = torch.empty(ws_need, dtype=torch.uint8, device=dev)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if gated:
        st = L.gated_retention_chunkwise_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(decay), _ptr(state_in), _ptr(grad_o),
                                             _ptr(grad_state_out), _ptr(gq), _ptr(gk), _ptr(gv), _ptr(gg), _ptr(gs),
                                             B, H, N, dk, dv, int(chunk), code, _ptr(workspace), ws_bytes,
                                             _stream(stream))
        _check(st, "gated_retention_chunkwise_bwd")
        return (gq, gk, gv, gg, gs) if return_grad_state_in else (gq, gk, gv, gg)
    st = L.retention_chunkwise_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(decay), _ptr(state_in), _ptr(grad_o),
                                   _ptr(grad_state_out), _ptr(gq), _ptr(gk), _ptr(gv), _ptr(gs), B, H, N, dk, dv,
                                   int(chunk), code, _ptr(workspace), ws_bytes, _stream(stream))
    _check(st, "retention_chunkwise_bwd")
    return (gq, gk, gv, gs) if return_grad_state_in else (gq, gk, gv)


def _bwd_call(q, k, v, decay, grad_o, chunk, state_in, grad_state_out, return_grad_state_in, stream, workspace,
              gated):
    with _on_stream(stream):
        return _bwd_call_impl(q, k, v, decay, grad_o, chunk, state_in, grad_state_out, return_grad_state_in, stream,
                              workspace, gated)


def retention_chunkwise_bwd(q, k, v, gamma, grad_o, chunk, state_in=None, grad_state_out=None,
                            return_grad_state_in=False, stream=None, workspace=None):
    """Backward of retention_chunkwise_fwd for L = <grad_o, o> + <grad_state_out, state_out>.

    Returns (grad_q, grad_k, grad_v), plus grad_state_in [B,H,dk,dv] fp32 when
    return_grad_state_in is set.
    """
    return _bwd_call(q, k, v, gamma, grad_o, chunk, state_in, grad_state_out, return_grad_state_in, stream,
                     workspace, False)


def gated_retention_chunkwise_bwd(q, k, v, g, grad_o, chunk, state_in=None, grad_state_out=None,
                                  return_grad_state_in=False, stream=None, workspace=None):
    """Backward of gated_retention_chunkwise_fwd: (grad_q, grad_k, grad_v, grad_g[, grad_state_in])."""
    return _bwd_call(q, k, v, g, grad_o, chunk, state_in, grad_state_out, return_grad_state_in, stream,
                     workspace, True)


def _decode_call_impl(fn_name, q, k, v, decay, state, out, stream, gated):
    torch = _torch()
    L = lib()
    _require(q, "q")
    dev = q.device
    _require(k, "k", q.dtype, dev)
    _require(v, "v", q.dtype, dev)
    _require(decay, "g" if gated else "gamma", torch.float32, dev)
    _require(state, "state", torch.float32, dev)
    if q.dim() != 3 or k.shape != q.shape or v.dim() != 3 or v.shape[:2] != q.shape[:2]:
        raise ValueError("expected q,k [B,H,dk] and v [B,H,dv]")
    B, H, dk = q.shape
    dv = v.shape[-1]
    if tuple(decay.shape) != ((B, H) if gated else (H,)):
        raise ValueError("decay has the wrong shape")
    if tuple(state.shape) != (B, H, dk, dv):
        raise ValueError("state must be [B,H,dk,dv]")
    if out is None:
        out = torch.empty((B, H, dv), dtype=q.dtype, device=dev)
    else:
        _require(out, "out", q.dtype, dev)
        if tuple(out.shape) != (B, H, dv):
            raise ValueError(f"out must be [B,H,dv] = {(B, H, dv)}, got {tuple(out.shape)}")
    st = getattr(L, fn_name)(_ptr(q), _ptr(k), _ptr(v), _ptr(decay), _ptr(state), _ptr(out), B, H, dk,
                             dv, _dtype_code(q), _stream(stream))
    _check(st, fn_name)
    return out


def _decode_call(fn_name, q, k, v, decay, state, out, stream, gated):
    with _on_stream(stream):
        return _decode_call_impl(fn_name, q, k, v, decay, state, out, stream, gated)


def retention_decode_step(q, k, v, gamma, state, out=None, stream=None):
    """One decode step: state <- gamma state + k^T v (in place, fp32), returns o = q state."""
    return _decode_call("retention_decode_step", q, k, v, gamma, state, out, stream, False)


def gated_retention_decode_step(q, k, v, g, state, out=None, stream=None):
    """One gated decode step with log-decay g[B,H]: state <- exp(g) state + k^T v, o = q state."""
    return _decode_call("gated_retention_decode_step", q, k, v, g, state, out, stream, True)


def profile_enable(on: bool = True) -> None:
    """Start (or stop) timing every kernel launch with HIP events on its stream."""
    _check(lib().retention_profile_enable(1 if on else 0), "retention_profile_enable")


def profile_read() -> dict:
    """Wait for the recorded launches; per kernel kind the summed milliseconds and the
    number of launches since the last read-out (plus the count of dropped launches)."""
    n = len(PROFILE_KINDS)
    ms = (ctypes.c_double * n)()
    cnt = (ctypes.c_int * n)()
    dropped = ctypes.c_int(0)
    _check(lib().retention_profile_read(ctypes.cast(ms, _vp), ctypes.cast(cnt, _vp), n,
                                        ctypes.byref(dropped)), "retention_profile_read")
    out = {k: {"ms": ms[i], "launches": cnt[i]} for i, k in enumerate(PROFILE_KINDS)}
    out["dropped"] = dropped.value
    return out


def calib_mfma(blocks: int, waves: int, iters: int, out=None, stream=None) -> float:
    """Launch the matrix-core loop reference (see retention_calib_mfma); returns the flops
    it performs.  The caller times it."""
    torch = _torch()
    if out is None:
        out = torch.empty(blocks * waves, dtype=torch.float32, device="cuda")
    _check(lib().retention_calib_mfma(_ptr(out), blocks, waves, iters, _stream(stream)), "retention_calib_mfma")
    return float(lib().retention_calib_mfma_flops(blocks, waves, iters))
