"""fp64 CPU oracle of the gated multi-scale retention layer (the mixer around the operator).

TEST INFRASTRUCTURE ONLY, like the rest of this package: only the test suite,
``__graft_entry__.smoke()`` and ``bench.py``'s CPU-baseline leg may import it, and it
imports nothing from the GPU library.

Source: "unilm RetNet 技术指南 ... YOCO 中 Gated RetNet 的源码解析" (pwwt.cn).  Section
GateRetention 模块的内部结构 gives the parts: five bias-free projections (q, k, v, the
SwiGLU-style gate g, and a per-head scalar gate gt), an interleaved rotary position
rotation of q and k, the log-domain gate logsigmoid(gt)/16, a per-head RMSNorm without
affine parameters over the head dimension ("subln"), and an output projection.  Section
三种计算路径与增量状态 scales k by d_k^-1/2 and gives the retention recurrence (the
operator oracle in retention_oracle.py).

Readings where the page is silent (also listed in the design notes):

* The rotation pairs adjacent elements (2i, 2i+1) of each head and turns pair i of token
  n by the angle n * base^(-2i/d_k), with base a parameter (10000 by default), the usual
  rotary schedule; positions start at 0.
* The gate is applied as silu(g) * RMSNorm(o), the SwiGLU-style product the page names,
  and the output projection follows.
* RMSNorm(x) = x / sqrt(mean(x^2) + eps), with eps a parameter (1e-5 by default, the
  value the page names for the layer norms).
* Weights are stored [out_features, in_features]: y = x W^T.
* Precision: the layer's definition is fp64 throughout.  An implementation with bf16
  activations rounds the rotated (and scaled) q and k, v, the gate projection, the gated
  product and the output; ``act`` applies such a rounding at exactly those points (None:
  none).  The
  output after RMSNorm is ill-conditioned where q.k nearly cancels (token 0's output is
  (q.k) v / sqrt((q.k)^2 mean(v^2) + eps)), so bf16 operands can move it by more than
  their own rounding there; the GPU comparison therefore names the rounding points.
"""
from __future__ import annotations

import numpy as np

from .retention_oracle import gated_retention_recurrent

__all__ = ["rope_interleaved", "rms_norm", "silu", "logsigmoid", "gated_msr_forward"]


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def rope_interleaved(x, base=10000.0):
    """Rotate adjacent pairs of the last axis: x [..., N, d] with token index on axis -2.
    Pair i = (x[..., 2i], x[..., 2i+1]) of token n turns by n * base^(-2i/d)."""
    x = _f64(x)
    N, d = x.shape[-2], x.shape[-1]
    i = np.arange(d // 2, dtype=np.float64)
    ang = np.arange(N, dtype=np.float64)[:, None] * base ** (-2.0 * i / d)[None, :]   # [N, d/2]
    c, s = np.cos(ang), np.sin(ang)
    x0, x1 = x[..., 0::2], x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = x0 * c - x1 * s
    out[..., 1::2] = x0 * s + x1 * c
    return out


def rms_norm(x, eps):
    """x / sqrt(mean(x^2) + eps) over the last axis (no affine parameters)."""
    x = _f64(x)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)


def silu(x):
    """x * sigmoid(x)."""
    x = _f64(x)
    return x / (1.0 + np.exp(-x))


def logsigmoid(x):
    """log(sigmoid(x)), computed as min(x, 0) - log1p(exp(-|x|))."""
    x = _f64(x)
    return np.minimum(x, 0.0) - np.log1p(np.exp(-np.abs(x)))


def gated_msr_forward(x, wq, wk, wv, wg, wgt, wo, H, dk, dv, rope_base=10000.0, eps=1e-5,
                      gate_norm=16.0, act=None):
    """The gated multi-scale retention layer on x [B, N, D]; weights [out, in].

    act: optional rounding of the stored activations (see the module notes).
    Returns y [B, N, D] and the intermediate decay g [B, H, N] (log-domain, <= 0)."""
    x = _f64(x)
    r = (lambda t: t) if act is None else (lambda t: _f64(act(t)))  # noqa: E731
    B, N, D = x.shape
    proj = lambda w: x @ _f64(w).T  # noqa: E731
    heads = lambda t, d: t.reshape(B, N, H, d).transpose(0, 2, 1, 3)  # noqa: E731  [B,H,N,d]
    q = r(rope_interleaved(heads(proj(wq), dk), rope_base))
    k = r(rope_interleaved(heads(proj(wk), dk), rope_base) / np.sqrt(dk))
    v = heads(r(proj(wv)), dv)
    g = logsigmoid(proj(wgt)).transpose(0, 2, 1) / gate_norm                    # [B,H,N]
    o, _ = gated_retention_recurrent(q, k, v, g)                                # [B,H,N,dv]
    o = rms_norm(o, eps).transpose(0, 2, 1, 3).reshape(B, N, H * dv)
    z = r(silu(r(proj(wg))) * o)
    return r(z @ _f64(wo).T), g
