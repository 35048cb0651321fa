"""Seeded synthetic inputs for the retention operator.

This module draws random numbers and casts them; it holds none of the operator's
arithmetic.  Both the GPU tests/benchmark and the CPU oracle take their inputs from
here, so the two sides see bit-identical values.

Recipe (one numpy PCG64 generator per workload, seeded with the workload's seed):
  * draw float64 standard normals in C order, in the sequence Q, K, V, then extras;
  * scale Q, K, V by 1/sqrt(d_k);
  * cast to float32, then (for bf16 workloads) to bfloat16 with round-to-nearest-even;
  * the returned float64 copies are the exact values of the cast tensors.

Workloads (sizes as named; the decay sets are the per-head gammas of each workload):
  tiny_f32         B=1 H=2 N=64 dk=dv=16 chunk=16, fp32, gamma = {0.9, 0.99}
  train_bf16       B=4 H=8 N=2048 dk=256 dv=512 chunk=64, gamma_h = 1 - 2^(-5-h)
  long_bf16        B=1 H=16 N=16384 dk=dv=128 chunk=512 (128, 256 swept),
                   gamma_h = 1 - 2^(-5 - 7h/15)
  decode_bf16      batch=128 H=32 dk=dv=128, fp32 state S0 ~ N(0, 0.1^2), 1024 steps of
                   fresh q,k,v, gamma_h = 1 - 2^(-5 - 7h/31)
  gated_bf16       B=2 H=16 N=8192 dk=dv=128 chunk=64, g = logsigmoid(x)/16, x ~ N(0,1)
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

try:  # torch is only needed for the bf16 cast
    import torch
except ImportError:  # pragma: no cover
    torch = None


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    kind: str            # "chunkwise" | "gated" | "decode"
    dtype: str           # "f32" | "bf16"
    B: int
    H: int
    N: int               # sequence length (decode: number of steps)
    dk: int
    dv: int
    chunk: int           # chunk size (0 for decode)
    seed: int
    sweep_chunks: tuple = ()

    @property
    def tokens(self) -> int:
        return self.B * self.N


WORKLOADS = {
    "tiny_f32": Workload("tiny_f32", "chunkwise", "f32", 1, 2, 64, 16, 16, 16, 1),
    "train_bf16": Workload("train_bf16", "chunkwise", "bf16", 4, 8, 2048, 256, 512, 64, 2),
    "long_bf16": Workload("long_bf16", "chunkwise", "bf16", 1, 16, 16384, 128, 128, 512, 3,
                          sweep_chunks=(128, 256, 512)),
    "decode_bf16": Workload("decode_bf16", "decode", "bf16", 128, 32, 1024, 128, 128, 0, 4),
    "gated_bf16": Workload("gated_bf16", "gated", "bf16", 2, 16, 8192, 128, 128, 64, 5),
}


def gammas(name: str, H: int) -> np.ndarray:
    """Per-head decay set of a workload, as float32."""
    h = np.arange(H, dtype=np.float64)
    if name == "tiny_f32":
        g = np.array([0.9, 0.99][:H], dtype=np.float64)
    elif name == "train_bf16":
        g = 1.0 - 2.0 ** (-5.0 - h)
    elif name == "long_bf16":
        g = 1.0 - 2.0 ** (-5.0 - h * 7.0 / 15.0)
    elif name == "decode_bf16":
        g = 1.0 - 2.0 ** (-5.0 - h * 7.0 / 31.0)
    else:
        raise KeyError(name)
    return g.astype(np.float32)


def to_dtype(x: np.ndarray, dtype: str):
    """Cast float64 -> float32 -> (bf16, RNE).  Returns (torch CPU tensor, exact f64 copy)."""
    x32 = np.ascontiguousarray(x, dtype=np.float32)
    t = torch.from_numpy(x32)
    if dtype == "bf16":
        t = t.to(torch.bfloat16)
    elif dtype != "f32":
        raise ValueError(dtype)
    return t, t.to(torch.float64).numpy()


def logsigmoid(x: np.ndarray) -> np.ndarray:
    """Numerically stable log(1/(1+exp(-x))) in float64."""
    x = np.asarray(x, dtype=np.float64)
    return np.where(x >= 0, -np.log1p(np.exp(-x)), x - np.log1p(np.exp(x)))


def qkv(rng: np.random.Generator, B, H, N, dk, dv, dtype):
    """Q, K, V ~ N(0,1)/sqrt(dk), drawn in that order.  Returns dict of (tensor, f64)."""
    s = 1.0 / math.sqrt(dk)
    out = {}
    for nm, d in (("q", dk), ("k", dk), ("v", dv)):
        out[nm] = to_dtype(rng.standard_normal((B, H, N, d)) * s, dtype)
    return out


def make_chunkwise(w: Workload, *, B=None, H=None, N=None, seed=None, state_in=False):
    """Inputs for a chunkwise or gated workload, optionally with smaller B/H/N.

    Returns dict name -> (torch CPU tensor, float64 numpy).  Keys: q, k, v, and either
    gamma [H] (fp32) or g [B,H,N] (fp32); plus state_in [B,H,dk,dv] fp32 if requested
    (drawn after the decay inputs, ~ N(0, 0.1^2)).
    """
    B = w.B if B is None else B
    H = w.H if H is None else H
    N = w.N if N is None else N
    rng = np.random.default_rng(w.seed if seed is None else seed)
    out = qkv(rng, B, H, N, w.dk, w.dv, w.dtype)
    if w.kind == "gated":
        x = rng.standard_normal((B, H, N))
        out["g"] = to_dtype(logsigmoid(x) / 16.0, "f32")
    else:
        if w.name in ("train_bf16", "long_bf16", "tiny_f32") and H <= w.H:
            gm = gammas(w.name, w.H)[:H]
        else:
            gm = gammas("long_bf16", 16)[np.arange(H) % 16]
        out["gamma"] = to_dtype(gm.astype(np.float64), "f32")
    if state_in:
        out["state_in"] = to_dtype(rng.standard_normal((B, H, w.dk, w.dv)) * 0.1, "f32")
    return out


def make_decode(w: Workload, *, B=None, steps=None, seed=None):
    """Decode workload: S0 ~ N(0, 0.1^2) fp32 [B,H,dk,dv], then per-step q,k,v.

    Drawing order: S0, then for each step t: q_t [B,H,dk], k_t [B,H,dk], v_t [B,H,dv].
    Returns dict: state0 (tensor, f64); q, k, v as torch CPU tensors [steps,B,H,d] in the
    workload dtype (no float64 copies: at full size they would take ~13 GB; take rows
    with ``.to(torch.float64)`` where the oracle needs them); gamma (tensor, f64).
    """
    B = w.B if B is None else B
    steps = w.N if steps is None else steps
    rng = np.random.default_rng(w.seed if seed is None else seed)
    out = {"state0": to_dtype(rng.standard_normal((B, w.H, w.dk, w.dv)) * 0.1, "f32")}
    s = 1.0 / math.sqrt(w.dk)
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    bufs = {nm: torch.empty((steps, B, w.H, d), dtype=tdt) for nm, d in (("q", w.dk), ("k", w.dk), ("v", w.dv))}
    for t in range(steps):
        for nm, d in (("q", w.dk), ("k", w.dk), ("v", w.dv)):
            bufs[nm][t] = to_dtype(rng.standard_normal((B, w.H, d)) * s, w.dtype)[0]
    out.update(bufs)
    out["gamma"] = to_dtype(gammas("decode_bf16", w.H).astype(np.float64), "f32")
    return out


def decode_log_decays(seed, steps, B, H):
    """Per-step log-decays of a gated decode run: g_t = logsigmoid(x_t)/16 with
    x_t ~ N(0,1) [B,H], from a generator of its own seed, drawn step by step.  Returns
    (torch CPU tensor [steps,B,H] fp32, float64 copy)."""
    rng = np.random.default_rng(seed)
    return to_dtype(logsigmoid(rng.standard_normal((steps, B, H))) / 16.0, "f32")


def random_case(seed, B, H, N, dk, dv, dtype="bf16", gated=False, state_in=False,
                gamma_lo=0.8):
    """Generic seeded case for tests: Q,K,V ~ N(0,1)/sqrt(dk); gamma ~ U(gamma_lo, 1)
    per head, or g = logsigmoid(x)/16 per token."""
    rng = np.random.default_rng(seed)
    out = qkv(rng, B, H, N, dk, dv, dtype)
    if gated:
        out["g"] = to_dtype(logsigmoid(rng.standard_normal((B, H, N))) / 16.0, "f32")
    else:
        out["gamma"] = to_dtype(rng.uniform(gamma_lo, 1.0, size=H), "f32")
    if state_in:
        out["state_in"] = to_dtype(rng.standard_normal((B, H, dk, dv)) * 0.1, "f32")
    return out


def backward_grads(seed, B, H, N, dk, dv, dtype="bf16", state=False):
    """Upstream gradients for backward tests: grad_o ~ N(0,1) [B,H,N,dv] in the workload
    dtype, then (if state) grad_state_out ~ N(0, 0.1^2) [B,H,dk,dv] fp32.  Own generator
    (seed), drawn in that order; returns dict name -> (torch CPU tensor, float64)."""
    rng = np.random.default_rng(seed)
    out = {"grad_o": to_dtype(rng.standard_normal((B, H, N, dv)), dtype)}
    if state:
        out["grad_state_out"] = to_dtype(rng.standard_normal((B, H, dk, dv)) * 0.1, "f32")
    return out


def msr_case(seed, B, N, D, H, dk, dv):
    """Gated retention layer: x ~ N(0,1) [B,N,D], then the weights Wq, Wk [H*dk, D],
    Wv, Wg [H*dv, D], Wgt [H, D] and Wo [D, H*dv] ~ N(0, 1/D) (random init of the
    [out, in] layout), all drawn in that order from one generator and rounded to bf16.
    Returns dict name -> (torch CPU tensor, float64)."""
    rng = np.random.default_rng(seed)
    s = 1.0 / np.sqrt(D)
    out = {"x": to_dtype(rng.standard_normal((B, N, D)), "bf16")}
    for name, shape in (("wq", (H * dk, D)), ("wk", (H * dk, D)), ("wv", (H * dv, D)), ("wg", (H * dv, D)),
                        ("wgt", (H, D)), ("wo", (D, H * dv))):
        out[name] = to_dtype(rng.standard_normal(shape) * s, "bf16")
    return out
