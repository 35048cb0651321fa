"""fp64 CPU oracle for the retention operator.

TEST INFRASTRUCTURE ONLY.  Only the test suite, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  The GPU library never
imports, links or calls it, and it imports nothing from the GPU library.

Everything is plain numpy in float64.  Inputs of any float dtype are promoted to
float64 exactly (bf16 and fp32 values are representable in fp64), so the oracle sees
the very values the GPU sees and only the GPU's own arithmetic error is measured.

Sources (web pages on RetNet; cited by page title and section):

* "RetNet retention mechanism" tutorial (aiqz.cc), section 递归推理 (recurrent
  inference): the state update S_n = gamma * S_{n-1} + K_n^T V_n and the read-out
  R_n = Q_n S_n.  This is the definition the oracle of record follows.
* Same page, section 保留机制初识: R_n = sum_{m<=n} gamma^(n-m) (Q_n K_m^T) V_m,
  section 衰减矩阵: D_nm = gamma^(n-m) for n >= m and 0 otherwise, and section
  并行训练: R = (Q K^T (.) D) V.  These give the parallel cross-check form.
* Same page, section 块级循环 (chunk-level recurrence): inside a chunk the parallel
  form, across chunks the state relay.  The page writes a single factor gamma^c on
  the cross-chunk query term; only a per-row factor gamma^(j+1) (j = 0-based row in
  the chunk) agrees with the recurrent and parallel forms that every page calls
  equivalent, so the chunkwise cross-check uses the per-row factor.
* "Retentive Network (RetNet) 详解" (171host.com), section 3.1: the same three forms
  (recurrent, parallel, chunkwise recurrent) and their equivalence.
* "unilm RetNet 技术指南 ... YOCO 中 Gated RetNet 的源码解析" (pwwt.cn), sections
  GateRetention 模块的内部结构 and 三种计算路径与增量状态: the gated variant uses a
  per-token, per-head log-decay g (a logsigmoid divided by 16), all decays are
  exp of differences of cumsum(g), and the one-token path adds k^T v to the previous
  state scaled by the decay.  Section Triton 内核与自校验测试: cross-chunk weights
  exp(g_last - g_l) and the intra-chunk mask g_n - g_m.

Readings taken where the pages are silent (each also listed with its reason in the
design notes):

* The output of token n uses the state AFTER token n was added (R_n = Q_n S_n with the
  updated S_n), so the diagonal of D is 1.
* Gated: the state is first multiplied by exp(g_n), then k_n^T v_n is added; the
  cumulative sum G is inclusive, so the weight of token m in output n >= m is
  exp(G_n - G_m) and the initial state reaches output n with weight exp(G_n).
* An optional initial state S0 is decayed like any state at the first step.
* No key scaling and no normalisation inside the operator.
* d_k may differ from d_v; S has shape d_k x d_v.
* Backward: the pages name a backward recurrence for the chunked kernels and check its
  gradients against a naive loop ("unilm RetNet 技术指南", section Triton 内核与自校验
  测试) but print no formula.  The oracle applies the chain rule to the recurrence of
  record (the adjoint recurrence below); the tests pin it to central finite
  differences of the forward oracle.  The loss whose gradients are returned is
  L = <dO, o> + <dS, S_N>.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "retention_recurrent",
    "gated_retention_recurrent",
    "retention_parallel",
    "gated_retention_parallel",
    "retention_chunkwise",
    "gated_retention_chunkwise",
    "retention_decode_step",
    "gated_retention_decode_step",
    "retention_recurrent_bwd",
    "gated_retention_recurrent_bwd",
]


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def _check_qkv(q, k, v):
    q, k, v = _f64(q), _f64(k), _f64(v)
    if q.ndim != 4 or k.shape != q.shape or v.ndim != 4 or v.shape[:3] != q.shape[:3]:
        raise ValueError(f"expected q,k [B,H,N,dk] and v [B,H,N,dv]; got {q.shape} {k.shape} {v.shape}")
    return q, k, v


def _initial_state(state_in, B, H, dk, dv):
    if state_in is None:
        return np.zeros((B, H, dk, dv), dtype=np.float64)
    s = _f64(state_in).copy()
    if s.shape != (B, H, dk, dv):
        raise ValueError(f"state_in must be [B,H,dk,dv]={B,H,dk,dv}; got {s.shape}")
    return s


# ---------------------------------------------------------------------------------
# Recurrent form: the oracle of record.
# ---------------------------------------------------------------------------------

def _recurrence(q, k, v, lam, state_in):
    """Token-by-token recurrence with a per-token multiplicative decay lam[B,H,N].

    For every (b, h) and n = 0..N-1:  S <- lam[n] * S + outer(k_n, v_n);  o_n = q_n . S
    ("RetNet retention mechanism" tutorial, section 递归推理).  Vectorised over (b, h);
    the loop over n is the definition itself.
    """
    B, H, N, dk = q.shape
    dv = v.shape[-1]
    S = _initial_state(state_in, B, H, dk, dv)
    o = np.zeros((B, H, N, dv), dtype=np.float64)
    for n in range(N):
        S *= lam[:, :, n, None, None]
        S += k[:, :, n, :, None] * v[:, :, n, None, :]
        o[:, :, n, :] = np.einsum("bhi,bhij->bhj", q[:, :, n, :], S)
    return o, S


def retention_recurrent(q, k, v, gamma, state_in=None):
    """Per-head-decay retention, recurrent form.

    q, k: [B,H,N,dk]; v: [B,H,N,dv]; gamma: [H] with each gamma in (0, 1];
    state_in: optional [B,H,dk,dv] (zeros when None).
    Returns (o [B,H,N,dv], state_out [B,H,dk,dv]) in float64.
    """
    q, k, v = _check_qkv(q, k, v)
    B, H, N, _ = q.shape
    gamma = _f64(gamma).reshape(H)
    lam = np.broadcast_to(gamma[None, :, None], (B, H, N))
    return _recurrence(q, k, v, lam, state_in)


def gated_retention_recurrent(q, k, v, g, state_in=None):
    """Gated retention (per-token, per-head log-decay g[B,H,N], g <= 0), recurrent form.

    The per-step multiplier is exp(g_n): the gate is a log-decay, so the previous
    state is scaled by exp(g_n) before k_n^T v_n is added ("unilm RetNet 技术指南",
    sections GateRetention 模块的内部结构 and 三种计算路径与增量状态).
    """
    q, k, v = _check_qkv(q, k, v)
    B, H, N, _ = q.shape
    g = _f64(g)
    if g.shape != (B, H, N):
        raise ValueError(f"g must be [B,H,N]={B,H,N}; got {g.shape}")
    return _recurrence(q, k, v, np.exp(g), state_in)


def retention_decode_step(q, k, v, gamma, state):
    """One recurrent decode step: S <- gamma_h S + k^T v, then o = q S (updated S).

    q, k: [B,H,dk]; v: [B,H,dv]; gamma: [H]; state: [B,H,dk,dv].
    Returns (o [B,H,dv], new_state [B,H,dk,dv]); the input state is not modified.
    ("RetNet retention mechanism" tutorial, section 递归推理.)
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    S = _f64(state).copy()
    H = q.shape[1]
    S *= _f64(gamma).reshape(1, H, 1, 1)
    S += k[..., :, None] * v[..., None, :]
    o = np.einsum("bhi,bhij->bhj", q, S)
    return o, S


def gated_retention_decode_step(q, k, v, g, state):
    """One gated decode step with log-decay g[B,H]: S <- exp(g) S + k^T v, o = q S."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    S = _f64(state).copy()
    S *= np.exp(_f64(g))[..., None, None]
    S += k[..., :, None] * v[..., None, :]
    o = np.einsum("bhi,bhij->bhj", q, S)
    return o, S


# ---------------------------------------------------------------------------------
# Decay weights.  Per-head: powers of gamma (the decay matrix D_nm = gamma^(n-m) of the
# tutorial's section 衰减矩阵).  Gated: exp of differences of the inclusive cumsum G.
# Each returns, for positions a (rows) and b (columns) of one segment [p0, p1):
#   W[.., a, b] = prod_{b<t<=a} lam_t for a >= b, 0 above the diagonal;
#   Gam[.., a]  = prod_{p0<=t<=a} lam_t  (weight of the segment's incoming state).
# ---------------------------------------------------------------------------------

def _weights_gamma(gamma, B, p0, p1):
    L = p1 - p0
    idx = np.arange(L)
    expo = idx[:, None] - idx[None, :]
    causal = expo >= 0
    gm = gamma[None, :, None, None]                                  # [1,H,1,1]
    W = np.where(causal, gm ** np.where(causal, expo, 0), 0.0)       # [1,H,L,L]
    Gam = gamma[None, :, None] ** (idx[None, None, :] + 1)           # [1,H,L]
    H = gamma.shape[0]
    return np.broadcast_to(W, (B, H, L, L)), np.broadcast_to(Gam, (B, H, L))


def _weights_gated(g, p0, p1):
    G = np.cumsum(g[:, :, p0:p1], axis=-1)                           # inclusive, segment-local
    L = p1 - p0
    causal = np.tril(np.ones((L, L), dtype=bool))
    diff = G[:, :, :, None] - G[:, :, None, :]
    # select before exp: the masked (upper) entries would be exp of a positive number
    W = np.where(causal, np.exp(np.where(causal, diff, 0.0)), 0.0)
    return W, np.exp(G)


# ---------------------------------------------------------------------------------
# Parallel form (cross-check): R = (Q K^T (.) D) V, plus the initial state's share.
# ---------------------------------------------------------------------------------

def _parallel(q, k, v, W, Gam, state_in):
    """o = (Q K^T (.) W) V + diag(Gam) Q S0;  S_N = Gam_{N-1} S0 + sum_m W[N-1, m] k_m^T v_m."""
    B, H, N, dk = q.shape
    dv = v.shape[-1]
    S0 = _initial_state(state_in, B, H, dk, dv)
    scores = np.einsum("bhnd,bhmd->bhnm", q, k) * W
    o = np.einsum("bhnm,bhmv->bhnv", scores, v)
    o = o + Gam[..., None] * np.einsum("bhnd,bhdv->bhnv", q, S0)
    if N == 0:
        return o, S0
    S = np.einsum("bhm,bhmd,bhmv->bhdv", W[:, :, -1, :], k, v)
    S = S + Gam[:, :, -1, None, None] * S0
    return o, S


def retention_parallel(q, k, v, gamma, state_in=None):
    """Parallel form (QK^T (.) D) V with D_nm = gamma^(n-m), n >= m ("RetNet retention
    mechanism" tutorial, sections 衰减矩阵 and 并行训练); the initial state reaches
    output n with weight gamma^(n+1)."""
    q, k, v = _check_qkv(q, k, v)
    B, H, N, _ = q.shape
    W, Gam = _weights_gamma(_f64(gamma).reshape(H), B, 0, N)
    return _parallel(q, k, v, W, Gam, state_in)


def gated_retention_parallel(q, k, v, g, state_in=None):
    """Gated parallel form: D_nm = exp(G_n - G_m) for n >= m, G = inclusive cumsum(g)
    ("unilm RetNet 技术指南", section 三种计算路径与增量状态: the mask g_n - g_m plus a
    causal mask, exponentiated)."""
    q, k, v = _check_qkv(q, k, v)
    W, Gam = _weights_gated(_f64(g), 0, q.shape[2])
    return _parallel(q, k, v, W, Gam, state_in)


# ---------------------------------------------------------------------------------
# Chunkwise-recurrent form (cross-check): parallel inside a chunk, recurrence across.
# ---------------------------------------------------------------------------------

def _chunkwise(q, k, v, weights, chunk, state_in):
    """Chunkwise form.  For a chunk of length L with local weights W (D of the chunk) and
    Gam_j = prod of the chunk's multipliers up to and including row j:
        O     = (Q K^T (.) W) V + diag(Gam) (Q S_prev)
        S_new = Gam_{L-1} S_prev + K^T (V (.) W[L-1, :])
    ("RetNet retention mechanism" tutorial, section 块级循环, with the per-row query
    decay; W[L-1, l] = Gam_{L-1}/Gam_l are the chunk-end decays described in "unilm
    RetNet 技术指南", section Triton 内核与自校验测试.)  The last chunk may be shorter.
    """
    B, H, N, dk = q.shape
    dv = v.shape[-1]
    if chunk < 1:
        raise ValueError("chunk must be >= 1")
    S = _initial_state(state_in, B, H, dk, dv)
    o = np.zeros((B, H, N, dv), dtype=np.float64)
    for c0 in range(0, N, chunk):
        c1 = min(c0 + chunk, N)
        Qc, Kc, Vc = q[:, :, c0:c1], k[:, :, c0:c1], v[:, :, c0:c1]
        W, Gam = weights(c0, c1)
        inner = np.einsum("bhjl,bhlv->bhjv", np.einsum("bhjd,bhld->bhjl", Qc, Kc) * W, Vc)
        cross = Gam[..., None] * np.einsum("bhjd,bhdv->bhjv", Qc, S)
        o[:, :, c0:c1] = inner + cross
        zeta = W[:, :, -1, :]
        S = Gam[:, :, -1, None, None] * S + np.einsum("bhld,bhlv->bhdv", Kc, Vc * zeta[..., None])
    return o, S


def retention_chunkwise(q, k, v, gamma, chunk, state_in=None):
    """Per-head-decay chunkwise form (cross-check of the recurrent oracle)."""
    q, k, v = _check_qkv(q, k, v)
    B, H = q.shape[:2]
    gm = _f64(gamma).reshape(H)
    return _chunkwise(q, k, v, lambda a, b: _weights_gamma(gm, B, a, b), int(chunk), state_in)


def gated_retention_chunkwise(q, k, v, g, chunk, state_in=None):
    """Gated chunkwise form (cross-check of the recurrent oracle)."""
    q, k, v = _check_qkv(q, k, v)
    g = _f64(g)
    return _chunkwise(q, k, v, lambda a, b: _weights_gated(g, a, b), int(chunk), state_in)


# ---------------------------------------------------------------------------------
# Backward of the recurrent form: the chain rule applied to the recurrence of record.
# ---------------------------------------------------------------------------------

def _recurrence_bwd(q, k, v, lam, state_in, do, dstate, want_dlam, ckpt=64):
    """Gradients of L = <dO, o> + <dS, S_{N-1}> for S_n = lam_n S_{n-1} + k_n^T v_n,
    o_n = q_n S_n, S_{-1} = S0 ("RetNet retention mechanism" tutorial, section 递归推理).

    The adjoint U_n = dL/dS_n collects every later use of S_n:
        U_{N-1} = q_{N-1}^T dO_{N-1} + dS,     U_n = q_n^T dO_n + lam_{n+1} U_{n+1},
    and then  dq_n = S_n dO_n,  dk_n = U_n v_n,  dv_n = U_n^T k_n,  dS0 = lam_0 U_0,
    dlam_n = <U_n, S_{n-1}>.  The forward sweep yields dq and keeps every ckpt-th state;
    when dlam is wanted the backward sweep recomputes each block's states from its
    checkpoint.  Returns (dq, dk, dv, dS0, dlam or None).
    """
    B, H, N, dk = q.shape
    dv = v.shape[-1]
    S = _initial_state(state_in, B, H, dk, dv)
    dq = np.zeros((B, H, N, dk), dtype=np.float64)
    ckpts = {}
    for n in range(N):
        if want_dlam and n % ckpt == 0:
            ckpts[n] = S.copy()                      # S_{n-1}
        S *= lam[:, :, n, None, None]
        S += k[:, :, n, :, None] * v[:, :, n, None, :]
        dq[:, :, n, :] = np.einsum("bhij,bhj->bhi", S, do[:, :, n, :])
    dkk = np.zeros((B, H, N, dk), dtype=np.float64)
    dvv = np.zeros((B, H, N, dv), dtype=np.float64)
    dlam = np.zeros((B, H, N), dtype=np.float64) if want_dlam else None
    U = np.zeros((B, H, dk, dv), dtype=np.float64) if dstate is None else _f64(dstate).copy()
    prev = {}
    for n in range(N - 1, -1, -1):
        if want_dlam and (n + 1) % ckpt == 0 or (want_dlam and n == N - 1):
            # states S_{m-1} for m in this checkpoint block, recomputed from its start
            c0 = (n // ckpt) * ckpt
            Sb = ckpts[c0].copy()
            prev = {}
            for m in range(c0, n + 1):
                prev[m] = Sb.copy()
                Sb *= lam[:, :, m, None, None]
                Sb += k[:, :, m, :, None] * v[:, :, m, None, :]
        U += q[:, :, n, :, None] * do[:, :, n, None, :]          # U_n
        dkk[:, :, n, :] = np.einsum("bhij,bhj->bhi", U, v[:, :, n, :])
        dvv[:, :, n, :] = np.einsum("bhij,bhi->bhj", U, k[:, :, n, :])
        if want_dlam:
            dlam[:, :, n] = np.einsum("bhij,bhij->bh", U, prev[n])
        U *= lam[:, :, n, None, None]                             # lam_n U_n, toward U_{n-1}
    return dq, dkk, dvv, U, dlam


def _check_bwd(q, do, dstate, B, H, N, dk, dv):
    do = _f64(do)
    if do.shape != (B, H, N, dv):
        raise ValueError(f"do must be [B,H,N,dv]={B,H,N,dv}; got {do.shape}")
    if dstate is not None and _f64(dstate).shape != (B, H, dk, dv):
        raise ValueError(f"dstate must be [B,H,dk,dv]={B,H,dk,dv}")
    return do


def retention_recurrent_bwd(q, k, v, gamma, do, state_in=None, dstate=None):
    """Backward of retention_recurrent for L = <do, o> + <dstate, state_out>.

    Returns (dq, dk, dv, dstate_in) in float64; dstate_in = gamma U_0 is the gradient
    with respect to state_in (zeros when no state was given, as for a zero state).
    """
    q, k, v = _check_qkv(q, k, v)
    B, H, N, dk = q.shape
    dv = v.shape[-1]
    do = _check_bwd(q, do, dstate, B, H, N, dk, dv)
    gamma = _f64(gamma).reshape(H)
    lam = np.broadcast_to(gamma[None, :, None], (B, H, N))
    dq, dkk, dvv, dS0, _ = _recurrence_bwd(q, k, v, lam, state_in, do, dstate, False)
    if N == 0 and dstate is not None:
        dS0 = _f64(dstate).copy()
    return dq, dkk, dvv, dS0


def gated_retention_recurrent_bwd(q, k, v, g, do, state_in=None, dstate=None):
    """Backward of gated_retention_recurrent: returns (dq, dk, dv, dg, dstate_in), with
    dg_n = exp(g_n) <U_n, S_{n-1}> (the multiplier is exp(g_n))."""
    q, k, v = _check_qkv(q, k, v)
    B, H, N, dk = q.shape
    dv = v.shape[-1]
    do = _check_bwd(q, do, dstate, B, H, N, dk, dv)
    g = _f64(g)
    if g.shape != (B, H, N):
        raise ValueError(f"g must be [B,H,N]={B,H,N}; got {g.shape}")
    lam = np.exp(g)
    dq, dkk, dvv, dS0, dlam = _recurrence_bwd(q, k, v, lam, state_in, do, dstate, True)
    if N == 0 and dstate is not None:
        dS0 = _f64(dstate).copy()
    return dq, dkk, dvv, lam * dlam, dS0
