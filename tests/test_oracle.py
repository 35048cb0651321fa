"""Pins of the fp64 oracle against what the pages and mathematics fix.

Each pin is independent of the oracle's own code path:
  * hand-worked fixtures (tests/golden/hand_worked.json), derived from the recurrence;
  * exact rational brute force of the *sum* definition (Fraction arithmetic);
  * closed forms on all-ones inputs;
  * gamma = 1 reduces to causal linear attention, computed with np.cumsum;
  * the decay matrix read back through one-hot values;
  * agreement of the three forms, split/resume, linearity.
The mutation tests at the end plant plausible mistakes in a copy of the oracle and
check that at least one pin fails for each.
"""
import json
import os
import types
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import retention_oracle as RO

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_worked.json")


def _t(x):
    """[N, d] list -> [1, 1, N, d] float64."""
    return np.asarray(x, dtype=np.float64)[None, None]


def _rel(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300)


# ------------------------------------------------------------------------- pin helpers
# Each helper takes the oracle module so the mutation tests can run it on a mutant.

def pin_golden(mod):
    with open(GOLDEN) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        q, k, v = _t(c["q"]), _t(c["k"]), _t(c["v"])
        S0 = None if "state_in" not in c else np.asarray(c["state_in"], float)[None, None]
        if "gamma" in c:
            gm = np.asarray(c["gamma"], float)
            forms = [mod.retention_recurrent(q, k, v, gm, S0),
                     mod.retention_parallel(q, k, v, gm, S0),
                     mod.retention_chunkwise(q, k, v, gm, 2, S0)]
            tol = 0.0
        else:
            g = np.log(np.asarray(c["g_as_decay"], float))[None, None]
            forms = [mod.gated_retention_recurrent(q, k, v, g, S0),
                     mod.gated_retention_parallel(q, k, v, g, S0),
                     mod.gated_retention_chunkwise(q, k, v, g, 2, S0)]
            tol = 1e-14
        for o, S in forms:
            assert _rel(o[0, 0], c["o"]) <= tol + 1e-15, (c["name"], o[0, 0], c["o"])
            assert _rel(S[0, 0], c["state_out"]) <= tol + 1e-15, (c["name"], S[0, 0])


def _fraction_sum_definition(q, k, v, lam, S0):
    """Exact output by the sum definition, with per-token multipliers lam[n] (Fractions):
    o_n = sum_{m<=n} (prod_{m<t<=n} lam_t) (q_n . k_m) v_m + (prod_{t<=n} lam_t) q_n S0."""
    N, dk = len(q), len(q[0])
    dv = len(v[0])
    out = []
    for n in range(N):
        row = []
        for j in range(dv):
            acc = Fraction(0)
            for m in range(n + 1):
                w = Fraction(1)
                for t in range(m + 1, n + 1):
                    w *= lam[t]
                acc += w * sum(q[n][i] * k[m][i] for i in range(dk)) * v[m][j]
            w0 = Fraction(1)
            for t in range(n + 1):
                w0 *= lam[t]
            acc += w0 * sum(q[n][i] * S0[i][j] for i in range(dk))
            row.append(acc)
        out.append(row)
    # final state by the same definition
    S = [[Fraction(0)] * dv for _ in range(dk)]
    for i in range(dk):
        for j in range(dv):
            acc = Fraction(0)
            for m in range(N):
                w = Fraction(1)
                for t in range(m + 1, N):
                    w *= lam[t]
                acc += w * k[m][i] * v[m][j]
            w0 = Fraction(1)
            for t in range(N):
                w0 *= lam[t]
            S[i][j] = acc + w0 * S0[i][j]
    return out, S


def pin_exact_rational(mod, trials=12, seed=0):
    rng = np.random.default_rng(seed)
    for _ in range(trials):
        N = int(rng.integers(1, 9))
        dk = int(rng.integers(1, 4))
        dv = int(rng.integers(1, 4))
        gam = [Fraction(1, 2), Fraction(1, 4), Fraction(3, 4), Fraction(1)][int(rng.integers(0, 4))]
        qi = rng.integers(-2, 3, size=(N, dk))
        ki = rng.integers(-2, 3, size=(N, dk))
        vi = rng.integers(-2, 3, size=(N, dv))
        Si = rng.integers(-2, 3, size=(dk, dv))
        F = lambda a: [[Fraction(int(x)) for x in r] for r in a]  # noqa: E731
        exp_o, exp_S = _fraction_sum_definition(F(qi), F(ki), F(vi), [gam] * N, F(Si))
        o, S = mod.retention_recurrent(qi[None, None].astype(float), ki[None, None].astype(float),
                                       vi[None, None].astype(float), np.array([float(gam)]),
                                       Si[None, None].astype(float))
        # dyadic inputs with few bits: fp64 must be exact
        assert np.array_equal(o[0, 0], np.array(exp_o, dtype=float)), (gam, o[0, 0], exp_o)
        assert np.array_equal(S[0, 0], np.array(exp_S, dtype=float))
        od, Sd = _decode_chain(mod, qi, ki, vi, float(gam), Si)
        assert np.array_equal(od, np.array(exp_o, dtype=float))
        assert np.array_equal(Sd, np.array(exp_S, dtype=float))


def _decode_chain(mod, qi, ki, vi, gam, Si):
    S = Si[None, None].astype(float)
    outs = []
    for n in range(len(qi)):
        o, S = mod.retention_decode_step(qi[None, None, n].astype(float), ki[None, None, n].astype(float),
                                         vi[None, None, n].astype(float), np.array([gam]), S)
        outs.append(o[0, 0])
    return np.array(outs), S[0, 0]


def pin_gated_exact(mod, trials=8, seed=1):
    """Gated form with dyadic per-token decays lam_n = exp(g_n); exact to ~1e-14."""
    rng = np.random.default_rng(seed)
    choices = [Fraction(1, 2), Fraction(1, 4), Fraction(3, 4), Fraction(1), Fraction(7, 8)]
    for _ in range(trials):
        N = int(rng.integers(1, 8))
        dk = int(rng.integers(1, 4))
        dv = int(rng.integers(1, 4))
        lam = [choices[int(i)] for i in rng.integers(0, len(choices), size=N)]
        qi = rng.integers(-2, 3, size=(N, dk))
        ki = rng.integers(-2, 3, size=(N, dk))
        vi = rng.integers(-2, 3, size=(N, dv))
        Si = rng.integers(-2, 3, size=(dk, dv))
        F = lambda a: [[Fraction(int(x)) for x in r] for r in a]  # noqa: E731
        exp_o, exp_S = _fraction_sum_definition(F(qi), F(ki), F(vi), lam, F(Si))
        g = np.log(np.array([float(x) for x in lam]))[None, None]
        args = (qi[None, None].astype(float), ki[None, None].astype(float), vi[None, None].astype(float), g,
                Si[None, None].astype(float))
        for o, S in (mod.gated_retention_recurrent(*args), mod.gated_retention_parallel(*args),
                     mod.gated_retention_chunkwise(*args[:4], 3, args[4])):
            eo = np.array(exp_o, dtype=float)
            eS = np.array(exp_S, dtype=float)
            assert np.allclose(o[0, 0], eo, rtol=1e-13, atol=1e-13 * max(1, np.abs(eo).max()))
            assert np.allclose(S[0, 0], eS, rtol=1e-13, atol=1e-13 * max(1, np.abs(eS).max()))


def pin_closed_form_all_ones(mod):
    """All-ones q, k, v from zero state: o_n = dk (1 - gamma^(n+1)) / (1 - gamma) in every
    column, and S_N = (1 - gamma^N)/(1 - gamma) everywhere (geometric series)."""
    B, H, N, dk, dv = 1, 3, 40, 5, 3
    gam = np.array([0.5, 0.9, 0.99])
    ones_q = np.ones((B, H, N, dk))
    ones_v = np.ones((B, H, N, dv))
    n = np.arange(N)
    exp_o = dk * (1 - gam[:, None] ** (n[None, :] + 1)) / (1 - gam[:, None])   # [H, N]
    exp_S = (1 - gam ** N) / (1 - gam)
    for o, S in (mod.retention_recurrent(ones_q, ones_q, ones_v, gam),
                 mod.retention_parallel(ones_q, ones_q, ones_v, gam),
                 mod.retention_chunkwise(ones_q, ones_q, ones_v, gam, 7)):
        assert _rel(o[0], np.broadcast_to(exp_o[:, :, None], (H, N, dv))) < 1e-13
        assert _rel(S[0], np.broadcast_to(exp_S[:, None, None], (H, dk, dv))) < 1e-13
    # gated with a constant g = log(gamma) is the same series
    g = np.broadcast_to(np.log(gam)[None, :, None], (B, H, N))
    for o, S in (mod.gated_retention_recurrent(ones_q, ones_q, ones_v, g),
                 mod.gated_retention_parallel(ones_q, ones_q, ones_v, g),
                 mod.gated_retention_chunkwise(ones_q, ones_q, ones_v, g, 9)):
        assert _rel(o[0], np.broadcast_to(exp_o[:, :, None], (H, N, dv))) < 1e-12
        assert _rel(S[0], np.broadcast_to(exp_S[:, None, None], (H, dk, dv))) < 1e-12


def pin_gamma_one_linear_attention(mod):
    """gamma = 1: undecayed causal linear attention (tutorial quiz, question 6):
    o_n = q_n . cumsum_{m<=n}(k_m^T v_m), computed here with np.cumsum."""
    rng = np.random.default_rng(3)
    B, H, N, dk, dv = 2, 2, 13, 4, 6
    q = rng.standard_normal((B, H, N, dk))
    k = rng.standard_normal((B, H, N, dk))
    v = rng.standard_normal((B, H, N, dv))
    outer = k[..., :, None] * v[..., None, :]            # [B,H,N,dk,dv]
    prefix = np.cumsum(outer, axis=2)
    exp_o = (q[..., :, None] * prefix).sum(axis=3)
    for o, S in (mod.retention_recurrent(q, k, v, np.ones(H)),
                 mod.retention_parallel(q, k, v, np.ones(H)),
                 mod.retention_chunkwise(q, k, v, np.ones(H), 4)):
        assert _rel(o, exp_o) < 1e-12
        assert _rel(S, prefix[:, :, -1]) < 1e-12
    ones = np.ones((1, 1, N, dk))
    o, _ = mod.retention_recurrent(ones, ones, np.ones((1, 1, N, 1)), np.ones(1))
    assert np.array_equal(o[0, 0, :, 0], dk * (np.arange(N) + 1.0))


def pin_decay_matrix(mod):
    """Read D back: with dk = 1, q = k = 1 and one-hot values v_m = e_m, the output is
    o_n[m] = D_nm = gamma^(n-m) for n >= m and 0 for n < m (tutorial, section 衰减矩阵
    and quiz question 3)."""
    N = 7
    gm = 0.5
    q = np.ones((1, 1, N, 1))
    v = np.eye(N)[None, None]
    exp_D = np.array([[gm ** (n - m) if n >= m else 0.0 for m in range(N)] for n in range(N)])
    for o, _ in (mod.retention_recurrent(q, q, v, np.array([gm])),
                 mod.retention_parallel(q, q, v, np.array([gm])),
                 mod.retention_chunkwise(q, q, v, np.array([gm]), 3)):
        assert np.array_equal(o[0, 0], exp_D)


def pin_N1(mod):
    rng = np.random.default_rng(4)
    q, k = rng.standard_normal((2, 1, 1, 1, 3))
    v = rng.standard_normal((1, 1, 1, 2))
    S0 = rng.standard_normal((1, 1, 3, 2))
    gm = np.array([0.7])
    exp = (q[0, 0, 0] @ k[0, 0, 0]) * v[0, 0, 0] + 0.7 * (q[0, 0, 0] @ S0[0, 0])
    o, _ = mod.retention_recurrent(q, k, v, gm, S0)
    assert _rel(o[0, 0, 0], exp) < 1e-15


def _loss(mod, gated, q, k, v, dec, S0, do, dS):
    """L = <do, o> + <dS, S_N>, through the forward oracle."""
    f = mod.gated_retention_recurrent if gated else mod.retention_recurrent
    o, S = f(q, k, v, dec, S0)
    return float(np.sum(do * o) + np.sum(dS * S))


def pin_bwd_finite_difference(mod):
    """Backward pinned to central differences of the forward oracle (brute force on tiny
    inputs): every element of q, k, v, the initial state and, gated, g."""
    rng = np.random.default_rng(11)
    B, H, N, dk, dv = 1, 2, 6, 3, 2
    q, k = rng.standard_normal((2, B, H, N, dk))
    v, do = rng.standard_normal((2, B, H, N, dv))
    S0, dS = rng.standard_normal((2, B, H, dk, dv))
    h = 1e-6
    for gated in (False, True):
        dec = -0.4 * np.abs(rng.standard_normal((B, H, N))) if gated else np.array([0.8, 0.55])
        if gated:
            dq, dk_, dv_, dg, dS0 = mod.gated_retention_recurrent_bwd(q, k, v, dec, do, S0, dS)
            inputs = dict(q=(q, dq), k=(k, dk_), v=(v, dv_), dec=(dec, dg), S0=(S0, dS0))
        else:
            dq, dk_, dv_, dS0 = mod.retention_recurrent_bwd(q, k, v, dec, do, S0, dS)
            inputs = dict(q=(q, dq), k=(k, dk_), v=(v, dv_), S0=(S0, dS0))
        for name, (x, grad) in inputs.items():
            fd = np.zeros_like(x)
            for idx in np.ndindex(*x.shape):
                args = dict(q=q, k=k, v=v, dec=dec, S0=S0)
                xp = x.copy(); xp[idx] += h
                xm = x.copy(); xm[idx] -= h
                args[name] = xp
                lp = _loss(mod, gated, args["q"], args["k"], args["v"], args["dec"], args["S0"], do, dS)
                args[name] = xm
                lm = _loss(mod, gated, args["q"], args["k"], args["v"], args["dec"], args["S0"], do, dS)
                fd[idx] = (lp - lm) / (2 * h)
            assert _rel(grad, fd) < 1e-6, (gated, name, _rel(grad, fd))


def pin_bwd_N1(mod):
    """One token, by hand: S = lam S0 + k^T v, o = q S, U = q^T dO + dS;
    dq = S dO, dk = U v, dv = U^T k, dS0 = lam U, dg = lam <U, S0>."""
    rng = np.random.default_rng(12)
    q, k = rng.standard_normal((2, 1, 1, 1, 3))
    v, do = rng.standard_normal((2, 1, 1, 1, 2))
    S0, dS = rng.standard_normal((2, 1, 1, 3, 2))
    lam = 0.6
    S = lam * S0[0, 0] + np.outer(k[0, 0, 0], v[0, 0, 0])
    U = np.outer(q[0, 0, 0], do[0, 0, 0]) + dS[0, 0]
    exp = dict(dq=S @ do[0, 0, 0], dk=U @ v[0, 0, 0], dv=U.T @ k[0, 0, 0], dS0=lam * U,
               dg=lam * np.sum(U * S0[0, 0]))
    dq, dk_, dv_, dS0 = mod.retention_recurrent_bwd(q, k, v, np.array([lam]), do, S0, dS)
    got = dict(dq=dq[0, 0, 0], dk=dk_[0, 0, 0], dv=dv_[0, 0, 0], dS0=dS0[0, 0])
    gq, gk, gv, gg, gS0 = mod.gated_retention_recurrent_bwd(q, k, v, np.log([[[lam]]]), do, S0, dS)
    for name in got:
        assert _rel(got[name], exp[name]) < 1e-14, name
    for name, val in dict(dq=gq[0, 0, 0], dk=gk[0, 0, 0], dv=gv[0, 0, 0], dS0=gS0[0, 0], dg=gg[0, 0, 0]).items():
        assert _rel(val, exp[name]) < 1e-14, ("gated", name)


ALL_PINS = [pin_golden, pin_exact_rational, pin_gated_exact, pin_closed_form_all_ones,
            pin_gamma_one_linear_attention, pin_decay_matrix, pin_N1,
            pin_bwd_finite_difference, pin_bwd_N1]


# ------------------------------------------------------------------------- the tests

@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    pin(RO)


@pytest.mark.parametrize("gated", [False, True])
@pytest.mark.parametrize("chunk", [1, 2, 3, 16, "N"])
def test_three_forms_agree(gated, chunk):
    """Recurrent, parallel and chunkwise forms agree to 1e-10 (every page calls them
    equivalent), including ragged last chunks and a nonzero initial state."""
    rng = np.random.default_rng(11)
    for N in (1, 5, 17, 64):
        B, H, dk, dv = 2, 3, 8, 5
        q = rng.standard_normal((B, H, N, dk)) / np.sqrt(dk)
        k = rng.standard_normal((B, H, N, dk)) / np.sqrt(dk)
        v = rng.standard_normal((B, H, N, dv)) / np.sqrt(dk)
        S0 = rng.standard_normal((B, H, dk, dv)) * 0.1
        C = N if chunk == "N" else chunk
        if gated:
            from retnet_retention_fwd_amd.inputs import logsigmoid
            g = logsigmoid(rng.standard_normal((B, H, N))) / 16
            ref = RO.gated_retention_recurrent(q, k, v, g, S0)
            outs = [RO.gated_retention_parallel(q, k, v, g, S0),
                    RO.gated_retention_chunkwise(q, k, v, g, C, S0)]
        else:
            gm = np.array([0.9, 0.99, 1.0])
            ref = RO.retention_recurrent(q, k, v, gm, S0)
            outs = [RO.retention_parallel(q, k, v, gm, S0),
                    RO.retention_chunkwise(q, k, v, gm, C, S0)]
        for o, S in outs:
            assert _rel(o, ref[0]) <= 1e-10
            assert _rel(S, ref[1]) <= 1e-10


def test_tiny_workload_forms_agree():
    """The tiny fp32 workload's own inputs: three forms agree to 1e-10."""
    from retnet_retention_fwd_amd.inputs import WORKLOADS, make_chunkwise
    w = WORKLOADS["tiny_f32"]
    x = make_chunkwise(w)
    q, k, v, gm = (x[n][1] for n in ("q", "k", "v", "gamma"))
    o, S = RO.retention_recurrent(q, k, v, gm)
    for o2, S2 in (RO.retention_parallel(q, k, v, gm), RO.retention_chunkwise(q, k, v, gm, w.chunk)):
        assert _rel(o2, o) <= 1e-10 and _rel(S2, S) <= 1e-10


@pytest.mark.parametrize("gated", [False, True])
def test_split_resume(gated):
    """run(N1+N2) == run(N2, state_in = run(N1).state_out)."""
    rng = np.random.default_rng(5)
    B, H, N, dk, dv = 1, 2, 30, 4, 3
    q, k = rng.standard_normal((2, B, H, N, dk))
    v = rng.standard_normal((B, H, N, dv))
    g = -np.abs(rng.standard_normal((B, H, N))) / 8
    gm = np.array([0.8, 0.95])

    def f(sl, s):
        if gated:
            return RO.gated_retention_recurrent(q[:, :, sl], k[:, :, sl], v[:, :, sl], g[:, :, sl], s)
        return RO.retention_chunkwise(q[:, :, sl], k[:, :, sl], v[:, :, sl], gm, 4, s)

    o_full, S_full = f(slice(0, N), None)
    o1, S1 = f(slice(0, 11), None)
    o2, S2 = f(slice(11, N), S1)
    assert _rel(np.concatenate([o1, o2], axis=2), o_full) < 1e-13
    assert _rel(S2, S_full) < 1e-13


def test_prefill_then_decode():
    """A chunkwise prefill's final state seeds decode steps; the result equals the
    recurrence over the concatenated sequence (unilm guide, section 三种计算路径与增量状态:
    the prefill seeds the decode state)."""
    rng = np.random.default_rng(6)
    B, H, N, M, dk, dv = 2, 2, 20, 5, 4, 4
    q, k = rng.standard_normal((2, B, H, N + M, dk))
    v = rng.standard_normal((B, H, N + M, dv))
    gm = np.array([0.9, 0.97])
    o_ref, S_ref = RO.retention_recurrent(q, k, v, gm)
    _, S = RO.retention_chunkwise(q[:, :, :N], k[:, :, :N], v[:, :, :N], gm, 8)
    for t in range(N, N + M):
        o, S = RO.retention_decode_step(q[:, :, t], k[:, :, t], v[:, :, t], gm, S)
        assert _rel(o, o_ref[:, :, t]) < 1e-12
    assert _rel(S, S_ref) < 1e-12


def test_gated_decode_matches_recurrent():
    rng = np.random.default_rng(7)
    B, H, N, dk, dv = 2, 3, 9, 4, 5
    q, k = rng.standard_normal((2, B, H, N, dk))
    v = rng.standard_normal((B, H, N, dv))
    g = -np.abs(rng.standard_normal((B, H, N))) / 4
    S0 = rng.standard_normal((B, H, dk, dv))
    o_ref, S_ref = RO.gated_retention_recurrent(q, k, v, g, S0)
    S = S0
    for t in range(N):
        o, S = RO.gated_retention_decode_step(q[:, :, t], k[:, :, t], v[:, :, t], g[:, :, t], S)
        assert _rel(o, o_ref[:, :, t]) < 1e-12
    assert _rel(S, S_ref) < 1e-12


def test_linearity():
    """With a zero initial state, O is linear in Q and in V."""
    rng = np.random.default_rng(8)
    B, H, N, dk, dv = 1, 2, 12, 3, 4
    q1, q2, k = rng.standard_normal((3, B, H, N, dk))
    v1, v2 = rng.standard_normal((2, B, H, N, dv))
    gm = np.array([0.6, 0.9])
    a, b = 1.75, -0.5
    f = lambda q, v: RO.retention_recurrent(q, k, v, gm)[0]  # noqa: E731
    assert _rel(f(a * q1 + b * q2, v1), a * f(q1, v1) + b * f(q2, v1)) < 1e-13
    assert _rel(f(q1, a * v1 + b * v2), a * f(q1, v1) + b * f(q1, v2)) < 1e-13


def test_empty_sequence():
    """N = 0: no outputs, and the final state is the initial state."""
    q = np.zeros((1, 2, 0, 3))
    v = np.zeros((1, 2, 0, 4))
    S0 = np.arange(24, dtype=float).reshape(1, 2, 3, 4)
    for o, S in (RO.retention_recurrent(q, q, v, np.array([0.5, 0.9]), S0),
                 RO.retention_chunkwise(q, q, v, np.array([0.5, 0.9]), 4, S0),
                 RO.gated_retention_recurrent(q, q, v, np.zeros((1, 2, 0)), S0)):
        assert o.shape == (1, 2, 0, 4)
        assert np.array_equal(S, S0)


def test_public_surface():
    for name in oracle.__all__:
        assert callable(getattr(oracle, name))


# ------------------------------------------------------------------ mutation testing

def _mutant(replacements):
    """A copy of the oracle module with textual edits applied (mistakes planted on the CPU)."""
    src = open(RO.__file__).read()
    for old, new in replacements:
        assert old in src, old
        src = src.replace(old, new, 1)
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src, "oracle_mutant", "exec"), mod.__dict__)
    return mod


MUTANTS = {
    # read-out before the state update (D_nn would be 0)
    "readout_before_update": [(
        "        S *= lam[:, :, n, None, None]\n        S += k[:, :, n, :, None] * v[:, :, n, None, :]\n"
        "        o[:, :, n, :] = np.einsum(\"bhi,bhij->bhj\", q[:, :, n, :], S)\n",
        "        o[:, :, n, :] = np.einsum(\"bhi,bhij->bhj\", q[:, :, n, :], S)\n"
        "        S *= lam[:, :, n, None, None]\n        S += k[:, :, n, :, None] * v[:, :, n, None, :]\n")],
    # decay applied after adding the new outer product
    "decay_after_add": [(
        "        S *= lam[:, :, n, None, None]\n        S += k[:, :, n, :, None] * v[:, :, n, None, :]\n",
        "        S += k[:, :, n, :, None] * v[:, :, n, None, :]\n        S *= lam[:, :, n, None, None]\n")],
    # decay dropped
    "no_decay": [("        S *= lam[:, :, n, None, None]\n", "")],
    # q and k swapped in the outer product
    "q_in_state": [("        S += k[:, :, n, :, None] * v[:, :, n, None, :]\n",
                    "        S += q[:, :, n, :, None] * v[:, :, n, None, :]\n")],
    # decode step: old state not decayed
    "decode_no_decay": [("    S *= _f64(gamma).reshape(1, H, 1, 1)\n", "")],
    # gated: decay exp(-g) (wrong sign)
    "gated_sign": [("    return _recurrence(q, k, v, np.exp(g), state_in)",
                    "    return _recurrence(q, k, v, np.exp(-g), state_in)")],
    # parallel form: D transposed (anti-causal)
    "parallel_anticausal": [("    causal = expo >= 0\n", "    causal = expo <= 0\n    expo = -expo\n")],
    # gated weights: exclusive instead of inclusive cumsum
    "gated_exclusive": [("    G = np.cumsum(g[:, :, p0:p1], axis=-1)  ", "    G = np.cumsum(g[:, :, p0:p1], axis=-1) - g[:, :, p0:p1]  ")],
    # per-head initial-state weight gamma^n instead of gamma^(n+1)
    "state_weight_off_by_one": [("** (idx[None, None, :] + 1)", "** (idx[None, None, :])")],
    # chunkwise: one gamma^c factor for every row of the cross-chunk term (the
    # simplification written on the tutorial page)
    "chunk_single_factor": [("        cross = Gam[..., None] * ",
                             "        cross = Gam[..., -1:, None] * ")],
    # chunkwise: key-side decay dropped from the state update
    "chunk_no_zeta": [("\"bhld,bhlv->bhdv\", Kc, Vc * zeta[..., None])", "\"bhld,bhlv->bhdv\", Kc, Vc)")],
    # chunkwise: state carried without the chunk decay
    "chunk_no_carry_decay": [("        S = Gam[:, :, -1, None, None] * S + ", "        S = S + ")],
    # backward: adjoint state not decayed between tokens
    "bwd_no_adjoint_decay": [("        U *= lam[:, :, n, None, None]                             # lam_n U_n, toward U_{n-1}\n", "")],
    # backward: dq from the state before the token's update
    "bwd_dq_old_state": [(
        "        S *= lam[:, :, n, None, None]\n        S += k[:, :, n, :, None] * v[:, :, n, None, :]\n"
        "        dq[:, :, n, :] = np.einsum(\"bhij,bhj->bhi\", S, do[:, :, n, :])\n",
        "        dq[:, :, n, :] = np.einsum(\"bhij,bhj->bhi\", S, do[:, :, n, :])\n"
        "        S *= lam[:, :, n, None, None]\n        S += k[:, :, n, :, None] * v[:, :, n, None, :]\n")],
    # backward: dv contracted with q instead of k
    "bwd_dv_uses_q": [("dvv[:, :, n, :] = np.einsum(\"bhij,bhi->bhj\", U, k[:, :, n, :])",
                       "dvv[:, :, n, :] = np.einsum(\"bhij,bhi->bhj\", U, q[:, :, n, :])")],
    # backward: gate gradient against S_n instead of S_{n-1}
    "bwd_dlam_new_state": [("                prev[m] = Sb.copy()\n                Sb *= lam[:, :, m, None, None]\n"
                            "                Sb += k[:, :, m, :, None] * v[:, :, m, None, :]\n",
                            "                Sb *= lam[:, :, m, None, None]\n"
                            "                Sb += k[:, :, m, :, None] * v[:, :, m, None, :]\n                prev[m] = Sb.copy()\n")],
    # backward: final-state gradient ignored
    "bwd_no_dstate": [("    U = np.zeros((B, H, dk, dv), dtype=np.float64) if dstate is None else _f64(dstate).copy()",
                       "    U = np.zeros((B, H, dk, dv), dtype=np.float64)")],
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name):
    mod = _mutant(MUTANTS[name])
    failed = []
    for pin in ALL_PINS:
        try:
            pin(mod)
        except (AssertionError, ValueError, IndexError):
            failed.append(pin.__name__)
    assert failed, f"no pin caught mutant {name}"


def test_unmutated_copy_passes_all_pins():
    mod = _mutant([])
    for pin in ALL_PINS:
        pin(mod)


# ------------------------------------------------------------------ backward structure

@pytest.mark.parametrize("gated", [False, True])
def test_bwd_checkpoint_blocks(gated):
    """The gate gradient's recomputation from checkpoints does not depend on the block."""
    rng = np.random.default_rng(21)
    B, H, N, dk, dv = 1, 2, 23, 4, 3
    q, k = rng.standard_normal((2, B, H, N, dk))
    v, do = rng.standard_normal((2, B, H, N, dv))
    lam = np.exp(-0.3 * np.abs(rng.standard_normal((B, H, N))))
    ref = RO._recurrence_bwd(q, k, v, lam, None, do, None, True, ckpt=64)
    for c in (1, 3, 7, 23):
        got = RO._recurrence_bwd(q, k, v, lam, None, do, None, True, ckpt=c)
        for a, b in zip(got, ref):
            assert np.array_equal(a, b)


def _flip(x):
    return np.ascontiguousarray(x[:, :, ::-1])


@pytest.mark.parametrize("gated", [False, True])
def test_bwd_as_forward_passes(gated):
    """The identities the GPU backward is built on, checked on the oracle alone:
    dq is a forward pass with (q, k, v) -> (do, v, k) and initial state S0^T; dv and dk
    are forward passes over the time-reversed sequence, (k, q, do) and (v, do, q), whose
    initial state is dS (scaled by 1/gamma, or with a reversed gate shifted by one
    whose first entry is 0), and dS0 is gamma (or exp(g_0)) times the state the dv pass
    ends with; gated, dg is the reversed cumulative sum of q.dq - k.dk plus <dS, S_N>."""
    rng = np.random.default_rng(22)
    B, H, N, dk, dv = 2, 2, 37, 5, 4
    q, k = rng.standard_normal((2, B, H, N, dk))
    v, do = rng.standard_normal((2, B, H, N, dv))
    S0, dS = rng.standard_normal((2, B, H, dk, dv))
    T = lambda S: np.ascontiguousarray(np.swapaxes(S, -1, -2))  # noqa: E731
    if gated:
        g = -0.3 * np.abs(rng.standard_normal((B, H, N)))
        dq, dk_, dv_, dg, dS0 = oracle.gated_retention_recurrent_bwd(q, k, v, g, do, S0, dS)
        gr = np.concatenate([np.zeros((B, H, 1)), g[:, :, :0:-1]], axis=-1)
        fq, S_fin_t = oracle.gated_retention_recurrent(do, v, k, g, T(S0))
        fv, U0 = oracle.gated_retention_recurrent(_flip(k), _flip(q), _flip(do), gr, dS)
        fk, _ = oracle.gated_retention_recurrent(_flip(v), _flip(do), _flip(q), gr, T(dS))
        lam0 = np.exp(g[:, :, 0])[..., None, None]
    else:
        gm = np.array([0.9, 0.45])
        dq, dk_, dv_, dS0 = oracle.retention_recurrent_bwd(q, k, v, gm, do, S0, dS)
        sc = (1.0 / gm)[None, :, None, None]
        fq, S_fin_t = oracle.retention_recurrent(do, v, k, gm, T(S0))
        fv, U0 = oracle.retention_recurrent(_flip(k), _flip(q), _flip(do), gm, dS * sc)
        fk, _ = oracle.retention_recurrent(_flip(v), _flip(do), _flip(q), gm, T(dS * sc))
        lam0 = gm[None, :, None, None]
    assert _rel(fq, dq) < 1e-12
    assert _rel(_flip(fv), dv_) < 1e-12
    assert _rel(_flip(fk), dk_) < 1e-12
    assert _rel(lam0 * U0, dS0) < 1e-12
    if gated:
        _, S_fin = oracle.gated_retention_recurrent(q, k, v, g, S0)
        assert _rel(T(S_fin_t), S_fin) < 1e-12
        dG = np.sum(q * dq, -1) - np.sum(k * dk_, -1)
        dG[:, :, -1] += np.sum(dS * S_fin, axis=(-1, -2))
        assert _rel(np.cumsum(dG[:, :, ::-1], -1)[:, :, ::-1], dg) < 1e-10
