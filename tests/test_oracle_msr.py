"""Pins of the gated retention layer's oracle (oracle/msr_oracle.py) against what the
page and mathematics fix, independent of the oracle's own code path:
  * the rotation equals multiplication of (x[2i] + i x[2i+1]) by exp(i n theta_i) in
    numpy's complex arithmetic, is the identity at position 0, and makes q.k depend only
    on the distance between positions;
  * RMSNorm has unit root-mean-square (eps = 0) and is scale invariant;
  * silu and logsigmoid against scipy's expit and numpy's logaddexp;
  * the whole layer on one and on two tokens, worked out by hand from the recurrence
    (S = lambda S + k^T v, o = q S) with the rotation done in complex arithmetic, both in
    full precision and with bf16 activations (every tensor handed from one operation to
    the next rounded to bf16 where it is stored, with torch's round-to-nearest-even
    cast), which pins the oracle's optional rounding path.
The mutation tests plant plausible mistakes in a copy of the oracle and check that a
pin fails for each.
"""
import types

import numpy as np
import pytest
from scipy.special import expit

import oracle
from oracle import msr_oracle as MO


def _rot_complex(x, n, base):
    """Rotate one vector x [d] as token n, through complex multiplication."""
    d = x.shape[-1]
    theta = base ** (-2.0 * np.arange(d // 2) / d)
    z = (x[0::2] + 1j * x[1::2]) * np.exp(1j * n * theta)
    out = np.empty(d)
    out[0::2], out[1::2] = z.real, z.imag
    return out


def _weights(rng, D, H, dk, dv):
    s = 1.0 / np.sqrt(D)
    return dict(wq=rng.standard_normal((H * dk, D)) * s, wk=rng.standard_normal((H * dk, D)) * s,
                wv=rng.standard_normal((H * dv, D)) * s, wg=rng.standard_normal((H * dv, D)) * s,
                wgt=rng.standard_normal((H, D)) * s, wo=rng.standard_normal((D, H * dv)) * s)


def pin_rope_complex(mod):
    rng = np.random.default_rng(0)
    x = rng.standard_normal((2, 3, 9, 8))
    got = mod.rope_interleaved(x, 500.0)
    for n in range(9):
        assert np.allclose(got[1, 2, n], _rot_complex(x[1, 2, n], n, 500.0), rtol=0, atol=1e-12)


def pin_rope_position_zero_and_relative(mod):
    rng = np.random.default_rng(1)
    d = 16
    q, k = rng.standard_normal(d), rng.standard_normal(d)
    seq = np.zeros((12, d))
    seq[0] = q
    assert np.array_equal(mod.rope_interleaved(seq)[0], q)
    # <rot(q, m), rot(k, n)> depends on m - n only
    def dot_at(m, n):
        a = np.zeros((12, d)); a[m] = q
        b = np.zeros((12, d)); b[n] = k
        return mod.rope_interleaved(a)[m] @ mod.rope_interleaved(b)[n]
    for (m, n, s) in ((5, 2, 4), (7, 7, 3), (3, 0, 8)):
        assert abs(dot_at(m, n) - dot_at(m + s - s // 2, n + s - s // 2)) < 1e-12


def pin_rms_norm(mod):
    rng = np.random.default_rng(2)
    x = rng.standard_normal((4, 5, 32)) * 3.0
    y = mod.rms_norm(x, 0.0)
    assert np.allclose(np.mean(y * y, axis=-1), 1.0, atol=1e-12)
    assert np.allclose(mod.rms_norm(7.5 * x, 0.0), y, atol=1e-12)
    # with eps: x / sqrt(ms + eps), checked on a row of constant magnitude
    row = np.full(8, 2.0)
    assert np.allclose(mod.rms_norm(row, 5.0), row / 3.0, atol=1e-15)


def pin_activations(mod):
    x = np.linspace(-30, 30, 121)
    assert np.allclose(mod.silu(x), x * expit(x), rtol=1e-13, atol=1e-300)
    assert np.allclose(mod.logsigmoid(x), -np.logaddexp(0.0, -x), rtol=1e-13, atol=1e-300)
    assert mod.silu(0.0) == 0.0 and mod.logsigmoid(0.0) == -np.log(2.0)


def pin_layer_one_token(mod):
    """N = 1: S = k^T v, o = (q.k) v per head; no rotation at position 0."""
    rng = np.random.default_rng(3)
    B, D, H, dk, dv, eps = 2, 12, 2, 4, 6, 0.3
    x = rng.standard_normal((B, 1, D))
    w = _weights(rng, D, H, dk, dv)
    y, _ = mod.gated_msr_forward(x, **w, H=H, dk=dk, dv=dv, eps=eps)
    for b in range(B):
        xb = x[b, 0]
        z = []
        for h in range(H):
            q = w["wq"][h * dk:(h + 1) * dk] @ xb
            k = w["wk"][h * dk:(h + 1) * dk] @ xb / np.sqrt(dk)
            v = w["wv"][h * dv:(h + 1) * dv] @ xb
            o = (q @ k) * v
            o = o / np.sqrt(np.mean(o ** 2) + eps)
            gate = w["wg"][h * dv:(h + 1) * dv] @ xb
            z.append(gate * expit(gate) * o)
        assert np.allclose(y[b, 0], w["wo"] @ np.concatenate(z), rtol=1e-12, atol=1e-12)


def pin_layer_two_tokens(mod):
    """N = 2: o_1 = lam_1 (q_1.k_0) v_0 + (q_1.k_1) v_1, lam_1 = sigmoid(gt_1)^(1/16),
    with token 1's q and k rotated as position 1."""
    rng = np.random.default_rng(4)
    D, H, dk, dv, eps, base = 10, 2, 4, 3, 1e-3, 10.0
    x = rng.standard_normal((1, 2, D))
    w = _weights(rng, D, H, dk, dv)
    y, g = mod.gated_msr_forward(x, **w, H=H, dk=dk, dv=dv, eps=eps, rope_base=base)
    x0, x1 = x[0, 0], x[0, 1]
    z = []
    for h in range(H):
        sl, sv = slice(h * dk, (h + 1) * dk), slice(h * dv, (h + 1) * dv)
        k0 = w["wk"][sl] @ x0 / np.sqrt(dk)
        q1 = _rot_complex(w["wq"][sl] @ x1, 1, base)
        k1 = _rot_complex(w["wk"][sl] @ x1, 1, base) / np.sqrt(dk)
        v0, v1 = w["wv"][sv] @ x0, w["wv"][sv] @ x1
        lam1 = expit(w["wgt"][h] @ x1) ** (1.0 / 16.0)
        assert abs(np.exp(g[0, h, 1]) - lam1) < 1e-14
        o = lam1 * (q1 @ k0) * v0 + (q1 @ k1) * v1
        o = o / np.sqrt(np.mean(o ** 2) + eps)
        gate = w["wg"][sv] @ x1
        z.append(gate * expit(gate) * o)
    assert np.allclose(y[0, 1], w["wo"] @ np.concatenate(z), rtol=1e-12, atol=1e-12)


def _bf16(a):
    """Round to bfloat16 (nearest even) with torch's cast, the library routine the GPU
    comparison also uses; returned as float64."""
    import torch
    return torch.tensor(np.asarray(a, dtype=np.float64)).to(torch.bfloat16).double().numpy()


def _bf16_inputs(rng, B, N, D, H, dk, dv):
    x = _bf16(rng.standard_normal((B, N, D)))
    w = {n: _bf16(a) for n, a in _weights(rng, D, H, dk, dv).items()}
    return x, w


def pin_layer_one_token_bf16(mod):
    """The layer with bf16 activations on one token, worked step by step: every tensor
    the layer hands from one operation to the next is stored in bf16 (q, and k after its
    scaling; v; the gate projection; the gated product; y), the retention output and the
    norm stay in full precision.  d_k = 6 makes the key scale irrational, so rounding
    before or after it differs."""
    rng = np.random.default_rng(13)
    B, D, H, dk, dv, eps = 2, 10, 2, 6, 4, 1e-5
    x, w = _bf16_inputs(rng, B, 1, D, H, dk, dv)
    y, _ = mod.gated_msr_forward(x, **w, H=H, dk=dk, dv=dv, eps=eps, act=_bf16)
    for b in range(B):
        xb = x[b, 0]
        z = []
        for h in range(H):
            sl, sv = slice(h * dk, (h + 1) * dk), slice(h * dv, (h + 1) * dv)
            q = _bf16(w["wq"][sl] @ xb)                    # position 0: no rotation
            k = _bf16(w["wk"][sl] @ xb / np.sqrt(dk))
            v = _bf16(w["wv"][sv] @ xb)
            o = (q @ k) * v                                 # S = k^T v, o = q S
            o = o / np.sqrt(np.mean(o ** 2) + eps)
            gate = _bf16(w["wg"][sv] @ xb)
            z.append(gate * expit(gate) * o)
        want = _bf16(w["wo"] @ _bf16(np.concatenate(z)))
        assert np.array_equal(y[b, 0], want), (y[b, 0], want)


def pin_layer_two_tokens_bf16(mod):
    """Two tokens with bf16 activations: token 1's q and k are rotated as position 1 in
    full precision and then rounded; the decay and the recurrence stay in full
    precision."""
    rng = np.random.default_rng(14)
    D, H, dk, dv, eps, base = 12, 2, 6, 3, 1e-5, 10.0
    x, w = _bf16_inputs(rng, 1, 2, D, H, dk, dv)
    y, _ = mod.gated_msr_forward(x, **w, H=H, dk=dk, dv=dv, eps=eps, rope_base=base, act=_bf16)
    x0, x1 = x[0, 0], x[0, 1]
    z = []
    for h in range(H):
        sl, sv = slice(h * dk, (h + 1) * dk), slice(h * dv, (h + 1) * dv)
        k0 = _bf16(w["wk"][sl] @ x0 / np.sqrt(dk))
        q1 = _bf16(_rot_complex(w["wq"][sl] @ x1, 1, base))
        k1 = _bf16(_rot_complex(w["wk"][sl] @ x1, 1, base) / np.sqrt(dk))
        v0, v1 = _bf16(w["wv"][sv] @ x0), _bf16(w["wv"][sv] @ x1)
        lam1 = expit(w["wgt"][h] @ x1) ** (1.0 / 16.0)
        o = lam1 * (q1 @ k0) * v0 + (q1 @ k1) * v1
        o = o / np.sqrt(np.mean(o ** 2) + eps)
        gate = _bf16(w["wg"][sv] @ x1)
        z.append(gate * expit(gate) * o)
    want = _bf16(w["wo"] @ _bf16(np.concatenate(z)))
    assert np.allclose(y[0, 1], want, rtol=0, atol=0), (y[0, 1], want)


PINS = [pin_rope_complex, pin_rope_position_zero_and_relative, pin_rms_norm, pin_activations,
        pin_layer_one_token, pin_layer_two_tokens, pin_layer_one_token_bf16, pin_layer_two_tokens_bf16]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_msr_oracle_pin(pin):
    pin(MO)


def test_activation_rounding_hook_is_inert_when_identity():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((1, 5, 8))
    w = _weights(rng, 8, 2, 4, 4)
    a, _ = MO.gated_msr_forward(x, **w, H=2, dk=4, dv=4)
    b, _ = MO.gated_msr_forward(x, **w, H=2, dk=4, dv=4, act=lambda t: t)
    assert np.array_equal(a, b)


def test_package_exports_layer():
    assert oracle.gated_msr_forward is MO.gated_msr_forward


def _mutant(replacements):
    src = open(MO.__file__).read()
    for old, new in replacements:
        assert old in src, old
        src = src.replace(old, new, 1)
    src = src.replace("from .retention_oracle import", "from oracle.retention_oracle import")
    mod = types.ModuleType("msr_oracle_mutant")
    exec(compile(src, "msr_oracle_mutant", "exec"), mod.__dict__)
    return mod


MUTANTS = {
    # rotation of the two halves instead of adjacent pairs
    "rope_halves": [("    x0, x1 = x[..., 0::2], x[..., 1::2]\n", "    x0, x1 = x[..., : d // 2], x[..., d // 2:]\n"),
                    ("    out[..., 0::2] = x0 * c - x1 * s\n    out[..., 1::2] = x0 * s + x1 * c\n",
                     "    out[..., : d // 2] = x0 * c - x1 * s\n    out[..., d // 2:] = x0 * s + x1 * c\n")],
    # positions counted from 1
    "rope_from_one": [("np.arange(N, dtype=np.float64)[:, None]", "np.arange(1, N + 1, dtype=np.float64)[:, None]")],
    # rotation angle with the wrong sign
    "rope_sign": [("    out[..., 1::2] = x0 * s + x1 * c\n", "    out[..., 1::2] = -x0 * s + x1 * c\n"),
                  ("    out[..., 0::2] = x0 * c - x1 * s\n", "    out[..., 0::2] = x0 * c + x1 * s\n")],
    # keys not scaled
    "no_key_scale": [(" / np.sqrt(dk))\n", ")\n")],
    # gate without the 1/16
    "gate_unnormalised": [("    g = logsigmoid(proj(wgt)).transpose(0, 2, 1) / gate_norm",
                           "    g = logsigmoid(proj(wgt)).transpose(0, 2, 1)")],
    # normalisation over all heads of a token instead of per head
    "norm_across_heads": [("    o = rms_norm(o, eps).transpose(0, 2, 1, 3).reshape(B, N, H * dv)\n",
                           "    o = rms_norm(o.transpose(0, 2, 1, 3).reshape(B, N, H * dv), eps)\n")],
    # gate activation on the retention output instead of the gate projection
    "silu_on_output": [("    z = r(silu(r(proj(wg))) * o)\n", "    z = r(r(proj(wg)) * silu(o))\n")],
    # sigmoid instead of silu
    "sigmoid_gate": [("    return x / (1.0 + np.exp(-x))\n", "    return 1.0 / (1.0 + np.exp(-x))\n")],
    # bf16 activations rounded at other points than the stored tensors:
    # q rounded before its rotation
    "act_q_before_rotation": [("    q = r(rope_interleaved(heads(proj(wq), dk), rope_base))\n",
                               "    q = rope_interleaved(heads(r(proj(wq)), dk), rope_base)\n")],
    # k rounded before its scaling
    "act_k_before_scale": [("    k = r(rope_interleaved(heads(proj(wk), dk), rope_base) / np.sqrt(dk))\n",
                            "    k = r(rope_interleaved(heads(proj(wk), dk), rope_base)) / np.sqrt(dk)\n")],
    # v kept in full precision
    "act_v_unrounded": [("    v = heads(r(proj(wv)), dv)\n", "    v = heads(proj(wv), dv)\n")],
    # the retention output rounded before the norm
    "act_o_rounded": [("    o, _ = gated_retention_recurrent(q, k, v, g)", "    o = r(gated_retention_recurrent(q, k, v, g)[0]); _ = 0")],
    # the gate projection kept in full precision
    "act_gate_unrounded": [("    z = r(silu(r(proj(wg))) * o)\n", "    z = r(silu(proj(wg)) * o)\n")],
    # the output left unrounded
    "act_y_unrounded": [("    return r(z @ _f64(wo).T), g\n", "    return z @ _f64(wo).T, g\n")],
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name):
    mod = _mutant(MUTANTS[name])
    failed = 0
    for pin in PINS:
        try:
            pin(mod)
        except AssertionError:
            failed += 1
    assert failed > 0, f"no pin caught {name}"
