"""Pins of the gate variants (oracle/variants.py), CPU only.

GDN through the per-channel oracle is checked against an exact rational GDN
recurrence written in GDN's own order (erase, then one decay per token), and
DeltaNet against the exact recurrence with no decay and the delta write-back
identity. Each check_* takes the variants module so that mutated copies can
be checked too (test_oracle_mutations.py).
"""
import math
from fractions import Fraction

import numpy as np
import pytest

from oracle import brute, reference, variants

LN_HALF = math.log(0.5)


def _case(rng, T, H, Dk, Dv):
    q = rng.standard_normal((T, H, Dk)).astype(np.float32)
    k = rng.standard_normal((T, H, Dk))
    k = (k / np.linalg.norm(k, axis=-1, keepdims=True)).astype(np.float32)
    v = rng.standard_normal((T, H, Dv)).astype(np.float32)
    beta = rng.uniform(0.1, 0.9, (T, H)).astype(np.float32)
    S0 = (0.3 * rng.standard_normal((1, H, Dk, Dv))).astype(np.float64)
    return q, k, v, beta, S0


def _exact(x):
    return [[Fraction(float(e)) for e in row] for row in x]


def check_gdn_matches_exact_scalar_gate(var):
    rng = np.random.default_rng(31)
    T, H, Dk, Dv = 10, 2, 4, 3
    q, k, v, beta, S0 = _case(rng, T, H, Dk, Dv)
    g = rng.uniform(LN_HALF, 0.0, (T, H)).astype(np.float32)       # one log-decay per token and head
    g[3, 0] = -2.0                                                   # below the floor: clamped to ln 1/2
    gc = var.gate_per_channel(g, var.GATE_HEAD, (T, H, Dk))
    o, fin, _ = reference.prefill(q, k, v, gc, beta, initial_state=S0, scale=0.5)
    for h in range(H):
        a = [Fraction(math.exp(min(max(float(x), LN_HALF), 0.0))) for x in g[:, h]]
        o_ex, st_ex = brute.exact_recurrence_scalar_gate(
            _exact(q[:, h]), _exact(k[:, h]), _exact(v[:, h]), a, [Fraction(float(b)) for b in beta[:, h]],
            S0=_exact(S0[0, h]), scale=Fraction(1, 2))
        o_ex = np.array([[float(x) for x in r] for r in o_ex])
        s_ex = np.array([[float(x) for x in r] for r in st_ex[-1]])
        assert np.abs(o[:, h] - o_ex).max() <= 1e-12 * max(1.0, np.abs(o_ex).max())
        assert np.abs(fin[0, h] - s_ex).max() <= 1e-12 * max(1.0, np.abs(s_ex).max())


def check_gdn_gate_is_per_head(var):
    g = np.arange(12, dtype=np.float32).reshape(4, 3) * -0.05          # [T=4, H=3]
    gc = var.gate_per_channel(g, var.GATE_HEAD, (4, 3, 5))
    assert gc.shape == (4, 3, 5)
    for t in range(4):
        for h in range(3):
            assert np.all(gc[t, h] == np.float64(g[t, h]))


def check_deltanet_is_ungated_delta_rule(var):
    rng = np.random.default_rng(37)
    T, H, Dk, Dv = 9, 1, 3, 4
    q, k, v, beta, S0 = _case(rng, T, H, Dk, Dv)
    gc = var.gate_per_channel(None, var.GATE_NONE, (T, H, Dk))
    o, fin, _ = reference.prefill(q, k, v, gc, beta, initial_state=S0)
    ones = [[Fraction(1)] * Dk for _ in range(T)]
    o_ex, st_ex = brute.exact_recurrence(_exact(q[:, 0]), _exact(k[:, 0]), _exact(v[:, 0]), ones,
                                         [Fraction(float(b)) for b in beta[:, 0]], S0=_exact(S0[0, 0]))
    o_ex = np.array([[float(x) for x in r] for r in o_ex])
    assert np.abs(o[:, 0] - o_ex).max() <= 1e-12 * max(1.0, np.abs(o_ex).max())
    # delta write-back with beta = 1: S_t^T k_t = v_t after every token, for
    # keys of exactly unit norm (entries +-1/2 over 4 channels)
    T, Dk = 9, 4
    kx = (0.5 * rng.choice([-1.0, 1.0], (T, 1, Dk))).astype(np.float32)
    qx = rng.standard_normal((T, 1, Dk)).astype(np.float32)
    gx = var.gate_per_channel(None, var.GATE_NONE, (T, 1, Dk))
    _, _, ck = reference.prefill(qx, kx, v, gx, np.ones((T, 1), np.float32), ckpt_interval=1)
    for t in range(T):
        assert np.allclose(ck[t, 0].T @ kx[t, 0].astype(np.float64), v[t, 0], rtol=0, atol=1e-12)


CHECKS = [check_gdn_matches_exact_scalar_gate, check_gdn_gate_is_per_head,
          check_deltanet_is_ungated_delta_rule]


@pytest.mark.parametrize("check", CHECKS, ids=lambda f: f.__name__)
def test_variant_pin(check):
    check(variants)
