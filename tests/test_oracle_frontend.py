"""Pins of the fp64 front-end oracle (oracle/frontend.py), CPU only.

Each check_* takes the front-end module as an argument, so that
test_oracle_mutations.py can rerun the checks on copies with planted mistakes.
The expected values are closed forms and hand-worked numbers:
  - L2 normalisation: (3, 4) -> (0.6, 0.8); with eps = 11, sqrt(25 + 11) = 6;
    rows of any scale come out unit-norm and pointing the same way.
  - gate: -softplus(0) = ln 1/2; the decay e^g equals 1 / (1 + e^a); logits
    a = ln(1/alpha - 1) give back g = ln alpha.
  - beta: sigmoid(0) = 1/2, sigmoid(ln 3) = 3/4, sigmoid(b) + sigmoid(-b) = 1.
"""
import math

import numpy as np
import pytest

from oracle import frontend, reference


def check_l2norm_worked_values(fe):
    x = np.zeros((2, 3, 2))                # [tokens, heads, channels]
    x[0, 0] = (3, 4)
    x[0, 1] = (-6, 8)
    x[0, 2] = (0, 5)
    x[1, 0] = (0.3, 0.4)
    x[1, 1] = (1, 0)
    x[1, 2] = (-2, 0)
    y = fe.l2_normalize(x, 0.0)
    want = np.array([[(0.6, 0.8), (-0.6, 0.8), (0, 1)], [(0.6, 0.8), (1, 0), (-1, 0)]])
    assert np.allclose(y, want, rtol=0, atol=1e-15)
    y = fe.l2_normalize(np.array([3.0, 4.0]), 11.0)
    assert np.allclose(y, [0.5, 4 / 6], rtol=0, atol=1e-15)
    y = fe.l2_normalize(np.ones(3), 1.0)
    assert np.allclose(y, [0.5, 0.5, 0.5], rtol=0, atol=1e-15)


def check_l2norm_unit_rows(fe):
    rng = np.random.default_rng(3)
    x = rng.standard_normal((7, 4, 16)) * rng.uniform(0.01, 100, (7, 4, 1))
    y = fe.l2_normalize(x, 0.0)
    assert np.allclose(np.linalg.norm(y, axis=-1), 1.0, rtol=0, atol=1e-14)
    # same direction: y . x = |x|
    assert np.allclose(np.sum(y * x, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-14, atol=0)


def check_gate_values(fe):
    assert fe.gate_from_logits(0.0) == pytest.approx(math.log(0.5), rel=0, abs=1e-16)
    a = np.linspace(-30, 30, 61)
    g = fe.gate_from_logits(a)
    assert np.all(g < 0)
    assert np.allclose(np.exp(g) * (1.0 + np.exp(a)), 1.0, rtol=0, atol=1e-14)
    alpha = np.array([0.5, 0.6, 0.75, 0.9, 0.99, 0.999999])
    # (1/alpha - 1 loses digits as alpha -> 1: about 1e-10 relative at alpha = 1 - 1e-6)
    assert np.allclose(fe.gate_from_logits(np.log(1.0 / alpha - 1.0)), np.log(alpha), rtol=1e-9, atol=0)
    assert fe.gate_from_logits(800.0) == pytest.approx(-800.0, rel=1e-15)   # no overflow
    assert -1e-300 < fe.gate_from_logits(-800.0) <= 0.0


def check_beta_values(fe):
    assert fe.beta_from_logits(0.0) == 0.5
    assert fe.beta_from_logits(math.log(3.0)) == pytest.approx(0.75, rel=0, abs=1e-16)
    assert fe.beta_from_logits(-math.log(3.0)) == pytest.approx(0.25, rel=0, abs=1e-16)
    b = np.linspace(-20, 20, 41)
    assert np.allclose(fe.beta_from_logits(b) + fe.beta_from_logits(-b), 1.0, rtol=0, atol=1e-15)
    assert fe.beta_from_logits(-800.0) == 0.0 and fe.beta_from_logits(800.0) == 1.0


def check_flags_are_independent(fe):
    rng = np.random.default_rng(5)
    q, k, g = (rng.standard_normal((3, 2, 8)) for _ in range(3))
    b = rng.standard_normal((3, 2))
    for flag, changed in ((fe.L2NORM_QK, (0, 1)), (fe.GATE_LOGITS, (2,)), (fe.BETA_LOGITS, (3,))):
        out = fe.apply(q, k, g, b, flag, eps=0.0)
        for i, (x, y) in enumerate(zip((q, k, g, b), out)):
            assert np.array_equal(x, y) == (i not in changed), (flag, i)
    out = fe.apply(q, k, g, b, 0)
    assert all(np.array_equal(x, y) for x, y in zip((q, k, g, b), out))


def check_front_end_then_recurrence(fe):
    """Raw inputs built from prepared ones (q, k scaled by arbitrary positive
    factors, logits inverted by hand) give the prepared inputs' recurrence."""
    rng = np.random.default_rng(9)
    T, H, D = 37, 2, 8
    qn = rng.standard_normal((T, H, D))
    qn /= np.linalg.norm(qn, axis=-1, keepdims=True)
    kn = rng.standard_normal((T, H, D))
    kn /= np.linalg.norm(kn, axis=-1, keepdims=True)
    v = rng.standard_normal((T, H, D))
    alpha = rng.uniform(0.5, 0.999, (T, H, D))
    beta = rng.uniform(0.05, 0.95, (T, H))
    q_raw = qn * rng.uniform(0.1, 10, (T, H, 1))
    k_raw = kn * rng.uniform(0.1, 10, (T, H, 1))
    a = np.log(1.0 / alpha - 1.0)
    b = np.log(beta / (1.0 - beta))
    q2, k2, g2, beta2 = fe.apply(q_raw, k_raw, a, b, fe.L2NORM_QK | fe.GATE_LOGITS | fe.BETA_LOGITS,
                                 eps=0.0)
    o_ref, s_ref, _ = reference.prefill(qn, kn, v, np.log(alpha), beta)
    o, s, _ = reference.prefill(q2, k2, v, g2, beta2)
    assert np.allclose(o, o_ref, rtol=0, atol=1e-5 * np.abs(o_ref).max())
    assert np.allclose(s, s_ref, rtol=0, atol=1e-5 * np.abs(s_ref).max())


CHECKS = [check_l2norm_worked_values, check_l2norm_unit_rows, check_gate_values, check_beta_values,
          check_flags_are_independent, check_front_end_then_recurrence]


@pytest.mark.parametrize("check", CHECKS, ids=lambda f: f.__name__)
def test_front_end_pin(check):
    check(frontend)
