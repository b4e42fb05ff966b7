"""Brute-force forms of the KDA recurrence, for pinning the C oracle.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

Two forms that share no code with kda_oracle.c:

* ``exact_recurrence``: the token recurrence in exact rational arithmetic
  (fractions.Fraction). Decays are given directly as rational alpha (so the
  gate is exact); the C oracle is fed g = log(alpha).
* ``transition_form``: the closed form obtained by unrolling the recurrence
  with dense D_k x D_k transition matrices
      A_t = (I - beta_t k_t k_t^T) Diag(alpha_t),
      S_t = A_t ... A_1 S_0 + sum_{i<=t} A_t ... A_{i+1} beta_i k_i v_i^T,
  recomputed from S_0 for every t (O(T^2 D^3), tiny inputs only).

The recurrence being pinned is the reading of [K3-SA, 배경/Background]
(delta rule + diagonal per-channel gate) stated in kda_oracle.c, where
[K3-SA] = "LLM - Semianalysis, Kimi K3 아키텍처".
"""
from fractions import Fraction

import numpy as np


def exact_recurrence(q, k, v, alpha, beta, S0=None, scale=Fraction(1)):
    """q, k, alpha: T lists of Dk Fractions; v: T lists of Dv Fractions;
    beta: T Fractions. Returns (o: T x Dv, states: T+1 states (Dk x Dv))."""
    T = len(k)
    Dk = len(k[0])
    Dv = len(v[0])
    S = [[Fraction(0)] * Dv for _ in range(Dk)] if S0 is None else [list(r) for r in S0]
    states = [[list(r) for r in S]]
    outs = []
    for t in range(T):
        S = [[alpha[t][c] * S[c][j] for j in range(Dv)] for c in range(Dk)]
        u = [sum(S[c][j] * k[t][c] for c in range(Dk)) for j in range(Dv)]
        d = [beta[t] * (v[t][j] - u[j]) for j in range(Dv)]
        S = [[S[c][j] + k[t][c] * d[j] for j in range(Dv)] for c in range(Dk)]
        outs.append([scale * sum(S[c][j] * q[t][c] for c in range(Dk)) for j in range(Dv)])
        states.append([list(r) for r in S])
    return outs, states


def transition_form(q, k, v, alpha, beta, S0=None, scale=1.0):
    """fp64 numpy; q,k,alpha: [T,Dk]; v: [T,Dv]; beta: [T]. Returns (o, S_T)."""
    q, k, v, alpha, beta = (np.asarray(x, np.float64) for x in (q, k, v, alpha, beta))
    T, Dk = k.shape
    Dv = v.shape[1]
    S0 = np.zeros((Dk, Dv)) if S0 is None else np.asarray(S0, np.float64)
    A = [(np.eye(Dk) - beta[t] * np.outer(k[t], k[t])) @ np.diag(alpha[t]) for t in range(T)]
    o = np.zeros((T, Dv))
    S_t = S0
    for t in range(T):
        # from scratch: S_t = (A_t..A_0) S0 + sum_i (A_t..A_{i+1}) beta_i k_i v_i^T
        M = np.eye(Dk)
        S_t = np.zeros((Dk, Dv))
        for i in range(t, -1, -1):
            S_t = S_t + M @ (beta[i] * np.outer(k[i], v[i]))
            M = M @ A[i]
        S_t = S_t + M @ S0
        o[t] = scale * (S_t.T @ q[t])
    return o, S_t


def exact_recurrence_scalar_gate(q, k, v, a, beta, S0=None, scale=Fraction(1)):
    """Gated DeltaNet in exact rational arithmetic, written the way that model
    is usually stated: erase and write first, with ONE decay a_t per token
    applied to the whole erased state ([K3-SA] "LLM - Semianalysis, Kimi K3
    아키텍처", Background: Gated DeltaNet puts an LSTM-style forget gate on the
    delta rule):
        S_t = a_t (S_{t-1} - beta_t k_t (k_t^T S_{t-1})) + beta_t k_t v_t^T.
    q, k: T lists of Dk Fractions; v: T lists of Dv Fractions; a, beta: T
    Fractions. Returns (o: T x Dv, states: T+1 states)."""
    T = len(k)
    Dk = len(k[0])
    Dv = len(v[0])
    S = [[Fraction(0)] * Dv for _ in range(Dk)] if S0 is None else [list(r) for r in S0]
    states = [[list(r) for r in S]]
    outs = []
    for t in range(T):
        kS = [sum(k[t][c] * S[c][j] for c in range(Dk)) for j in range(Dv)]
        S = [[a[t] * (S[c][j] - beta[t] * k[t][c] * kS[j]) + beta[t] * k[t][c] * v[t][j]
              for j in range(Dv)] for c in range(Dk)]
        outs.append([scale * sum(S[c][j] * q[t][c] for c in range(Dk)) for j in range(Dv)])
        states.append([list(r) for r in S])
    return outs, states
