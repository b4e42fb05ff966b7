"""fp64 reference of the optional KDA front end: TEST INFRASTRUCTURE ONLY
(see oracle/__init__.py).

The front end is the step just before the recurrence. It turns raw
projections into the operator's inputs. Each part is switched on by its own
flag, with the same names as the C ABI's KDA_FE_* flags:

  L2NORM_QK    keys and queries are unit-norm rows ([K3-SA] "LLM - Semianalysis,
               Kimi K3 아키텍처", Background: the delta rule is a gradient step
               on the L2 value-retrieval loss, stated for normalised keys).
               Row x becomes x / sqrt(sum_i x_i^2 + eps). The pages give no
               epsilon; it is a parameter here.
  GATE_LOGITS  the per-channel log-decay comes from a raw logit a as
               g = -softplus(a) = -ln(1 + e^a). The decay e^g = 1 / (1 + e^a)
               then lies in (0, 1). The floor at g_min
               ([K3-DD] "MoonshotAI/Kimi-K3 딥다이브", 4-1 KDA, first bullet) is
               applied afterwards by the recurrence, as for any g.
  BETA_LOGITS  the write strength comes from a raw logit b as
               beta = sigmoid(b) = 1 / (1 + e^-b).

Everything is fp64 numpy, one formula per step, applied row by row. The
results feed oracle.reference, which takes them as float32. That rounding is
one part in 2^24, far inside every parity tolerance.
"""
import numpy as np

L2NORM_QK = 1
GATE_LOGITS = 2
BETA_LOGITS = 4


def l2_normalize(x, eps):
    """x / sqrt(sum over the last axis of x^2 + eps), in fp64."""
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + float(eps))


def gate_from_logits(a):
    """g = -softplus(a) = -ln(1 + e^a), in fp64 (logaddexp(0, a) = ln(e^0 + e^a))."""
    return -np.logaddexp(0.0, np.asarray(a, dtype=np.float64))


def beta_from_logits(b):
    """beta = 1 / (1 + e^-b), in fp64."""
    b = np.asarray(b, dtype=np.float64)
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-b))


def apply(q, k, g, beta, flags, eps=1e-6):
    """The operator's (q, k, g, beta) from the raw ones under `flags`.
    Inputs that no flag names are returned unchanged (as fp64)."""
    q, k, g, beta = (np.asarray(x, dtype=np.float64) for x in (q, k, g, beta))
    if flags & L2NORM_QK:
        q, k = l2_normalize(q, eps), l2_normalize(k, eps)
    if flags & GATE_LOGITS:
        g = gate_from_logits(g)
    if flags & BETA_LOGITS:
        beta = beta_from_logits(beta)
    return q, k, g, beta
