"""Gate layouts of the delta-rule family, mapped onto the per-channel KDA gate:
TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

[K3-SA] "LLM - Semianalysis, Kimi K3 아키텍처", Background, describes the line:
  - DeltaNet: the delta rule, with no decay;
  - Gated DeltaNet (GDN): one forget gate per token (an LSTM-style scalar);
  - KDA: the gate becomes a diagonal, one decay per key channel.
A scalar decay a commutes with the erase step, so
a (I - beta k k^T) S = (I - beta k k^T) Diag(a, ..., a) S. GDN is therefore KDA
with every key channel given the same log-decay, and DeltaNet is KDA with
g = 0. The same floor [g_min, 0] applies to the scalar log-decay. The names
match the C ABI's kda_gate values.
"""
import numpy as np

GATE_CHANNEL = 0   # g [.., H, Dk]: KDA
GATE_HEAD = 1      # g [.., H]: Gated DeltaNet
GATE_NONE = 2      # no g: DeltaNet


def gate_per_channel(g, kind, shape):
    """The per-channel log-decay [.., H, Dk] (shape) that a gate of `kind` means."""
    if kind == GATE_CHANNEL:
        return np.asarray(g, dtype=np.float64)
    if kind == GATE_HEAD:
        return np.broadcast_to(np.asarray(g, dtype=np.float64)[..., None], shape).copy()
    if kind == GATE_NONE:
        return np.zeros(shape)
    raise ValueError(kind)
