"""Seeded synthetic inputs for the KDA workloads.

This module holds only input generation (shapes, distributions, seeds); it
contains none of the operator's arithmetic. Both the oracle-side tests and the
device path draw their inputs from here.

Recipe (all draws from numpy ``default_rng(seed)``, in this order: q, k, v,
beta-logits, g-logits, initial state, lengths):
  q, k  ~ N(0, 1) in fp32, L2-normalised per (token, head) in fp32, then
        rounded to bf16 (round-to-nearest-even) unless the workload is fp32;
  v     ~ N(0, 1), rounded to bf16 likewise;
  beta  = sigmoid(N(0, 1)) in fp32;
  g     = -softplus(N(0, 1)) clamped to [ln 0.5, 0] in fp32 (per key channel);
  S0    ~ N(0, 0.02^2) in fp32 where the workload starts from cached states;
  lengths (packed variable-length workload): lognormal(ln 4096, sigma=1),
        rounded, clipped to [1, 32768].
Values are returned as float32 arrays that hold the exact device values
(bf16 values are exactly representable in fp32).
"""
from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np

LN_HALF = float(np.log(0.5))


@dataclass
class Workload:
    name: str
    H: int
    D: int
    lengths: List[int]          # per-sequence token counts (decode: 1 each)
    bf16: bool = True
    initial_state: bool = False
    ckpt_interval: int = 0
    decode: bool = False
    seed: int = 0
    note: str = ""

    @property
    def num_seqs(self):
        return len(self.lengths)

    @property
    def total_tokens(self):
        return int(sum(self.lengths))


def varlen_lengths(n=16, seed=5, median=4096, sigma=1.0, lo=1, hi=32768):
    rng = np.random.default_rng(seed + 1000)
    L = np.rint(rng.lognormal(np.log(median), sigma, size=n)).astype(np.int64)
    return [int(x) for x in np.clip(L, lo, hi)]


def workload(cfg: int) -> Workload:
    """The five workloads by number (1..5)."""
    if cfg == 1:
        return Workload("tiny: B=1 H=2 T=64 D=16 fp32", H=2, D=16, lengths=[64], bf16=False, seed=1)
    if cfg == 2:
        return Workload("prefill: B=1 H=32 T=8192 D=128 bf16", H=32, D=128, lengths=[8192], seed=2)
    if cfg == 3:
        return Workload("decode: 256 seqs x H=32 D=128, one token", H=32, D=128, lengths=[1] * 256,
                        initial_state=True, decode=True, seed=3)
    if cfg == 4:
        return Workload("long prefill: B=1 H=32 T=131072 D=128, checkpoint every 32768", H=32, D=128,
                        lengths=[131072], ckpt_interval=32768, seed=4)
    if cfg == 5:
        return Workload("append-prefill: 16 packed varlen seqs, H=32 D=128, cached initial states", H=32,
                        D=128, lengths=varlen_lengths(), initial_state=True, seed=5)
    raise ValueError(cfg)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round fp32 to the nearest bf16 (ties to even); returns fp32 values."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    b = x.view(np.uint32).astype(np.uint64)
    b = ((b + 0x7FFF + ((b >> 16) & 1)) >> 16) << 16
    return b.astype(np.uint32).view(np.float32)


def _l2n(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True).astype(np.float32)


@dataclass
class Inputs:
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    g: np.ndarray
    beta: np.ndarray
    cu_seqlens: np.ndarray
    initial_state: Optional[np.ndarray] = None
    extra: dict = field(default_factory=dict)


def make_inputs(T, H, Dk, Dv=None, seed=0, bf16=True, num_seqs=None, lengths=None,
                initial_state=False, g_scale=1.0, raw=False) -> Inputs:
    """Packed inputs [T, H, D]; ``lengths`` (or one sequence) sets cu_seqlens.

    raw=True returns the same draws before the front-end step: q and k as
    drawn (not normalised), g and beta as the N(0, 1) logits."""
    Dv = Dk if Dv is None else Dv
    rng = np.random.default_rng(seed)
    if lengths is None:
        lengths = [T] if num_seqs is None else None
    assert lengths is not None and sum(lengths) == T
    norm = (lambda x: x) if raw else _l2n
    q = norm(rng.standard_normal((T, H, Dk), dtype=np.float32))
    k = norm(rng.standard_normal((T, H, Dk), dtype=np.float32))
    v = rng.standard_normal((T, H, Dv), dtype=np.float32)
    if bf16:
        q, k, v = bf16_round(q), bf16_round(k), bf16_round(v)
    bl = rng.standard_normal((T, H), dtype=np.float32)
    beta = bl if raw else (1.0 / (1.0 + np.exp(-bl))).astype(np.float32)
    gl = rng.standard_normal((T, H, Dk), dtype=np.float32)
    if raw:
        g = gl
    else:
        g = np.clip(-np.logaddexp(np.float32(0), gl), np.float32(LN_HALF), np.float32(0)).astype(np.float32)
    if g_scale != 1.0:
        g = (g * np.float32(g_scale)).astype(np.float32)
    s0 = None
    if initial_state:
        s0 = (0.02 * rng.standard_normal((len(lengths), H, Dk, Dv), dtype=np.float32)).astype(np.float32)
    cu = np.zeros(len(lengths) + 1, np.int64)
    cu[1:] = np.cumsum(lengths)
    return Inputs(q, k, v, g, beta, cu, s0)


def workload_inputs(w: Workload) -> Inputs:
    return make_inputs(w.total_tokens, w.H, w.D, seed=w.seed, bf16=w.bf16, lengths=w.lengths,
                       initial_state=w.initial_state)


def make_inputs_device(T, H, D, seed, device, lengths=None, initial_state=False, bf16=True, raw=False):
    """Same recipe as make_inputs, drawn with a seeded torch generator on the
    device (for the large workloads, where host generation would dominate).
    Returns torch tensors: q, k, v (bf16 or fp32), g, beta (fp32), cu (int32,
    host), s0 (fp32 or None). raw=True as in make_inputs."""
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    lengths = [T] if lengths is None else list(lengths)
    assert sum(lengths) == T

    def normal(*shape):
        return torch.randn(*shape, generator=gen, device=device, dtype=torch.float32)

    q = normal(T, H, D)
    k = normal(T, H, D)
    if not raw:
        q = q / q.norm(dim=-1, keepdim=True)
        k = k / k.norm(dim=-1, keepdim=True)
    v = normal(T, H, D)
    dt = torch.bfloat16 if bf16 else torch.float32
    q, k, v = q.to(dt), k.to(dt), v.to(dt)
    beta = normal(T, H)
    g = normal(T, H, D)
    if not raw:
        beta = torch.sigmoid(beta)
        g = (-torch.nn.functional.softplus(g)).clamp_(min=LN_HALF, max=0.0)
    s0 = 0.02 * normal(len(lengths), H, D, D) if initial_state else None
    cu = torch.zeros(len(lengths) + 1, dtype=torch.int32)
    cu[1:] = torch.cumsum(torch.tensor(lengths, dtype=torch.int64), 0).to(torch.int32)
    return q, k, v, g, beta, cu, s0
