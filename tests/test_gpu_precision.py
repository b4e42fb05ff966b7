"""GPU parity in the precision-sensitive regimes, through the C ABI against
the fp64 oracle, every (sequence, head) compared:

  - slow decay: gates scaled towards 1 (g x 0, 1/64, 1/256, and a mix of
    slow and fast channels) over 8192 tokens, KDA and Gated DeltaNet layouts,
    and a varlen case with checkpoints and cached states. With alpha near 1
    the state is long lived and K~+ S nearly cancels V, the case where bf16
    rounding of the state or of the decayed keys would show;
  - gates outside [g_min, 0] (both signs, far below the floor), which every
    entry point clamps on load;
  - decay floors below ln 1/2 with half the channels on the floor;
  - seeded sweeps over lengths, heads, head size, storage type, gate layout,
    checkpoint interval, initial states, gate scale, floors, segments and
    record windows, and over decode calls (sequences, tokens, accept
    lengths, unclamped gates, floors). KDA_SWEEP_EXTRA=n adds n more seeds
    to every sweep (indices from 1000 on).

Tolerances as in test_gpu_parity.py: outputs 2e-2 and fp32 states 1e-3,
relative to the largest reference value per (sequence, head).
"""
import os

import numpy as np
import pytest
import torch

from gated_delta_rule_109_amd import kda
from gated_delta_rule_109_amd.workloads import LN_HALF, make_inputs, make_inputs_device
from oracle import reference
from oracle import variants as var_oracle
from test_gpu_parity import DEV, O_TOL, check_outputs, check_states, rel_err, to_dev

pytestmark = pytest.mark.gpu

GATE_VALUES = np.array([-5.0, -1.0, -0.3, 0.0, 0.375], np.float32)
SWEEP_EXTRA = int(os.environ.get("KDA_SWEEP_EXTRA", "0"))


def _seeds(n):
    """Sweep indices: the first n, plus KDA_SWEEP_EXTRA more from 1000 on."""
    return list(range(n)) + list(range(1000, 1000 + SWEEP_EXTRA))


def _options(gate):
    return None if gate == kda.GATE_CHANNEL else kda.Options(gate=gate)


def _gate_arg(g, gate):
    """The g argument for a gate layout, from a per-channel draw [.., H, D]."""
    if gate == kda.GATE_CHANNEL:
        return g
    if gate == kda.GATE_HEAD:
        return g[..., 0].contiguous() if torch.is_tensor(g) else np.ascontiguousarray(g[..., 0])
    return None


def _host(t):
    return None if t is None else t.float().cpu().numpy()


# ------------------------------------------------------------ slow decay
@pytest.mark.parametrize("gate,g_scale", [(gate, sc) for gate in (kda.GATE_CHANNEL, kda.GATE_HEAD)
                                          for sc in (0.0, 1.0 / 64, 1.0 / 256)]
                         + [(kda.GATE_CHANNEL, "mixed")])
def test_slow_decay_8192_tokens(gate, g_scale):
    """T=8192, 4 heads, D=128; every head against the oracle."""
    T, H, D = 8192, 4, 128
    print(f"case: slow decay gate={gate} g_scale={g_scale}", flush=True)
    q, k, v, g, beta, cu, _ = make_inputs_device(T, H, D, seed=201, device=DEV)
    if g_scale == "mixed":
        # per-channel gates: some channels forget fast, others barely at all
        sc = torch.ones(D, device=DEV)
        sc[D // 2:] = 1.0 / 256
        sc[D // 4: D // 2] = 0.0
        g = g * sc
    else:
        g = g * g_scale
    gv = _gate_arg(g, gate)
    o, fin, _ = kda.prefill(q, k, v, gv, beta, cu_seqlens=cu, options=_options(gate))
    torch.cuda.synchronize()
    gc = var_oracle.gate_per_channel(_host(gv), gate, (T, H, D))
    o_ref, f_ref, _ = reference.prefill(_host(q), _host(k), _host(v), gc, _host(beta), cu_seqlens=cu.numpy())
    check_outputs(_host(o), o_ref, cu.numpy(), H)
    check_states(fin.cpu().numpy(), f_ref, "final")


@pytest.mark.parametrize("gate,g_scale", [(kda.GATE_CHANNEL, 1.0 / 64), (kda.GATE_HEAD, 1.0 / 256),
                                          (kda.GATE_CHANNEL, 0.0)])
def test_slow_decay_varlen_with_checkpoints(gate, g_scale):
    """Packed sequences with cached initial states and a checkpoint every 512
    tokens, gates near 1."""
    lengths = [3000, 17, 0, 5000, 190, 33]
    H, D = 3, 128
    print(f"case: slow decay varlen gate={gate} g_scale={g_scale}", flush=True)
    inp = make_inputs(sum(lengths), H, D, seed=211 + gate, lengths=lengths, initial_state=True,
                      g_scale=g_scale)
    gv = _gate_arg(inp.g, gate)
    o, fin, ck = kda.prefill(to_dev(inp.q, torch.bfloat16), to_dev(inp.k, torch.bfloat16),
                             to_dev(inp.v, torch.bfloat16), None if gv is None else to_dev(gv),
                             to_dev(inp.beta), cu_seqlens=inp.cu_seqlens,
                             initial_state=to_dev(inp.initial_state), ckpt_interval=512,
                             options=_options(gate))
    torch.cuda.synchronize()
    gc = var_oracle.gate_per_channel(gv, gate, inp.q.shape)
    o_ref, f_ref, ck_ref = reference.prefill(inp.q, inp.k, inp.v, gc, inp.beta, cu_seqlens=inp.cu_seqlens,
                                             initial_state=inp.initial_state, ckpt_interval=512)
    check_outputs(_host(o), o_ref, inp.cu_seqlens, H)
    check_states(fin.cpu().numpy(), f_ref, "final")
    assert ck.shape == ck_ref.shape == (sum(L // 512 for L in lengths), H, D, D)
    check_states(ck.cpu().numpy(), ck_ref, "checkpoint")


# ------------------------------------------------------------ gates outside [g_min, 0]
def _wild_gates(shape, seed):
    rng = np.random.default_rng(seed)
    return GATE_VALUES[rng.integers(0, len(GATE_VALUES), size=shape)]


@pytest.mark.parametrize("D", [128, 16])
@pytest.mark.parametrize("g_min", [LN_HALF, -2.5, -5.0])
def test_prefill_unclamped_gates(D, g_min):
    """g drawn from {-5, -1, -0.3, 0, 0.375}: the kernel clamps to [g_min, 0]
    on load, as the oracle does."""
    lengths = [70, 33, 1, 64]
    H = 2
    print(f"case: prefill unclamped gates D={D} g_min={g_min:.4f}", flush=True)
    inp = make_inputs(sum(lengths), H, D, seed=221 + D, lengths=lengths, initial_state=True)
    g = _wild_gates(inp.g.shape, 222 + D)
    o, fin, ck = kda.prefill(to_dev(inp.q, torch.bfloat16), to_dev(inp.k, torch.bfloat16),
                             to_dev(inp.v, torch.bfloat16), to_dev(g), to_dev(inp.beta),
                             cu_seqlens=inp.cu_seqlens, initial_state=to_dev(inp.initial_state),
                             g_min=g_min, ckpt_interval=16)
    torch.cuda.synchronize()
    o_ref, f_ref, ck_ref = reference.prefill(inp.q, inp.k, inp.v, g, inp.beta, cu_seqlens=inp.cu_seqlens,
                                             initial_state=inp.initial_state, g_min=g_min, ckpt_interval=16)
    check_outputs(_host(o), o_ref, inp.cu_seqlens, H)
    check_states(fin.cpu().numpy(), f_ref, "final")
    check_states(ck.cpu().numpy(), ck_ref, "checkpoint")


@pytest.mark.parametrize("D", [128, 16])
@pytest.mark.parametrize("g_min", [LN_HALF, -1.5, -10.0])
def test_decode_step_unclamped_gates(D, g_min):
    N, H = 7, 3
    print(f"case: decode_step unclamped gates D={D} g_min={g_min}", flush=True)
    d = make_inputs(N, H, D, seed=231 + D, lengths=[1] * N, initial_state=True)
    g = _wild_gates(d.g.shape, 232 + D)
    state = to_dev(d.initial_state)
    o = kda.decode_step(to_dev(d.q, torch.bfloat16), to_dev(d.k, torch.bfloat16), to_dev(d.v, torch.bfloat16),
                        to_dev(g), to_dev(d.beta), state, g_min=g_min)
    torch.cuda.synchronize()
    o_ref, s_ref = reference.decode(d.q, d.k, d.v, g, d.beta, d.initial_state, g_min=g_min)
    o = _host(o)
    for idx in np.ndindex(N, H):
        assert rel_err(o[idx], o_ref[idx]) <= O_TOL, idx
    check_states(state.cpu().numpy(), s_ref, "state")


@pytest.mark.parametrize("D", [128, 16])
@pytest.mark.parametrize("g_min", [LN_HALF, -1.5, -10.0])
def test_decode_tokens_unclamped_gates(D, g_min):
    N, T, H = 5, 4, 2
    print(f"case: decode_tokens unclamped gates D={D} g_min={g_min}", flush=True)
    d = make_inputs(N * T, H, D, seed=241 + D, lengths=[T] * N, initial_state=True)
    shp = lambda a: np.ascontiguousarray(a.reshape(N, T, *a.shape[1:]))
    q, k, v, beta = map(shp, (d.q, d.k, d.v, d.beta))
    g = _wild_gates((N, T, H, D), 242 + D)
    accept = [T, 0, 2, 1, 3]
    state = to_dev(d.initial_state)
    o = kda.decode_tokens(to_dev(q, torch.bfloat16), to_dev(k, torch.bfloat16), to_dev(v, torch.bfloat16),
                          to_dev(g), to_dev(beta), state,
                          accept=torch.tensor(accept, dtype=torch.int32, device=DEV), g_min=g_min)
    torch.cuda.synchronize()
    o, S = _host(o), state.cpu().numpy()
    st = d.initial_state.astype(np.float64)
    for t in range(T):
        o_t, st_next = reference.decode(q[:, t], k[:, t], v[:, t], g[:, t], beta[:, t], st, g_min=g_min)
        for n, h in np.ndindex(N, H):
            assert rel_err(o[n, t, h], o_t[n, h]) <= O_TOL, (n, t, h)
        for n in range(N):
            if accept[n] == t + 1:
                check_states(S[n:n + 1], st_next[n:n + 1], f"seq {n}")
        st = st_next
    for n in range(N):
        if accept[n] == 0:
            assert np.array_equal(S[n], d.initial_state[n])


# ------------------------------------------------------------ decay floors below ln 1/2
@pytest.mark.parametrize("D", [128, 16])
@pytest.mark.parametrize("g_min", [-5.0, -4.0, -2.5, -1.5])
def test_prefill_low_decay_floor(D, g_min):
    """Half the key channels sit on the floor g_min (alpha = e^g_min every
    token), the others draw -softplus(N(0, 1)) down to g_min: varlen, cached
    states, checkpoints inside and at the end of blocks."""
    lengths = [100, 37, 64, 0, 161]
    H = 2
    print(f"case: prefill decay floor g_min={g_min} D={D}", flush=True)
    inp = make_inputs(sum(lengths), H, D, seed=251 + D, lengths=lengths, initial_state=True)
    rng = np.random.default_rng(252 + D)
    g = (-np.logaddexp(0.0, rng.standard_normal(inp.g.shape))).astype(np.float32)
    g[..., ::2] = -5.0
    o, fin, ck = kda.prefill(to_dev(inp.q, torch.bfloat16), to_dev(inp.k, torch.bfloat16),
                             to_dev(inp.v, torch.bfloat16), to_dev(g), to_dev(inp.beta),
                             cu_seqlens=inp.cu_seqlens, initial_state=to_dev(inp.initial_state),
                             g_min=g_min, ckpt_interval=48)
    torch.cuda.synchronize()
    o_ref, f_ref, ck_ref = reference.prefill(inp.q, inp.k, inp.v, g, inp.beta, cu_seqlens=inp.cu_seqlens,
                                             initial_state=inp.initial_state, g_min=g_min, ckpt_interval=48)
    check_outputs(_host(o), o_ref, inp.cu_seqlens, H)
    check_states(fin.cpu().numpy(), f_ref, "final")
    check_states(ck.cpu().numpy(), ck_ref, "checkpoint")


@pytest.mark.parametrize("D", [128, 16])
@pytest.mark.parametrize("g_min", [-5.0, -2.5])
def test_prefill_floor_in_one_chunk_only(D, g_min):
    """Decay at the floor in one 16-token chunk of every block and none in the
    other (per channel, both orders), so the two chunks' decays differ by up
    to exp(16 g_min): the A and L tiles between the chunks and the checkpoints
    after a block's first chunk. Varlen with cached states and a checkpoint
    every 16 tokens."""
    lengths = [96, 45, 0, 130]
    H = 2
    print(f"case: prefill floor in one chunk g_min={g_min} D={D}", flush=True)
    inp = make_inputs(sum(lengths), H, D, seed=261 + D, lengths=lengths, initial_state=True)
    g = np.zeros_like(inp.g)
    cu = inp.cu_seqlens
    for n in range(len(lengths)):
        t = np.arange(cu[n + 1] - cu[n])
        first = (t % 32) < 16            # a block's first chunk (blocks start at each sequence's start)
        g[cu[n]:cu[n + 1], :, 0::2] = np.where(first, g_min, 0.0)[:, None, None]
        g[cu[n]:cu[n + 1], :, 1::2] = np.where(first, 0.0, g_min)[:, None, None]
    g = g.astype(np.float32)
    o, fin, ck = kda.prefill(to_dev(inp.q, torch.bfloat16), to_dev(inp.k, torch.bfloat16),
                             to_dev(inp.v, torch.bfloat16), to_dev(g), to_dev(inp.beta),
                             cu_seqlens=inp.cu_seqlens, initial_state=to_dev(inp.initial_state),
                             g_min=g_min, ckpt_interval=16)
    torch.cuda.synchronize()
    o_ref, f_ref, ck_ref = reference.prefill(inp.q, inp.k, inp.v, g, inp.beta, cu_seqlens=inp.cu_seqlens,
                                             initial_state=inp.initial_state, g_min=g_min, ckpt_interval=16)
    check_outputs(_host(o), o_ref, inp.cu_seqlens, H)
    check_states(fin.cpu().numpy(), f_ref, "final")
    check_states(ck.cpu().numpy(), ck_ref, "checkpoint")


# ------------------------------------------------------------ seeded sweep
def _sweep_case(i):
    rng = np.random.default_rng(3000 + i)
    N = int(rng.integers(1, 6))
    lengths = [int(x) for x in rng.choice([0, 1, 15, 16, 17, 31, 32, 33, 64, 95, 130, 257, 400], size=N)]
    if sum(lengths) == 0:
        lengths[0] = 45
    H, D = int(rng.integers(1, 4)), int(rng.choice([16, 128]))
    segments = int(rng.choice([0, 0, 1, 3]))
    if segments > 1 and N * H * (D // 16) > kda.SEGMENT_SLICE_LIMIT:
        segments = 0     # forcing segments needs few (sequence, head, 16-column) slices
    return dict(
        lengths=lengths,
        H=H,
        D=D,
        bf16=bool(rng.integers(0, 2)),
        gate=int(rng.choice([kda.GATE_CHANNEL, kda.GATE_CHANNEL, kda.GATE_HEAD, kda.GATE_NONE])),
        ckpt=int(rng.choice([0, 16, 32, 48, 64, 96])),
        initial=bool(rng.integers(0, 2)),
        g_scale=float(rng.choice([1.0, 1.0 / 16, 1.0 / 256])),
        g_min=float(rng.choice([LN_HALF, LN_HALF, -1.5, -2.5, -5.0])),
        segments=segments,
        scale=float(rng.choice([1.0, 0.5])),
    )


def _sweep_case_many_slices(i):
    """Many sequence-head pairs at D = 128 (usually more 16-column slices than
    compute units, so the chain runs two slices per workgroup)."""
    rng = np.random.default_rng(5000 + i)
    c = _sweep_case(100 + i)
    N, H = int(rng.integers(8, 25)), int(rng.integers(4, 9))
    c["lengths"] = [int(x) for x in rng.choice([0, 1, 15, 16, 17, 31, 32, 33, 64, 95, 130, 257], size=N)]
    if sum(c["lengths"]) == 0:
        c["lengths"][0] = 45
    c.update(H=H, D=128, segments=0)
    return c


def _sweep_case_windows(i):
    """Record windows of 1 to 8 blocks (a workspace sized for them), with
    sequences long enough to span several windows."""
    rng = np.random.default_rng(7000 + i)
    c = _sweep_case(200 + i)
    N = int(rng.integers(1, 5))
    c["lengths"] = [int(x) for x in rng.choice([0, 1, 17, 33, 95, 130, 257, 400, 700], size=N)]
    if sum(c["lengths"]) == 0:
        c["lengths"][0] = 300
    c["window"] = int(rng.choice([1, 2, 3, 5, 8]))
    if c["segments"] > 1 and N * c["H"] * (c["D"] // 16) > kda.SEGMENT_SLICE_LIMIT:
        c["segments"] = 0    # the new sequence count must still allow forced segments
    return c


def _sweep_case_large(i):
    """Up to 40 sequences of lognormal lengths (median 200 tokens, up to
    3000, some empty), up to 8 heads, with floors down to -5, segments and
    record windows of 1 to 64 blocks drawn independently."""
    rng = np.random.default_rng(9000 + i)
    N = int(rng.integers(1, 41))
    lengths = [int(x) for x in np.clip(np.round(rng.lognormal(np.log(200), 1.2, size=N)), 0, 3000)]
    lengths = [0 if rng.random() < 0.1 else x for x in lengths]
    if sum(lengths) == 0:
        lengths[0] = 77
    H, D = int(rng.integers(1, 9)), int(rng.choice([16, 128, 128]))
    segments = int(rng.choice([0, 0, 0, 1, 2, 4]))
    if segments > 1 and N * H * (D // 16) > kda.SEGMENT_SLICE_LIMIT:
        segments = 0
    return dict(
        lengths=lengths,
        H=H,
        D=D,
        bf16=bool(rng.integers(0, 2)),
        gate=int(rng.choice([kda.GATE_CHANNEL, kda.GATE_CHANNEL, kda.GATE_HEAD, kda.GATE_NONE])),
        ckpt=int(rng.choice([0, 16, 32, 48, 80, 256])),
        initial=bool(rng.integers(0, 2)),
        g_scale=float(rng.choice([1.0, 1.0 / 16, 1.0 / 256])),
        g_min=float(rng.choice([LN_HALF, LN_HALF, -1.0, -2.5, -3.0, -5.0])),
        segments=segments,
        scale=float(rng.choice([1.0, 0.5])),
        window=int(rng.choice([0, 0, 1, 4, 16, 64])),
    )


def _run_sweep_case(seed, c):
    """One sweep case through kda_prefill_chunked_ex against the oracle (with
    a workspace for record windows of c["window"] blocks, if given)."""
    lengths, H, D = c["lengths"], c["H"], c["D"]
    inp = make_inputs(sum(lengths), H, D, seed=seed, lengths=lengths, initial_state=c["initial"],
                      bf16=c["bf16"], g_scale=c["g_scale"])
    g = inp.g
    if c["g_min"] < LN_HALF:     # gates reaching the lower floor
        g = (g * np.float32(-c["g_min"] / -LN_HALF)).astype(np.float32)
    gv = _gate_arg(g, c["gate"])
    dt = torch.bfloat16 if c["bf16"] else torch.float32
    opt = kda.Options(gate=c["gate"], segments=c["segments"])
    plan = None
    if c.get("window"):
        plan = kda.make_plan(inp.cu_seqlens, H, D, DEV, c["ckpt"], window_blocks=c["window"])
    o, fin, ck = kda.prefill(to_dev(inp.q, dt), to_dev(inp.k, dt), to_dev(inp.v, dt),
                             None if gv is None else to_dev(gv), to_dev(inp.beta), cu_seqlens=inp.cu_seqlens,
                             initial_state=None if inp.initial_state is None else to_dev(inp.initial_state),
                             scale=c["scale"], g_min=c["g_min"], ckpt_interval=c["ckpt"], options=opt, plan=plan)
    torch.cuda.synchronize()
    gc = var_oracle.gate_per_channel(gv, c["gate"], inp.q.shape)
    o_ref, f_ref, ck_ref = reference.prefill(inp.q, inp.k, inp.v, gc, inp.beta, cu_seqlens=inp.cu_seqlens,
                                             initial_state=inp.initial_state, scale=c["scale"],
                                             g_min=c["g_min"], ckpt_interval=c["ckpt"])
    check_outputs(_host(o), o_ref, inp.cu_seqlens, H)
    check_states(fin.cpu().numpy(), f_ref, "final")
    if c["ckpt"]:
        assert ck is None and len(ck_ref) == 0 or ck.shape == ck_ref.shape
        if ck is not None:
            check_states(ck.cpu().numpy(), ck_ref, "checkpoint")


@pytest.mark.parametrize("i", _seeds(20))
def test_seeded_sweep(i):
    c = _sweep_case(i)
    print(f"case: sweep {i} {c}", flush=True)
    _run_sweep_case(4000 + i, c)


@pytest.mark.parametrize("i", _seeds(8))
def test_seeded_sweep_many_slices(i):
    c = _sweep_case_many_slices(i)
    print(f"case: sweep (many slices) {i} N={len(c['lengths'])} {c}", flush=True)
    _run_sweep_case(4100 + i, c)


@pytest.mark.parametrize("i", _seeds(10))
def test_seeded_sweep_record_windows(i):
    c = _sweep_case_windows(i)
    print(f"case: sweep (record windows) {i} {c}", flush=True)
    _run_sweep_case(4200 + i, c)


@pytest.mark.parametrize("i", _seeds(6))
def test_seeded_sweep_large(i):
    c = _sweep_case_large(i)
    print(f"case: sweep (large) {i} N={len(c['lengths'])} tokens={sum(c['lengths'])} {c}", flush=True)
    _run_sweep_case(4300 + i, c)


def _decode_case(i):
    rng = np.random.default_rng(6000 + i)
    N, H = int(rng.integers(1, 300)), int(rng.integers(1, 9))
    T = 1 if rng.random() < 0.25 else int(rng.integers(2, 17))
    return dict(N=N, T=T, H=H, D=int(rng.choice([16, 128])), bf16=bool(rng.integers(0, 2)),
                g_min=float(rng.choice([LN_HALF, -1.0, -2.5, -5.0, -8.0])),
                step=bool(T == 1 and rng.random() < 0.5), unclamped=bool(rng.random() < 0.5),
                accept=bool(rng.random() < 0.6), seed=int(rng.integers(0, 1 << 30)))


@pytest.mark.parametrize("i", _seeds(12))
def test_seeded_decode_sweep(i):
    """decode_step (T = 1) or decode_tokens against T oracle token steps:
    every output, and the committed state after accept[n] tokens (accept
    drawn from [-2, T + 2], clamped to [0, T] by the entry point)."""
    c = _decode_case(i)
    print(f"case: decode sweep {i} {c}", flush=True)
    N, T, H, D = c["N"], c["T"], c["H"], c["D"]
    rng = np.random.default_rng(c["seed"])
    d = make_inputs(N * T, H, D, seed=6500 + i, lengths=[T] * N, initial_state=True, bf16=c["bf16"])
    g = d.g
    if c["unclamped"]:
        g = rng.choice(np.append(GATE_VALUES, np.float32(-9.0)), size=g.shape).astype(np.float32)
    shp = lambda a: np.ascontiguousarray(a.reshape(N, T, *a.shape[1:]))
    q, k, v, g, beta = map(shp, (d.q, d.k, d.v, g, d.beta))
    states = [d.initial_state.astype(np.float64)]
    o_ref = np.zeros((N, T, H, D))
    for t in range(T):
        o_ref[:, t], st = reference.decode(q[:, t], k[:, t], v[:, t], g[:, t], beta[:, t], states[-1],
                                           scale=0.5, g_min=c["g_min"])
        states.append(st)
    dt = torch.bfloat16 if c["bf16"] else torch.float32
    state = to_dev(d.initial_state)
    accept = rng.integers(-2, T + 3, size=N).astype(np.int32) if c["accept"] and not c["step"] else None
    if c["step"]:
        o = kda.decode_step(to_dev(q[:, 0], dt), to_dev(k[:, 0], dt), to_dev(v[:, 0], dt), to_dev(g[:, 0]),
                            to_dev(beta[:, 0]), state, scale=0.5, g_min=c["g_min"])[:, None]
    else:
        o = kda.decode_tokens(to_dev(q, dt), to_dev(k, dt), to_dev(v, dt), to_dev(g), to_dev(beta), state,
                              accept=None if accept is None else torch.tensor(accept, device=DEV),
                              scale=0.5, g_min=c["g_min"])
    torch.cuda.synchronize()
    o, S = _host(o), state.cpu().numpy()
    for n, h in np.ndindex(N, H):
        err = rel_err(o[n, :, h], o_ref[n, :, h])
        assert err <= O_TOL, f"o seq {n} head {h}: rel err {err:.3e}"
    for n in range(N):
        a = T if accept is None else min(max(int(accept[n]), 0), T)
        if a == 0:
            assert np.array_equal(S[n], d.initial_state[n]), f"seq {n}: state changed with accept 0"
        else:
            check_states(S[n:n + 1], states[a][n:n + 1], f"state seq {n} after {a}")
