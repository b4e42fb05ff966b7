"""kda_prefill_chunked_noalloc (static per-device scratch, no workspace
argument) against kda_prefill_chunked_ex (caller's workspace) on the same
inputs, through the C ABI: calls in a row, each smaller than the one before,
every output, final state and checkpoint bit-identical (both run the same
kernels; the scratch keeps the previous call's contents, which the prefill
must not depend on). Calls whose records exceed the scratch run in record
windows."""
import numpy as np
import pytest
import torch

from gated_delta_rule_109_amd import kda
from gated_delta_rule_109_amd.workloads import make_inputs, make_inputs_device

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def to_dev(a, dt=torch.float32):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dt).to(DEV)


def _both(q, k, v, g, beta, cu, s0, ckpt, options):
    outs = []
    for noalloc in (True, False):
        outs.append(kda.prefill(q, k, v, g, beta, cu_seqlens=cu, initial_state=s0, ckpt_interval=ckpt,
                                options=options, noalloc=noalloc))
    torch.cuda.synchronize()
    return outs


def _same(a, b, what):
    for x, y, name in zip(a, b, ("o", "final state", "checkpoints")):
        if x is None or y is None:
            assert x is None and y is None, f"{what}: {name}"
        else:
            assert torch.equal(x, y), f"{what}: {name} differs"


def test_noalloc_equals_workspace_entry_point_on_shrinking_calls():
    # 1. near the scratch limit: 4096 tokens x 32 heads at D = 128
    T, H, D = 4096, 32, 128
    assert kda.workspace_size(1, T, H, D) <= kda.NOALLOC_SCRATCH_BYTES
    print(f"case: noalloc call 1: T={T} H={H} D={D}", flush=True)
    q, k, v, g, beta, cu, _ = make_inputs_device(T, H, D, seed=301, device=DEV)
    a, b = _both(q, k, v, g, beta, cu, None, 1024, None)
    _same(a, b, "call 1")
    # 2. smaller: one sequence, 4 heads, the library's segments (their states
    #    live in the scratch too), Gated DeltaNet layout
    lengths = [2000]
    print(f"case: noalloc call 2: lengths={lengths} H=4 D=128 segments", flush=True)
    inp = make_inputs(sum(lengths), 4, 128, seed=302, lengths=lengths, initial_state=True)
    gv = np.ascontiguousarray(inp.g[..., 0])
    a, b = _both(to_dev(inp.q, torch.bfloat16), to_dev(inp.k, torch.bfloat16), to_dev(inp.v, torch.bfloat16),
                 to_dev(gv), to_dev(inp.beta), inp.cu_seqlens, to_dev(inp.initial_state), 0,
                 kda.Options(gate=kda.GATE_HEAD))
    _same(a, b, "call 2")
    # 3. smaller still: ragged varlen, checkpoints, fp32 storage, D = 16
    lengths = [17, 0, 64, 1]
    print(f"case: noalloc call 3: lengths={lengths} H=2 D=16 fp32", flush=True)
    inp = make_inputs(sum(lengths), 2, 16, seed=303, lengths=lengths, initial_state=True, bf16=False)
    a, b = _both(to_dev(inp.q), to_dev(inp.k), to_dev(inp.v), to_dev(inp.g), to_dev(inp.beta), inp.cu_seqlens,
                 to_dev(inp.initial_state), 16, None)
    _same(a, b, "call 3")


def test_noalloc_runs_long_calls_in_record_windows():
    """8192 tokens x 32 heads: 386 MB of records do not fit the 256 MiB
    scratch at once, so the call runs in record windows; bit-identical to the
    one-window call with a workspace. Then a smaller call in a row."""
    T, H, D = 8192, 32, 128
    assert kda.workspace_size(1, T, H, D) > kda.NOALLOC_SCRATCH_BYTES
    print(f"case: noalloc in windows: T={T} H={H} checkpoints every 1024", flush=True)
    q, k, v, g, beta, cu, _ = make_inputs_device(T, H, D, seed=304, device=DEV)
    a, b = _both(q, k, v, g, beta, cu, None, 1024, None)
    _same(a, b, "windowed call")
    lengths = [33, 0, 500]
    print(f"case: noalloc after the windowed call: lengths={lengths} H=3", flush=True)
    inp = make_inputs(sum(lengths), 3, 128, seed=305, lengths=lengths, initial_state=True)
    a, b = _both(to_dev(inp.q, torch.bfloat16), to_dev(inp.k, torch.bfloat16), to_dev(inp.v, torch.bfloat16),
                 to_dev(inp.g), to_dev(inp.beta), inp.cu_seqlens, to_dev(inp.initial_state), 16, None)
    _same(a, b, "call after the windowed call")


def test_noalloc_refuses_shapes_beyond_the_scratch():
    """Only a shape whose tables and one block of records per head exceed the
    scratch is refused (8192 heads: 376 MiB per block), before any device
    work."""
    T, H, D = 32, 8192, 128
    assert kda.workspace_size(1, T, H, D, window_blocks=1) > kda.NOALLOC_SCRATCH_BYTES
    print(f"case: noalloc beyond the scratch: T={T} H={H}", flush=True)
    q, k, v, g, beta, cu, _ = make_inputs_device(T, H, D, seed=306, device=DEV)
    with pytest.raises(kda.KdaError) as e:
        kda.prefill(q, k, v, g, beta, cu_seqlens=cu, noalloc=True)
    assert e.value.status == kda.KDA_ERR_WORKSPACE


def test_noalloc_windowed_call_replays_from_a_captured_graph():
    """The allocation-free entry point captured in a graph, on a shape whose
    records exceed the scratch (8192 tokens x 32 heads: record windows):
    every replay equals the eager call on the same inputs bit for bit."""
    T, H, D = 8192, 32, 128
    print(f"case: noalloc graph capture T={T} H={H}", flush=True)
    plan = kda.make_plan([0, T], H, D, DEV, ckpt_interval=1024, workspace=False)
    bufs = {n: torch.empty(T, H, D, dtype=torch.bfloat16, device=DEV) for n in ("q", "k", "v")}
    g = torch.empty(T, H, D, device=DEV)
    beta = torch.empty(T, H, device=DEV)
    o = torch.empty(T, H, D, dtype=torch.bfloat16, device=DEV)
    fin = torch.empty(1, H, D, D, device=DEV)
    ck = torch.empty(plan.num_ckpt, H, D, D, device=DEV)

    def load(seed):
        q, k, v, gg, bb, _, _ = make_inputs_device(T, H, D, seed=seed, device=DEV)
        for n, x in (("q", q), ("k", k), ("v", v)):
            bufs[n].copy_(x)
        g.copy_(gg)
        beta.copy_(bb)

    def call():
        kda.prefill(bufs["q"], bufs["k"], bufs["v"], g, beta, plan=plan, o=o, final_state=fin, checkpoints=ck,
                    noalloc=True)

    load(310)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    for seed in (311, 312):
        load(seed)
        graph.replay()
        torch.cuda.synchronize()
        got = (o.clone(), fin.clone(), ck.clone())
        _ = torch.randn(1 << 20, device=DEV).sum()          # unrelated eager work
        call()
        torch.cuda.synchronize()
        for x, y in zip(got, (o, fin, ck)):
            assert torch.equal(x, y), f"replay with inputs {seed} differs from the eager call"
