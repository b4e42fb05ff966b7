"""The Python binding checks shapes and dtypes before it calls the C ABI (the
ABI takes raw pointers and cannot see sizes). CPU only: every case here is
rejected before any device work."""
import pytest
import torch

from gated_delta_rule_109_amd import kda

F32, BF16 = torch.float32, torch.bfloat16


def t(*shape, dtype=F32):
    return torch.zeros(*shape, dtype=dtype)


def prefill_args(T=40, H=2, D=16, dtype=BF16):
    return dict(q=t(T, H, D, dtype=dtype), k=t(T, H, D, dtype=dtype), v=t(T, H, D, dtype=dtype),
                g=t(T, H, D), beta=t(T, H))


@pytest.mark.parametrize("name,bad,msg", [
    ("k", t(40, 2, 8, dtype=BF16), "k: expected shape"),
    ("v", t(40, 2, 16, dtype=F32), "v: expected"),
    ("g", t(40, 2), "g: expected shape"),
    ("g", t(40, 2, 16, dtype=BF16), "g: expected torch.float32"),
    ("beta", t(40, 2, 1), "beta: expected shape"),
])
def test_prefill_rejects_bad_inputs(name, bad, msg):
    a = prefill_args()
    a[name] = bad
    with pytest.raises((ValueError, TypeError), match=msg):
        kda.prefill(**a)


def test_prefill_rejects_mismatched_lengths_and_states():
    with pytest.raises(ValueError, match="cu_seqlens ends at 30"):
        kda.prefill(**prefill_args(), cu_seqlens=[0, 10, 30])
    with pytest.raises(ValueError, match="initial_state: expected shape"):
        kda.prefill(**prefill_args(), cu_seqlens=[0, 10, 40], initial_state=t(1, 2, 16, 16))
    with pytest.raises(ValueError, match="o: expected shape"):
        kda.prefill(**prefill_args(), o=t(40, 2, 8, dtype=BF16))
    with pytest.raises(TypeError, match="bfloat16 or float32"):
        kda.prefill(**prefill_args(dtype=torch.float16))


def test_prefill_gate_layouts_set_the_shape_of_g():
    a = prefill_args()
    # a per-head gate must be [T, H]; the per-channel one is refused for it
    with pytest.raises(ValueError, match=r"g: expected shape \(40, 2\)"):
        kda.prefill(**a, options=kda.Options(gate=kda.GATE_HEAD))
    a["g"] = None
    with pytest.raises(ValueError, match="g is required"):
        kda.prefill(**a)
    # without a gate, g is not read: any g (or none) passes the checks and the
    # call stops only at the device check
    with pytest.raises(ValueError, match="contiguous device tensors"):
        kda.prefill(**a, options=kda.Options(gate=kda.GATE_NONE))


def test_decode_rejects_bad_inputs():
    q = t(4, 2, 16, dtype=BF16)
    with pytest.raises(ValueError, match="state: expected shape"):
        kda.decode_step(q, q, q, t(4, 2, 16), t(4, 2), t(4, 2, 16, 8))
    with pytest.raises(ValueError, match="beta: expected shape"):
        kda.decode_step(q, q, q, t(4, 2, 16), t(4), t(4, 2, 16, 16))


def test_decode_tokens_rejects_bad_inputs():
    q = t(3, 5, 2, 16, dtype=BF16)
    ok = dict(q=q, k=q, v=q, g=t(3, 5, 2, 16), beta=t(3, 5, 2), state=t(3, 2, 16, 16))
    with pytest.raises(TypeError, match="accept: expected torch.int32"):
        kda.decode_tokens(**ok, accept=torch.zeros(3, dtype=torch.int64))
    with pytest.raises(ValueError, match="accept: expected shape"):
        kda.decode_tokens(**ok, accept=torch.zeros(4, dtype=torch.int32))
    with pytest.raises(ValueError, match=r"g: expected shape \(3, 5, 2\)"):
        kda.decode_tokens(**ok, options=kda.Options(gate=kda.GATE_HEAD))
    with pytest.raises(ValueError, match="contiguous device tensors"):
        kda.decode_tokens(**ok)
