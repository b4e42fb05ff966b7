"""Thin ctypes binding of libkda (include/kda.h).

Argument marshalling only: every step of the computation runs in the HIP
kernels of libkda.so. PyTorch supplies device memory and the current stream.
The library must be built (``python -m gated_delta_rule_109_amd.build`` or
``__graft_entry__.build()``); there is no fallback of any kind when it is
missing.
"""
import ctypes
import math
import os
from dataclasses import dataclass
from typing import Optional

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
# the built library (KDA_LIB names another build of it, e.g. the host-sanitizer one)
LIB_PATH = os.environ.get("KDA_LIB") or os.path.join(HERE, "libkda.so")

KDA_OK, KDA_ERR_INVALID_ARG, KDA_ERR_UNSUPPORTED, KDA_ERR_WORKSPACE, KDA_ERR_HIP = range(5)
KDA_BF16, KDA_F32 = 0, 1
CHUNK = 16
LN_HALF = math.log(0.5)

EXPORTED = ("kda_status_string", "kda_prefill_num_checkpoints", "kda_prefill_workspace_size",
            "kda_prefill_workspace_size_window", "kda_prefill_chunked", "kda_prefill_chunked_ex", "kda_prefill_chunked_noalloc",
            "kda_decode_step", "kda_decode_tokens")
DECODE_MAX_TOKENS = 16
FE_L2NORM_QK, FE_GATE_LOGITS, FE_BETA_LOGITS = 1, 2, 4
FE_ALL = FE_L2NORM_QK | FE_GATE_LOGITS | FE_BETA_LOGITS
GATE_CHANNEL, GATE_HEAD, GATE_NONE = 0, 1, 2     # KDA, Gated DeltaNet, DeltaNet


MAX_SEGMENTS = 16
SEGMENT_SLICE_LIMIT = 80          # forced segments need num_seqs * H * (D / 16) <= this
NOALLOC_SCRATCH_BYTES = 256 << 20  # static scratch of kda_prefill_chunked_noalloc


class Options(ctypes.Structure):
    """kda_options: which inputs are raw (FE_* flags), the norm epsilon, the
    gate layout (GATE_CHANNEL: g [.., H, D]; GATE_HEAD: g [.., H]; GATE_NONE:
    no g), and the prefill's segments per sequence (0: the library's choice,
    1: none, 2 .. MAX_SEGMENTS: forced)."""
    _fields_ = [("flags", ctypes.c_uint32), ("norm_eps", ctypes.c_float), ("gate", ctypes.c_int32),
                ("segments", ctypes.c_int32)]

    def __init__(self, flags=0, norm_eps=1e-6, gate=GATE_CHANNEL, segments=0):
        super().__init__(int(flags), float(norm_eps), int(gate), int(segments))

_lib = None
_vp = ctypes.c_void_p
_i32 = ctypes.c_int32
_i32p = ctypes.POINTER(ctypes.c_int32)


class KdaError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: {lib().kda_status_string(status).decode()}")


def lib():
    """Load libkda.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        L.kda_status_string.restype = ctypes.c_char_p
        L.kda_status_string.argtypes = [ctypes.c_int]
        L.kda_prefill_num_checkpoints.restype = ctypes.c_int64
        L.kda_prefill_num_checkpoints.argtypes = [_i32p, _i32, _i32]
        L.kda_prefill_workspace_size.restype = ctypes.c_size_t
        L.kda_prefill_workspace_size.argtypes = [_i32, ctypes.c_int64, _i32, _i32, _i32]
        L.kda_prefill_workspace_size_window.restype = ctypes.c_size_t
        L.kda_prefill_workspace_size_window.argtypes = [_i32, ctypes.c_int64, _i32, _i32, _i32, ctypes.c_int64]
        L.kda_prefill_chunked.restype = ctypes.c_int
        L.kda_prefill_chunked.argtypes = [_vp, _vp, _vp, ctypes.c_int, _vp, _vp, _vp, _i32p, _i32,
                                          _i32, _i32, _i32, ctypes.c_float, ctypes.c_float, _vp,
                                          _vp, _i32, _vp, _vp, _vp, ctypes.c_size_t, _vp]
        L.kda_decode_step.restype = ctypes.c_int
        L.kda_decode_step.argtypes = [_vp, _vp, _vp, ctypes.c_int, _vp, _vp, _vp, _vp, _i32, _i32,
                                      _i32, _i32, ctypes.c_float, ctypes.c_float, _vp]
        L.kda_decode_tokens.restype = ctypes.c_int
        L.kda_decode_tokens.argtypes = [_vp, _vp, _vp, ctypes.c_int, _vp, _vp, _vp, _vp, _vp, _i32,
                                        _i32, _i32, _i32, _i32, ctypes.c_float, ctypes.c_float,
                                        ctypes.POINTER(Options), _vp]
        L.kda_prefill_chunked_ex.restype = ctypes.c_int
        L.kda_prefill_chunked_ex.argtypes = L.kda_prefill_chunked.argtypes[:-1] + [
            ctypes.POINTER(Options), _vp]
        L.kda_prefill_chunked_noalloc.restype = ctypes.c_int
        L.kda_prefill_chunked_noalloc.argtypes = L.kda_prefill_chunked.argtypes[:-3] + [
            ctypes.POINTER(Options), _vp]
        _lib = L
    return _lib


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dtype_code(t: torch.Tensor):
    if t.dtype == torch.bfloat16:
        return KDA_BF16
    if t.dtype == torch.float32:
        return KDA_F32
    raise TypeError(f"q/k/v must be bfloat16 or float32, got {t.dtype}")


def _host_cu(cu_seqlens):
    cu = torch.as_tensor(cu_seqlens, dtype=torch.int32).cpu().contiguous()
    return cu, cu.numpy().ctypes.data_as(_i32p)


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _check_dev(*ts):
    for t in ts:
        if t is not None and (not t.is_cuda or not t.is_contiguous()):
            raise ValueError("tensors must be contiguous device tensors")


def _expect(t, name, shape, dtype):
    """The C ABI takes raw pointers and cannot see sizes: a wrong shape would
    make a kernel read or write out of bounds, so every tensor is checked here
    before any call."""
    if t is None:
        return
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")


def _gate_shape(lead, H, D, options):
    """Shape of g for the gate layout of `options` (None: no g is read)."""
    gate = GATE_CHANNEL if options is None else options.gate
    if gate == GATE_NONE:
        return None
    return (*lead, H, D) if gate == GATE_CHANNEL else (*lead, H)


def _check_inputs(q, k, v, g, beta, lead, H, D, options, beta_shape):
    if q.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError(f"q/k/v must be bfloat16 or float32, got {q.dtype}")
    for t, name in ((q, "q"), (k, "k"), (v, "v")):
        _expect(t, name, (*lead, H, D), q.dtype)
    gshape = _gate_shape(lead, H, D, options)
    if gshape is None:
        g = None
    elif g is None:
        raise ValueError("g is required by this gate layout")
    _expect(g, "g", gshape if gshape else (), torch.float32)
    _expect(beta, "beta", beta_shape, torch.float32)
    return g


def num_checkpoints(cu_seqlens, ckpt_interval: int) -> int:
    cu, p = _host_cu(cu_seqlens)
    r = lib().kda_prefill_num_checkpoints(p, len(cu) - 1, int(ckpt_interval))
    if r < 0:
        raise KdaError(KDA_ERR_INVALID_ARG, "kda_prefill_num_checkpoints")
    return int(r)


def kda_check_cu(cu_host) -> int:
    """-1 if the host offsets are malformed (cu[0] != 0 or decreasing)."""
    return lib().kda_prefill_num_checkpoints(cu_host.numpy().ctypes.data_as(_i32p), len(cu_host) - 1, 0)


def workspace_size(num_seqs: int, total_tokens: int, H: int, D: int,
                   window_blocks: Optional[int] = None) -> int:
    """kda_prefill_workspace_size: bytes of device workspace for num_seqs
    sequences of total_tokens packed tokens (independent of the lengths);
    with window_blocks, kda_prefill_workspace_size_window: the bytes that run
    the call with the records of at most that many 32-token blocks at a time."""
    if window_blocks is None:
        return int(lib().kda_prefill_workspace_size(int(num_seqs), int(total_tokens), H, D, D))
    return int(lib().kda_prefill_workspace_size_window(int(num_seqs), int(total_tokens), H, D, D,
                                                       int(window_blocks)))


@dataclass
class PrefillPlan:
    """Host and device copies of cu_seqlens plus a workspace sized for them
    (None for kda_prefill_chunked_noalloc, which uses the library's static
    scratch)."""
    cu_host: torch.Tensor
    cu_dev: torch.Tensor
    workspace: Optional[torch.Tensor]
    num_ckpt: int
    ckpt_interval: int


def make_plan(cu_seqlens, H: int, D: int, device, ckpt_interval: int = 0,
              workspace: bool = True, window_blocks: Optional[int] = None) -> PrefillPlan:
    """window_blocks: size the workspace for record windows of at most that
    many blocks (None: the library's default size)."""
    cu_host, p = _host_cu(cu_seqlens)
    if int(kda_check_cu(cu_host)) < 0:
        raise KdaError(KDA_ERR_INVALID_ARG, "cu_seqlens")
    if workspace:
        ws = workspace_size(len(cu_host) - 1, int(cu_host[-1]), H, D, window_blocks)
        if ws == 0:
            raise KdaError(KDA_ERR_INVALID_ARG, "kda_prefill_workspace_size")
        workspace = torch.empty(max(ws, 256), dtype=torch.uint8, device=device)
    else:
        workspace = None
    return PrefillPlan(cu_host, cu_host.to(device), workspace,
                       num_checkpoints(cu_host, ckpt_interval) if ckpt_interval else 0,
                       int(ckpt_interval))


def _opt_ptr(options: Optional[Options]):
    return None if options is None else ctypes.byref(options)


def prefill(q, k, v, g, beta, cu_seqlens=None, initial_state=None, scale=1.0, g_min=LN_HALF,
            ckpt_interval=0, out_final_state=True, plan: Optional[PrefillPlan] = None,
            o=None, final_state=None, checkpoints=None, options: Optional[Options] = None,
            noalloc: bool = False):
    """kda_prefill_chunked on packed [T, H, D] tensors (kda_prefill_chunked_ex
    when Options are given: gate layout, and q, k, g, beta raw as the flags
    say; kda_prefill_chunked_noalloc when noalloc is set: no workspace, the
    library's static scratch instead).

    Returns (o, final_state or None, checkpoints or None)."""
    T, H, D = q.shape
    if plan is None:
        plan = make_plan([0, T] if cu_seqlens is None else cu_seqlens, H, D, q.device, ckpt_interval,
                         workspace=not noalloc)
    N = len(plan.cu_host) - 1
    if int(plan.cu_host[-1]) != T:
        raise ValueError(f"cu_seqlens ends at {int(plan.cu_host[-1])}, but q holds {T} tokens")
    g = _check_inputs(q, k, v, g, beta, (T,), H, D, options, (T, H))
    _expect(initial_state, "initial_state", (N, H, D, D), torch.float32)
    _expect(o, "o", (T, H, D), q.dtype)
    _expect(final_state, "final_state", (N, H, D, D), torch.float32)
    _expect(checkpoints, "checkpoints", (plan.num_ckpt, H, D, D), torch.float32)
    _check_dev(q, k, v, g, beta, initial_state, o, final_state, checkpoints)
    if o is None:
        o = torch.empty_like(v)
    if final_state is None and out_final_state:
        final_state = torch.empty(N, H, D, D, dtype=torch.float32, device=q.device)
    if checkpoints is None and plan.num_ckpt > 0:
        checkpoints = torch.empty(plan.num_ckpt, H, D, D, dtype=torch.float32, device=q.device)
    args = (_ptr(q), _ptr(k), _ptr(v), _dtype_code(q), _ptr(g), _ptr(beta), _ptr(plan.cu_dev),
            plan.cu_host.numpy().ctypes.data_as(_i32p), N, H, D, v.shape[2], float(scale),
            float(g_min), _ptr(initial_state), _ptr(final_state), plan.ckpt_interval,
            _ptr(checkpoints), _ptr(o))
    if noalloc:
        st = lib().kda_prefill_chunked_noalloc(*args, _opt_ptr(options), _stream(q.device))
        if st != KDA_OK:
            raise KdaError(st, "kda_prefill_chunked_noalloc")
        return o, final_state, checkpoints
    if plan.workspace is None:
        raise ValueError("this plan has no workspace (made for the noalloc entry point)")
    args += (_ptr(plan.workspace), plan.workspace.numel())
    if options is None:
        st = lib().kda_prefill_chunked(*args, _stream(q.device))
    else:
        st = lib().kda_prefill_chunked_ex(*args, _opt_ptr(options), _stream(q.device))
    if st != KDA_OK:
        raise KdaError(st, "kda_prefill_chunked")
    return o, final_state, checkpoints


def decode_step(q, k, v, g, beta, state, scale=1.0, g_min=LN_HALF, o=None):
    """kda_decode_step: q,k,g [N,H,D]; v [N,H,D]; beta [N,H]; state [N,H,D,D]
    updated in place. Returns o [N,H,D]."""
    N, H, D = q.shape
    _check_inputs(q, k, v, g, beta, (N,), H, D, None, (N, H))
    _expect(state, "state", (N, H, D, D), torch.float32)
    _expect(o, "o", (N, H, D), q.dtype)
    _check_dev(q, k, v, g, beta, state, o)
    if o is None:
        o = torch.empty_like(v)
    st = lib().kda_decode_step(_ptr(q), _ptr(k), _ptr(v), _dtype_code(q), _ptr(g), _ptr(beta),
                               _ptr(state), _ptr(o), N, H, D, v.shape[2], float(scale),
                               float(g_min), _stream(q.device))
    if st != KDA_OK:
        raise KdaError(st, "kda_decode_step")
    return o


def decode_tokens(q, k, v, g, beta, state, accept=None, scale=1.0, g_min=LN_HALF, o=None,
                  options: Optional[Options] = None):
    """kda_decode_tokens: q,k,g,v [N,T,H,D]; beta [N,T,H]; state [N,H,D,D]
    updated in place to the state after accept[n] tokens (all T when accept is
    None); accept is a device int32 [N] tensor; options as in prefill.
    Returns o [N,T,H,D]."""
    N, T, H, D = q.shape
    g = _check_inputs(q, k, v, g, beta, (N, T), H, D, options, (N, T, H))
    _expect(state, "state", (N, H, D, D), torch.float32)
    _expect(accept, "accept", (N,), torch.int32)
    _expect(o, "o", (N, T, H, D), q.dtype)
    _check_dev(q, k, v, g, beta, state, accept, o)
    if o is None:
        o = torch.empty_like(v)
    st = lib().kda_decode_tokens(_ptr(q), _ptr(k), _ptr(v), _dtype_code(q), _ptr(g), _ptr(beta),
                                 _ptr(state), _ptr(accept), _ptr(o), N, T, H, D, v.shape[3],
                                 float(scale), float(g_min), _opt_ptr(options), _stream(q.device))
    if st != KDA_OK:
        raise KdaError(st, "kda_decode_tokens")
    return o
