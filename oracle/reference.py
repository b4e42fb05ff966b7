"""ctypes front end of the C fp64 KDA oracle (oracle/kda_oracle.c).

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

Inputs are float32 arrays holding exactly the values the device consumes
(bf16 inputs upcast exactly); all arithmetic is fp64. The recurrence, its
readings and citations are documented in kda_oracle.c.
"""
import ctypes
import os

import numpy as np

from . import build as _build

_lib = None

_f = ctypes.POINTER(ctypes.c_float)
_d = ctypes.POINTER(ctypes.c_double)
_i64 = ctypes.POINTER(ctypes.c_int64)


def lib():
    """The compiled oracle: oracle/liboracle_kda.so, or the library named by
    KDA_ORACLE_LIB (the sanitizer build)."""
    global _lib
    if _lib is None:
        path = os.environ.get("KDA_ORACLE_LIB") or _build.LIB
        if path == _build.LIB and not os.path.exists(path):
            _build.build()
        L = ctypes.CDLL(path)
        L.kda_oracle_prefill.restype = ctypes.c_int
        L.kda_oracle_prefill.argtypes = [_f, _f, _f, _f, _f, _i64, ctypes.c_int32,
                                         ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                         ctypes.c_double, ctypes.c_double, _d, _d,
                                         ctypes.c_int64, _d, _d, ctypes.c_int32]
        L.kda_oracle_decode.restype = ctypes.c_int
        L.kda_oracle_decode.argtypes = [_f, _f, _f, _f, _f, _d, _d, _d, ctypes.c_int32,
                                        ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                        ctypes.c_double, ctypes.c_double, ctypes.c_int32]
        L.kda_oracle_num_checkpoints.restype = ctypes.c_int64
        L.kda_oracle_num_checkpoints.argtypes = [_i64, ctypes.c_int32, ctypes.c_int64]
        L.kda_oracle_max_threads.restype = ctypes.c_int32
        L.kda_oracle_max_threads.argtypes = []
        _lib = L
    return _lib


def _fp(a):
    return a.ctypes.data_as(_f)


def _dp(a):
    return None if a is None else a.ctypes.data_as(_d)


def _f32(a):
    return np.ascontiguousarray(a, dtype=np.float32)


LN_HALF = float(np.log(0.5))


def prefill(q, k, v, g, beta, cu_seqlens=None, initial_state=None, scale=1.0,
            g_min=LN_HALF, ckpt_interval=0, want_o=True, threads=0):
    """Run the recurrence over packed sequences.

    q, k, g: [T, H, Dk]; v: [T, H, Dv]; beta: [T, H]; cu_seqlens: [N+1]
    (default: one sequence of length T); initial_state: [N, H, Dk, Dv] or None.
    Returns (o [T,H,Dv] fp64 or None, final [N,H,Dk,Dv] fp64, ckpts fp64).
    """
    q, k, v, g, beta = map(_f32, (q, k, v, g, beta))
    T, H, Dk = q.shape
    Dv = v.shape[2]
    if cu_seqlens is None:
        cu_seqlens = [0, T]
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int64)
    N = len(cu) - 1
    s0 = None if initial_state is None else np.ascontiguousarray(initial_state, dtype=np.float64)
    final = np.zeros((N, H, Dk, Dv), np.float64)
    nck = int(lib().kda_oracle_num_checkpoints(cu.ctypes.data_as(_i64), N, int(ckpt_interval)))
    ck = np.zeros((max(nck, 1), H, Dk, Dv), np.float64)
    o = np.zeros((T, H, Dv), np.float64) if want_o else None
    rc = lib().kda_oracle_prefill(_fp(q), _fp(k), _fp(v), _fp(g), _fp(beta),
                                  cu.ctypes.data_as(_i64), N, H, Dk, Dv, float(scale),
                                  float(g_min), _dp(s0), _dp(final), int(ckpt_interval),
                                  _dp(ck), _dp(o), int(threads))
    if rc != 0:
        raise RuntimeError(f"kda_oracle_prefill failed with status {rc}")
    return o, final, ck[:nck]


def decode(q, k, v, g, beta, state, scale=1.0, g_min=LN_HALF, threads=0):
    """One token per sequence. q,k,g: [N,H,Dk]; v: [N,H,Dv]; beta: [N,H];
    state: [N,H,Dk,Dv]. Returns (o [N,H,Dv], new_state), both fp64."""
    q, k, v, g, beta = map(_f32, (q, k, v, g, beta))
    N, H, Dk = q.shape
    Dv = v.shape[2]
    s_in = np.ascontiguousarray(state, dtype=np.float64)
    s_out = np.empty_like(s_in)
    o = np.zeros((N, H, Dv), np.float64)
    rc = lib().kda_oracle_decode(_fp(q), _fp(k), _fp(v), _fp(g), _fp(beta), _dp(s_in),
                                 _dp(s_out), _dp(o), N, H, Dk, Dv, float(scale),
                                 float(g_min), int(threads))
    if rc != 0:
        raise RuntimeError(f"kda_oracle_decode failed with status {rc}")
    return o, s_out


def max_threads():
    return int(lib().kda_oracle_max_threads())
