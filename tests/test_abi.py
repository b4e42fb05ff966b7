"""Host-side checks of the C ABI (no GPU): the library loads, exports every
symbol include/kda.h declares, sizes workspaces and checkpoints, and rejects
bad arguments with the documented status before any device work."""
import ctypes
import os
import re

import pytest

from gated_delta_rule_109_amd import kda

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kda.h")


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const char\*|int64_t|size_t|kda_status)\s+(kda_\w+)\(",
                                 text, flags=re.M)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(kda.LIB_PATH):
        from gated_delta_rule_109_amd import build
        build.build()
    return kda.lib()


def test_every_declared_symbol_is_exported(L):
    names = declared_functions()
    assert set(names) == set(kda.EXPORTED)
    for name in names:
        assert hasattr(L, name), name


def test_status_strings(L):
    for code in range(5):
        assert L.kda_status_string(code).startswith(b"KDA_")
    assert L.kda_status_string(99) == b"KDA: unknown status"


def cu(*lengths):
    out = [0]
    for x in lengths:
        out.append(out[-1] + x)
    return out


def test_checkpoint_counts(L):
    assert kda.num_checkpoints(cu(131072), 32768) == 4
    assert kda.num_checkpoints(cu(48, 47, 16, 0, 33), 16) == 3 + 2 + 1 + 0 + 2
    assert kda.num_checkpoints(cu(100), 0) == 0
    with pytest.raises(kda.KdaError):
        kda.num_checkpoints([1, 5], 16)            # cu[0] != 0
    with pytest.raises(kda.KdaError):
        kda.num_checkpoints([0, 9, 3], 16)         # decreasing


def test_workspace_size(L):
    # per (32-token block, head) record: 47 KiB at D = 128, 15 KiB at D = 16,
    # sized for the most blocks num_seqs sequences of T tokens can have,
    # T / 32 + num_seqs, plus tables
    rec128, rec16 = 47 * 1024, 15 * 1024
    seg = lambda N, H, D: N * 16 * H * 3 * D * D * 4     # 16 segments at most
    w = kda.workspace_size(1, 8192, 32, 128)             # 32 x 8 slices > 80: no segments
    assert 257 * 32 * rec128 <= w < 257 * 32 * rec128 + 8192
    # the size depends on the total only, not on how it is split
    w4 = kda.workspace_size(1, 8192, 4, 128)             # 4 x 8 slices <= 80: segment states
    assert 257 * 4 * rec128 + seg(1, 4, 128) <= w4 < 257 * 4 * rec128 + seg(1, 4, 128) + 8192
    w16 = kda.workspace_size(1, 64, 2, 16)
    assert 3 * 2 * rec16 + seg(1, 2, 16) <= w16 < 3 * 2 * rec16 + seg(1, 2, 16) + 2048
    # ragged lengths never need more than T / 32 + num_seqs blocks
    wv = kda.workspace_size(3, 97, 1, 128)
    assert (97 // 32 + 3) * rec128 <= wv
    for lens in ((33, 33, 31), (1, 1, 95), (97, 0, 0), (32, 32, 33)):
        blocks = sum((x + 31) // 32 for x in lens)
        assert blocks * rec128 <= wv
    assert kda.workspace_size(1, 10, 2, 64) == 0          # unsupported D
    assert kda.workspace_size(-1, 10, 2, 128) == 0
    assert kda.workspace_size(1, -1, 2, 128) == 0
    assert kda.workspace_size(1, 10, 0, 128) == 0
    assert kda.workspace_size(1, 2 ** 40, 1, 128) == 0    # too many blocks


def test_workspace_size_windows(L):
    """Record windows: the default size caps the records at
    KDA_PREFILL_RECORD_CAP_BYTES (8 GiB), so it stops growing with T there
    (the tables still grow by 16 bytes per 32-token block); a single sequence
    takes windows of about KDA_PREFILL_SINGLE_SEQ_WINDOW_BYTES (1 GiB); a size
    for windows of W blocks holds W blocks of records per head plus two carry
    states per head."""
    rec128, cap = 47 * 1024, 8 << 30
    state = lambda H, D: H * D * D * 4
    # several sequences, below the cap: one window, the same bytes as a window
    # of every block (131072 / 32 + 2 blocks at most)
    w = kda.workspace_size(2, 131072, 32, 128)
    assert w == kda.workspace_size(2, 131072, 32, 128, window_blocks=4098)
    assert w == kda.workspace_size(2, 131072, 32, 128, window_blocks=10 ** 9)
    assert 4098 * 32 * rec128 <= w < 4098 * 32 * rec128 + 16 * 4098 + 4096
    # beyond the cap: records of cap / (H x 47 KiB) blocks, plus the carry
    blocks_cap = cap // (32 * rec128)
    for T in (1 << 20, 1 << 22, 1 << 24):
        wt = kda.workspace_size(2, T, 32, 128)
        tables = 16 * (T // 32 + 2) + 4096
        assert blocks_cap * 32 * rec128 + 2 * state(32, 128) <= wt
        assert wt < blocks_cap * 32 * rec128 + 2 * state(32, 128) + tables
    # growth from 1M to 16M tokens: the tables only
    assert kda.workspace_size(2, 1 << 24, 32, 128) - kda.workspace_size(2, 1 << 20, 32, 128) < 16 * (1 << 19) + 4096
    # one sequence: windows of 1 GiB of records (697 blocks at 32 heads)
    w1 = (1 << 30) // (32 * rec128)
    assert w1 == 697
    assert kda.workspace_size(1, 131072, 32, 128) == kda.workspace_size(1, 131072, 32, 128, window_blocks=w1)
    assert kda.workspace_size(1, 131072, 32, 128) < (1 << 30) + 2 * state(32, 128) + 16 * 4097 + 4096
    assert kda.workspace_size(1, 8192, 32, 128) == kda.workspace_size(1, 8192, 32, 128, window_blocks=257)
    # explicit windows: W blocks of records per head and two carry states
    for W in (1, 2, 7, 64):
        ww = kda.workspace_size(3, 8192, 4, 128, window_blocks=W)
        base = kda.workspace_size(3, 8192, 4, 128, window_blocks=10 ** 6)   # one window
        assert ww == base - (8192 // 32 + 3 - W) * 4 * rec128 + 2 * state(4, 128)
    assert kda.workspace_size(1, 64, 2, 16, window_blocks=1) < kda.workspace_size(1, 64, 2, 16)
    assert kda.workspace_size(1, 64, 2, 128, window_blocks=0) == 0
    assert kda.workspace_size(1, 64, 2, 128, window_blocks=-3) == 0
    # shapes the prefill refuses get no size: token-heads past INT32_MAX
    assert kda.workspace_size(1, 1 << 30, 4, 128) == 0
    assert kda.workspace_size(1, 1 << 31, 1, 128) == 0
    assert kda.workspace_size(1, (1 << 31) - 1, 1, 128) > 0


def _prefill_status(L, **over):
    """Call kda_prefill_chunked with dummy non-null pointers; every case here
    must fail validation before touching them."""
    host = (ctypes.c_int32 * 3)(*cu(20, 12))
    fake = ctypes.c_void_p(0x1000)
    args = dict(q=fake, k=fake, v=fake, dtype=kda.KDA_BF16, g=fake, beta=fake, cu=fake,
                cu_host=ctypes.cast(host, ctypes.POINTER(ctypes.c_int32)), N=2, H=4, Dk=128, Dv=128,
                scale=1.0, g_min=-0.69, s0=None, fin=None, ckpt=0, ckpts=None, o=fake, ws=fake,
                ws_bytes=0, stream=None)
    args.update(over)
    return L.kda_prefill_chunked(*args.values())


def test_prefill_argument_errors(L):
    E = kda
    assert _prefill_status(L, Dk=64, Dv=64) == E.KDA_ERR_UNSUPPORTED
    assert _prefill_status(L, Dk=128, Dv=16) == E.KDA_ERR_UNSUPPORTED
    assert _prefill_status(L, dtype=7) == E.KDA_ERR_UNSUPPORTED
    assert _prefill_status(L, H=0) == E.KDA_ERR_INVALID_ARG
    assert _prefill_status(L, cu=None) == E.KDA_ERR_INVALID_ARG
    assert _prefill_status(L, q=None) == E.KDA_ERR_INVALID_ARG
    assert _prefill_status(L, o=None) == E.KDA_ERR_INVALID_ARG
    assert _prefill_status(L, ckpt=24) == E.KDA_ERR_INVALID_ARG      # not a multiple of 16
    assert _prefill_status(L, ckpt=-16) == E.KDA_ERR_INVALID_ARG
    assert _prefill_status(L, ckpt=16, ckpts=None) == E.KDA_ERR_INVALID_ARG
    bad = (ctypes.c_int32 * 3)(0, 9, 3)
    assert _prefill_status(L, cu_host=ctypes.cast(bad, ctypes.POINTER(ctypes.c_int32))) == E.KDA_ERR_INVALID_ARG
    assert _prefill_status(L) == E.KDA_ERR_WORKSPACE                  # no workspace bytes
    assert _prefill_status(L, ws=None, ws_bytes=1 << 30) == E.KDA_ERR_WORKSPACE
    assert _prefill_status(L, ws=ctypes.c_void_p(0x1010), ws_bytes=1 << 30) == E.KDA_ERR_WORKSPACE
    assert _prefill_status(L, v=ctypes.c_void_p(0x1002)) == E.KDA_ERR_INVALID_ARG   # misaligned
    assert _prefill_status(L, g_min=-5.5) == E.KDA_ERR_INVALID_ARG     # decay floor below the supported range
    assert _prefill_status(L, g_min=0.5) == E.KDA_ERR_INVALID_ARG
    assert _prefill_status(L, g_min=float("nan")) == E.KDA_ERR_INVALID_ARG
    empty = (ctypes.c_int32 * 1)(0)
    assert _prefill_status(L, N=0, cu_host=ctypes.cast(empty, ctypes.POINTER(ctypes.c_int32))) == E.KDA_OK
    as_ptr = lambda a: ctypes.cast(a, ctypes.POINTER(ctypes.c_int32))
    assert _prefill_status(L, N=-1) == E.KDA_ERR_INVALID_ARG
    assert _prefill_status(L, cu_host=as_ptr((ctypes.c_int32 * 3)(4, 20, 32))) == E.KDA_ERR_INVALID_ARG  # cu[0] != 0
    # token-heads past INT32_MAX (2^30 tokens x 4 heads): refused before any device work
    big = (ctypes.c_int32 * 2)(0, 1 << 30)
    assert _prefill_status(L, N=1, cu_host=as_ptr(big)) == E.KDA_ERR_INVALID_ARG
    assert _prefill_status(L, N=1, H=1, cu_host=as_ptr(big)) == E.KDA_ERR_WORKSPACE   # within range: sizes next


def test_noalloc_prefill_errors_before_any_device_work(L):
    """kda_prefill_chunked_noalloc validates like kda_prefill_chunked_ex and
    refuses shapes whose workspace exceeds its static scratch, all before the
    scratch is looked up or any work is enqueued (so dummy pointers are safe
    here). Only failing cases are called."""
    fake = ctypes.c_void_p(0x1000)
    small = (ctypes.c_int32 * 3)(*cu(20, 12))
    big = (ctypes.c_int32 * 2)(*cu(8192))
    as_p = lambda a: ctypes.cast(a, ctypes.POINTER(ctypes.c_int32))

    def call(**over):
        a = dict(q=fake, k=fake, v=fake, dtype=kda.KDA_BF16, g=fake, beta=fake, cu=fake, cu_host=as_p(small),
                 N=2, H=4, Dk=128, Dv=128, scale=1.0, g_min=-0.69, s0=None, fin=None, ckpt=0, ckpts=None,
                 o=fake, opt=None, stream=None)
        a.update(over)
        return L.kda_prefill_chunked_noalloc(*a.values())
    assert call(Dk=64, Dv=64) == kda.KDA_ERR_UNSUPPORTED
    assert call(q=None) == kda.KDA_ERR_INVALID_ARG
    assert call(g_min=0.5) == kda.KDA_ERR_INVALID_ARG
    assert call(ckpt=24) == kda.KDA_ERR_INVALID_ARG
    assert call(opt=ctypes.byref(kda.Options(gate=-1))) == kda.KDA_ERR_INVALID_ARG
    # long calls run in record windows; only a shape whose tables and one block
    # per head exceed the scratch is refused (8192 heads: 376 MiB per block)
    assert kda.workspace_size(1, 8192, 32, 128) > kda.NOALLOC_SCRATCH_BYTES
    assert kda.workspace_size(1, 8192, 32, 128, window_blocks=1) < kda.NOALLOC_SCRATCH_BYTES
    assert kda.workspace_size(1, 8192, 8192, 128, window_blocks=1) > kda.NOALLOC_SCRATCH_BYTES
    assert call(cu_host=as_p(big), N=1, H=8192) == kda.KDA_ERR_WORKSPACE
    empty = (ctypes.c_int32 * 1)(0)
    assert call(N=0, cu_host=as_p(empty)) == kda.KDA_OK


def test_decode_argument_errors(L):
    fake = ctypes.c_void_p(0x1000)
    call = lambda **o: L.kda_decode_step(*dict(dict(q=fake, k=fake, v=fake, dtype=0, g=fake, beta=fake,
                                                    state=fake, o=fake, N=4, H=2, Dk=128, Dv=128,
                                                    scale=1.0, g_min=-0.69, stream=None), **o).values())
    assert call(Dk=32, Dv=32) == kda.KDA_ERR_UNSUPPORTED
    assert call(dtype=3) == kda.KDA_ERR_UNSUPPORTED
    assert call(N=-1) == kda.KDA_ERR_INVALID_ARG
    assert call(H=0) == kda.KDA_ERR_INVALID_ARG
    assert call(state=None) == kda.KDA_ERR_INVALID_ARG
    assert call(state=ctypes.c_void_p(0x1004)) == kda.KDA_ERR_INVALID_ARG
    assert call(N=0) == kda.KDA_OK                                    # nothing to do
    # the decay floor: any finite value at or below 0
    assert call(g_min=0.5) == kda.KDA_ERR_INVALID_ARG
    assert call(g_min=float("nan")) == kda.KDA_ERR_INVALID_ARG
    assert call(g_min=float("-inf")) == kda.KDA_ERR_INVALID_ARG
    assert call(g_min=-40.0, N=0) == kda.KDA_OK


def test_decode_tokens_argument_errors(L):
    fake = ctypes.c_void_p(0x1000)
    call = lambda **o: L.kda_decode_tokens(*dict(dict(q=fake, k=fake, v=fake, dtype=0, g=fake,
                                                      beta=fake, state=fake, accept=None, o=fake,
                                                      N=4, T=3, H=2, Dk=128, Dv=128, scale=1.0,
                                                      g_min=-0.69, fe=None, stream=None), **o).values())
    assert call(Dk=16, Dv=128) == kda.KDA_ERR_UNSUPPORTED
    assert call(dtype=2) == kda.KDA_ERR_UNSUPPORTED
    assert call(T=0) == kda.KDA_ERR_INVALID_ARG
    assert call(T=kda.DECODE_MAX_TOKENS + 1) == kda.KDA_ERR_INVALID_ARG
    assert call(N=-2) == kda.KDA_ERR_INVALID_ARG
    assert call(H=-1) == kda.KDA_ERR_INVALID_ARG
    assert call(N=1 << 20, T=16, H=256) == kda.KDA_ERR_INVALID_ARG   # N*T*H overflows int32
    assert call(o=None) == kda.KDA_ERR_INVALID_ARG
    assert call(beta=ctypes.c_void_p(0x1002)) == kda.KDA_ERR_INVALID_ARG
    assert call(N=0) == kda.KDA_OK
    for bad in (kda.Options(8), kda.Options(kda.FE_ALL, -1.0), kda.Options(1, float("nan")),
                kda.Options(1, float("inf"))):
        assert call(fe=ctypes.byref(bad)) == kda.KDA_ERR_INVALID_ARG
    assert call(fe=ctypes.byref(kda.Options(kda.FE_ALL, 0.0)), N=0) == kda.KDA_OK
    # gate layouts: unknown values and gate logits without a gate are rejected;
    # g may be NULL only without a gate
    assert call(fe=ctypes.byref(kda.Options(gate=3))) == kda.KDA_ERR_INVALID_ARG
    assert call(fe=ctypes.byref(kda.Options(kda.FE_GATE_LOGITS, gate=kda.GATE_NONE))) == kda.KDA_ERR_INVALID_ARG
    assert call(g=None) == kda.KDA_ERR_INVALID_ARG
    assert call(g=None, fe=ctypes.byref(kda.Options(gate=kda.GATE_HEAD))) == kda.KDA_ERR_INVALID_ARG
    assert call(g=None, fe=ctypes.byref(kda.Options(gate=kda.GATE_NONE)), N=0) == kda.KDA_OK
    assert call(g_min=1e-3) == kda.KDA_ERR_INVALID_ARG
    assert call(g_min=float("nan"), N=0) == kda.KDA_ERR_INVALID_ARG


def test_decode_max_tokens_matches_header():
    m = re.search(r"#define\s+KDA_DECODE_MAX_TOKENS\s+(\d+)", open(HEADER).read())
    assert m and int(m.group(1)) == kda.DECODE_MAX_TOKENS


def test_segment_limits_match_header():
    text = open(HEADER).read()
    for name, value in (("KDA_MAX_SEGMENTS", kda.MAX_SEGMENTS), ("KDA_SEGMENT_SLICE_LIMIT", kda.SEGMENT_SLICE_LIMIT)):
        m = re.search(r"#define\s+%s\s+(\d+)" % name, text)
        assert m and int(m.group(1)) == value, name


def test_noalloc_scratch_size_matches_header():
    m = re.search(r"#define\s+KDA_NOALLOC_SCRATCH_BYTES\s+\((\d+)u\s*<<\s*(\d+)\)", open(HEADER).read())
    assert m and int(m.group(1)) << int(m.group(2)) == kda.NOALLOC_SCRATCH_BYTES


def test_prefill_options_argument_errors(L):
    """kda_prefill_chunked_ex validates the options first; with opt = NULL
    it returns what kda_prefill_chunked returns."""
    fake = ctypes.c_void_p(0x1000)
    cu = (ctypes.c_int32 * 2)(0, 64)
    ws = ctypes.c_void_p(0x100000)

    def call(fe, **over):
        a = dict(q=fake, k=fake, v=fake, dtype=0, g=fake, beta=fake, cu=fake,
                 cu_host=ctypes.cast(cu, ctypes.POINTER(ctypes.c_int32)), N=1, H=2, Dk=128, Dv=128,
                 scale=1.0, g_min=-0.69, s0=None, fin=None, ck_int=0, ck=None, o=fake, ws=ws,
                 ws_bytes=0, fe=fe, stream=None)
        a.update(over)
        return L.kda_prefill_chunked_ex(*a.values())
    for bad in (kda.Options(16), kda.Options(kda.FE_L2NORM_QK, -0.5), kda.Options(2, float("nan")),
                kda.Options(gate=-1), kda.Options(kda.FE_GATE_LOGITS, gate=kda.GATE_NONE)):
        assert call(ctypes.byref(bad)) == kda.KDA_ERR_INVALID_ARG
    assert call(None, g=None) == kda.KDA_ERR_INVALID_ARG
    # segments: 0 .. 16; forcing needs few slices (here 1 x 2 x 8 = 16 <= 80)
    for bad in (kda.Options(segments=17), kda.Options(segments=-1)):
        assert call(ctypes.byref(bad)) == kda.KDA_ERR_INVALID_ARG
    assert call(ctypes.byref(kda.Options(segments=4))) == kda.KDA_ERR_WORKSPACE
    assert call(ctypes.byref(kda.Options(segments=16))) == kda.KDA_ERR_WORKSPACE
    assert call(ctypes.byref(kda.Options(segments=4)), H=16) == kda.KDA_ERR_INVALID_ARG   # 128 slices
    assert call(ctypes.byref(kda.Options(segments=1)), H=16) == kda.KDA_ERR_WORKSPACE
    # no gate: g may be NULL (the next failing check is the workspace)
    assert call(ctypes.byref(kda.Options(gate=kda.GATE_NONE)), g=None) == kda.KDA_ERR_WORKSPACE
    # valid descriptor: the next check that fails is the workspace size
    assert call(ctypes.byref(kda.Options(kda.FE_ALL, 1e-6))) == kda.KDA_ERR_WORKSPACE
    assert call(None) == kda.KDA_ERR_WORKSPACE
    assert call(None, Dk=64, Dv=64) == kda.KDA_ERR_UNSUPPORTED
