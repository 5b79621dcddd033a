"""CPU tests of the C-ABI boundary: the library loads, exports every entry point
that include/libkda.h declares, and rejects invalid arguments on the host before
anything would be launched (these calls never reach the GPU)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "libkda.h")

import gated_delta_rule_104_amd as kda  # noqa: E402

OK, ERR_NULL, ERR_SHAPE, ERR_UNSUPPORTED, ERR_ALIGN, ERR_WORKSPACE, ERR_PRECONDITION, ERR_HIP = range(8)
F32, BF16 = 0, 1
FAKE = 0x100000  # 16-byte aligned, never dereferenced: validation fails first


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(kda.lib_path()):
        from gated_delta_rule_104_amd import build
        build.build()
    return kda.load()


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(kda_[a-z_]+)\s*\(", src)))


def test_header_declares_the_four_calls():
    names = declared_functions()
    for n in ("kda_chunk_prefill", "kda_decode_step", "kda_segment_transfer", "kda_segment_merge"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_version_and_status_strings(lib):
    assert lib.kda_abi_version() == 8
    names = [lib.kda_status_string(st) for st in range(8)]
    assert all(names) and len(set(names)) == 8
    assert b"workspace" in names[ERR_WORKSPACE] and b"precondition" in names[ERR_PRECONDITION]
    assert b"HIP" in names[ERR_HIP]
    assert lib.kda_status_string(99) == b"unknown status"


def P(*xs):
    return [ctypes.c_void_p(x) if x is not None else None for x in xs]


def prefill(lib, q=FAKE, k=FAKE, v=FAKE, la=FAKE, beta=FAKE, S0=None, o=FAKE, ST=FAKE,
            B=1, H=1, T=64, dk=64, dv=64, dt=BF16):
    return lib.kda_chunk_prefill(*P(q, k, v, la, beta, S0, o, ST), B, H, T, dk, dv, dt, None, 0, None)


def test_prefill_validation(lib):
    assert prefill(lib, dk=64, dv=128) == ERR_SHAPE
    assert prefill(lib, dk=96, dv=96) == ERR_UNSUPPORTED
    assert prefill(lib, dk=96, dv=96, dt=F32) == ERR_UNSUPPORTED
    assert prefill(lib, dt=7) == ERR_UNSUPPORTED
    assert prefill(lib, T=-1) == ERR_SHAPE
    assert prefill(lib, B=-2) == ERR_SHAPE
    assert prefill(lib, q=None) == ERR_NULL
    assert prefill(lib, ST=None) == ERR_NULL
    assert prefill(lib, beta=FAKE + 4) == ERR_ALIGN
    assert prefill(lib, S0=FAKE + 8) == ERR_ALIGN
    assert b"16-byte" in lib.kda_last_error()
    assert prefill(lib, B=1 << 20, H=1 << 10, T=1 << 20) == ERR_SHAPE
    assert prefill(lib, B=1, H=1, T=1 << 23, dk=128, dv=128) == ERR_UNSUPPORTED
    assert lib.kda_chunk_prefill(*P(FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE), 1, 1, 64, 64, 64,
                                 BF16, ctypes.c_void_p(FAKE + 8), 1024, None) == ERR_ALIGN
    # nothing to do: no heads
    assert prefill(lib, B=0) == OK


STATE = 32 * 128 * 128 * 4  # bytes of one fp32 state per head, 32 heads
FLAG_SLOTS = 8              # words of one segment record


def split_ws(g, fixup=True, bh=32, d=128):
    """Workspace of the split path for g segments: Z of all g, M and start states
    of the g - 1 after the first, and their records (fixup); Z and M of g - 1
    segments, the first part's end state and g start states (fixup = 0)."""
    if fixup:
        return (3 * g - 2) * bh * d * d * 4 + (g - 1) * bh * FLAG_SLOTS * 4
    return (3 * g - 1) * bh * d * d * 4


def test_prefill_workspace_query(lib, kda_opts):
    """The sequence-split path asks for its states and segment records (see
    split_ws); it is not used for fp32 inputs, short sequences or many heads."""
    ws = lib.kda_prefill_workspace_bytes
    ws.restype = ctypes.c_size_t
    for fixup in (None, 0):
        kda_opts("fixup", fixup)
        assert ws(1, 32, 65536, 128, 128, F32) == 0
        assert ws(1, 32, 1024, 128, 128, BF16) == 0
        assert ws(64, 32, 65536, 128, 128, BF16) == 0
        assert ws(1, 32, 65536, 128, 64, BF16) == 0
    kda_opts("fixup", None)
    assert ws(1, 32, 65536, 128, 128, BF16) == split_ws(8)
    kda_opts("fixup", 0)
    n = ws(1, 32, 65536, 128, 128, BF16)
    assert n > 0 and n % STATE == 0 and (n // STATE) % 3 == 2


def test_prefill_plan(lib, kda_opts):
    """The plan matches the workspace query: split exactly when workspace is asked
    for; the first part (none by default: segment 0 starts from S0) and the
    segments are whole chunks and cover T exactly, the last segment being the
    only short one."""
    T0, G, Ts = ctypes.c_int(0), ctypes.c_int(0), ctypes.c_int(0)
    plan = lambda *a: lib.kda_prefill_plan(*a, ctypes.byref(T0), ctypes.byref(G), ctypes.byref(Ts))
    ws = lib.kda_prefill_workspace_bytes
    ws.restype = ctypes.c_size_t
    for fixup in (None, 0):
        kda_opts("fixup", fixup)
        for T in (4096, 10000, 65536, 1 << 20):
            assert plan(1, 32, T, 128, 128, BF16) == OK
            t0, g, ts = T0.value, G.value, Ts.value
            assert g > 1 and ts % 64 == 0 and t0 % 64 == 0 and (t0 == 0) == (fixup is None), (T, t0, g, ts)
            assert t0 + (g - 1) * ts < T <= t0 + g * ts, (T, t0, g, ts)
            assert ws(1, 32, T, 128, 128, BF16) == split_ws(g, fixup is None)
    kda_opts("fixup", None)
    assert plan(1, 32, 65536, 128, 128, BF16) == OK and (T0.value, G.value, Ts.value) == (0, 8, 8192)
    assert plan(64, 32, 65536, 128, 128, BF16) == OK and (T0.value, G.value, Ts.value) == (0, 1, 65536)
    assert plan(1, 32, 65536, 128, 128, F32) == OK and (T0.value, G.value) == (0, 1)
    assert plan(1, 32, 100, 96, 96, BF16) == ERR_UNSUPPORTED
    assert lib.kda_prefill_plan(1, 1, 64, 64, 64, BF16, None, ctypes.byref(G), ctypes.byref(Ts)) == ERR_NULL


def test_prefill_plan_cost_override(lib, kda_opts):
    """Option transfer_cost16 (the segment pass's cost per token relative to
    the prefill, in 16ths) moves the first part's length of the fixup = 0 plan;
    the cut still covers T exactly, and values outside 1..64 are refused."""
    T0, G, Ts = ctypes.c_int(0), ctypes.c_int(0), ctypes.c_int(0)
    kda_opts("fixup", 0)

    def plan(T=65536):
        assert lib.kda_prefill_plan(1, 32, T, 128, 128, BF16, ctypes.byref(T0), ctypes.byref(G),
                                    ctypes.byref(Ts)) == OK
        return T0.value, G.value, Ts.value

    kda_opts("transfer_cost16", None)
    default = plan()
    first = {}
    for c in (11, 15, 19):
        kda_opts("transfer_cost16", c)
        t0, g, ts = plan()
        assert t0 % 64 == 0 and ts % 64 == 0 and t0 + (g - 1) * ts < 65536 <= t0 + g * ts
        first[c] = t0 / ts
    assert first[11] < first[15] < first[19]
    kda_opts("transfer_cost16", 12)
    assert plan() == default
    for bad in (0, 65, -3):
        assert lib.kda_set_option(b"transfer_cost16", bad) == ERR_SHAPE
        assert plan() == default


def test_prefill_snap_validation(lib):
    """Snapshot interval: 0 (none) or a positive multiple of the 64-token chunk;
    the snapshot buffer is required only when at least one snapshot falls in T."""
    f = lib.kda_chunk_prefill_snap
    args = lambda **kw: [*P(FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, kw.get("snap", FAKE)),
                         kw.get("iv", 512), 1, 2, kw.get("T", 1024), 128, 128, BF16, None, 0, None]
    assert f(*args(iv=-64)) == ERR_SHAPE
    assert f(*args(iv=100)) == ERR_SHAPE
    assert b"multiple of 64" in lib.kda_last_error()
    assert f(*args(snap=None)) == ERR_NULL
    assert f(*args(snap=FAKE + 8)) == ERR_ALIGN
    # T = 0 with any valid interval and no heads: nothing to launch
    assert f(*[*P(FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, None), 512, 0, 2, 1024, 128, 128,
               BF16, None, 0, None]) == OK
    # shape errors of the plain prefill come first
    assert f(*[*P(FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE), 512, 1, 2, 1024, 128, 64,
               BF16, None, 0, None]) == ERR_SHAPE


def test_prefill_segments_validation(lib):
    f = lib.kda_chunk_prefill_segments
    args = lambda **kw: [*P(FAKE, FAKE, FAKE, FAKE, FAKE, kw.get("S", None), FAKE, kw.get("ST", FAKE)),
                         1, 2, kw.get("T", 256), kw.get("Tseg", 64), kw.get("dk", 128), 128,
                         kw.get("dt", BF16), None]
    assert f(*args(Tseg=0)) == ERR_SHAPE
    assert f(*args(T=0)) == ERR_SHAPE
    assert f(*args(ST=None)) == ERR_NULL
    assert f(*args(S=FAKE + 4)) == ERR_ALIGN
    assert f(*args(dk=64)) == ERR_SHAPE
    assert f(*args(dt=5)) == ERR_UNSUPPORTED


def test_decode_validation(lib):
    f = lib.kda_decode_step
    assert f(*P(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE), 4, 2, 128, 64, BF16, None) == ERR_SHAPE
    assert f(*P(FAKE, FAKE, None, FAKE, FAKE, FAKE, FAKE), 4, 2, 128, 128, BF16, None) == ERR_NULL
    assert f(*P(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE + 4, FAKE), 4, 2, 64, 64, F32, None) == ERR_ALIGN
    assert f(*P(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE), -1, 2, 64, 64, F32, None) == ERR_SHAPE
    assert f(*P(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE), 0, 2, 64, 64, F32, None) == OK


def test_decode_tokens_validation(lib):
    f = lib.kda_decode_tokens
    a = lambda *p, N=4, H=2, n=3, dk=128, dv=128, dt=BF16: [*P(*p), N, H, n, dk, dv, dt, None]
    full = (FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None)
    assert f(*a(*full, dv=64)) == ERR_SHAPE
    assert f(*a(*full, n=-1)) == ERR_SHAPE
    assert f(*a(FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, None)) == ERR_NULL  # S_in
    assert f(*a(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, None)) == ERR_NULL  # S_out
    assert f(*a(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE + 4)) == ERR_ALIGN  # S_pos
    assert f(*a(FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None)) == ERR_NULL
    assert f(*a(*full, dt=9)) == ERR_UNSUPPORTED
    assert f(*a(*full, N=0)) == OK


def test_segment_validation(lib):
    t = lib.kda_segment_transfer
    assert t(*P(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE), 1, 2, 4, 0, 128, 128, BF16, None) == ERR_SHAPE
    assert t(*P(FAKE, FAKE, FAKE, FAKE, None, FAKE), 1, 2, 4, 64, 128, 128, BF16, None) == ERR_NULL
    assert t(*P(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE), 1, 2, 4, 64, 96, 96, F32, None) == ERR_UNSUPPORTED
    assert t(*P(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE), 1, 2, 4, 64, 128, 128, 3, None) == ERR_UNSUPPORTED
    m = lib.kda_segment_merge
    assert m(*P(None, FAKE, FAKE, None, None), 1, 2, 4, 128, 128, None) == ERR_NULL
    assert m(*P(None, FAKE, FAKE, FAKE + 4, FAKE), 1, 2, 4, 128, 128, None) == ERR_ALIGN
    assert m(*P(None, FAKE, FAKE, None, FAKE), 1, 2, 4, 64, 128, None) == ERR_SHAPE


def test_binding_rejects_host_tensors():
    import torch
    x = torch.zeros(1, 1, 4, 64)
    with pytest.raises(kda.KdaError):
        kda.prefill(x, x, x, x, torch.zeros(1, 1, 4))


def backward(lib, q=FAKE, k=FAKE, v=FAKE, la=FAKE, beta=FAKE, S0=None, dO=FAKE, dST=None,
             dq=FAKE, dk=FAKE, dv=FAKE, dla=FAKE, db=FAKE, dS0=FAKE, B=1, H=1, T=64, D=64, dt=BF16,
             ws=FAKE, ws_bytes=None):
    if ws_bytes is None:
        ws_bytes = lib.kda_backward_workspace_bytes(B, H, T, D, D, dt)
    return lib.kda_prefill_backward(*P(q, k, v, la, beta, S0, dO, dST, dq, dk, dv, dla, db, dS0),
                                    B, H, T, D, D, dt, ctypes.c_void_p(ws) if ws else None, ws_bytes, None)


def test_backward_workspace_query(lib):
    """bf16 (chunked form): per chunk the start state and dS' (bf16 D x D each),
    W, Delta, Xbar (bf16 64 x D each) and the 10 lower 16x16 blocks of
    strict_lower(Kh Kb^T) (bf16), and one discarded fp32 end state per head.  fp32 (token steps):
    a checkpoint every 64 tokens plus 64 entering states (fp32 D x D) and 64
    fp32 D-vectors per head, then, with two workgroups per head (few heads),
    the second one's row sums of every token (dq, dk, dlog_alpha, dbeta:
    3D + 1 floats); with one workgroup per head none."""
    q = lib.kda_backward_workspace_bytes
    q.restype = ctypes.c_size_t
    kda.set_option("bw_split", None)  # the default: two workgroups per head while 2 B H fits the CUs
    assert q(1, 1, 64, 64, 64, F32) == ((1 + 64) * 64 * 64 + 64 * 64 + 64 * (3 * 64 + 1)) * 4
    assert q(2, 3, 65, 128, 128, F32) == 6 * ((2 + 64) * 128 * 128 + 64 * 128 + 65 * (3 * 128 + 1)) * 4
    assert q(64, 32, 65, 128, 128, F32) == 2048 * ((2 + 64) * 128 * 128 + 64 * 128) * 4
    assert q(1, 1, 0, 64, 64, F32) == (64 * 64 * 64 + 64 * 64) * 4
    def chunked(BH, nch, D):
        return BH * (nch * (2 * D * D + 3 * 64 * D + 10 * 256) * 2 + D * D * 4)
    assert q(1, 1, 64, 64, 64, BF16) == chunked(1, 1, 64) == 62464
    assert q(2, 3, 65, 128, 128, BF16) == chunked(6, 2, 128)
    assert q(4, 32, 8192, 128, 128, BF16) == chunked(128, 128, 128)
    assert q(1, 1, 0, 64, 64, BF16) == 64 * 64 * 4
    assert q(1, 1, 64, 64, 128, BF16) == 0 and q(1, 1, 64, 96, 96, F32) == 0 and q(0, 1, 64, 64, 64, BF16) == 0
    assert q(1, 1, 64, 64, 64, 5) == 0


def test_backward_validation(lib):
    assert backward(lib, D=96) == ERR_UNSUPPORTED
    assert backward(lib, dt=7) == ERR_UNSUPPORTED
    assert backward(lib, T=-1, ws_bytes=0) == ERR_SHAPE
    assert backward(lib, q=None) == ERR_NULL
    assert backward(lib, dS0=None) == ERR_NULL
    assert backward(lib, db=None) == ERR_NULL
    assert backward(lib, ws=None) == ERR_WORKSPACE
    assert backward(lib, ws_bytes=1024) == ERR_WORKSPACE
    assert b"needed" in lib.kda_last_error()
    assert backward(lib, ws=FAKE + 8) == ERR_ALIGN
    assert backward(lib, dq=FAKE + 4) == ERR_ALIGN
    assert backward(lib, dO=FAKE + 8) == ERR_ALIGN
    assert backward(lib, B=1 << 20, H=1 << 12, T=1 << 10) == ERR_SHAPE
    # no tokens: the per-token arrays are not needed, the workspace still is
    assert backward(lib, T=0, q=None, k=None, v=None, la=None, beta=None, dO=None, dq=None, dk=None,
                    dv=None, dla=None, db=None, ws=None) == ERR_WORKSPACE
    # no heads: nothing to do
    assert backward(lib, B=0, ws=None, ws_bytes=0) == OK


def test_main_launch_timer_validation(lib):
    """The main-launch timer checks its arguments on the host; disarming and
    reading back nothing touch no device."""
    n = ctypes.c_int(-1)
    assert lib.kda_debug_time_main_launches(-1) == ERR_SHAPE
    assert lib.kda_debug_time_main_launches(257) == ERR_SHAPE
    assert lib.kda_debug_time_main_launches(0) == OK
    assert lib.kda_debug_main_launch_ms(None, 0, ctypes.byref(n)) == OK and n.value == 0
    assert lib.kda_debug_main_launch_ms(None, 0, None) == ERR_NULL
    assert lib.kda_debug_main_launch_ms(None, 1, ctypes.byref(n)) == ERR_NULL
    buf = (ctypes.c_float * 1)()
    assert lib.kda_debug_main_launch_ms(buf, -1, ctypes.byref(n)) == ERR_SHAPE


def test_options(lib, kda_opts):
    """Options are validated by name and value, read back as set, and -1 restores
    the library default; calls that only validate are unaffected."""
    v = ctypes.c_longlong(0)
    get = lambda n: (lib.kda_get_option(n, ctypes.byref(v)), v.value)[1]
    for name, good, bad in ((b"split", (0, 2, 64), (1, -2)), (b"transfer_cost16", (1, 64), (0, 65)),
                            (b"map_skip", (0, 1), (2,)), (b"nc", (1, 2, 4, 8), (3, 16)),
                            (b"bw_split", (1, 2), (3,)), (b"check", (0, 1), (2,)), (b"log", (0, 1), (5,)),
                            (b"fixup", (0, 1), (2,)), (b"head_chunks", (1, 4, 1024), (0, 1025)),
                            (b"bw_overlap", (0, 1), (2,))):
        kda_opts(name.decode(), None)
        assert get(name) == -1
        for x in good:
            assert lib.kda_set_option(name, x) == OK and get(name) == x
        for x in bad:
            assert lib.kda_set_option(name, x) == ERR_SHAPE and get(name) == good[-1]
        assert lib.kda_set_option(name, -1) == OK and get(name) == -1
    assert lib.kda_set_option(b"no_such_option", 1) == ERR_SHAPE
    assert b"unknown option" in lib.kda_last_error()
    assert lib.kda_get_option(b"no_such_option", ctypes.byref(v)) == ERR_SHAPE
    assert lib.kda_set_option(None, 1) == ERR_NULL
    assert lib.kda_get_option(b"nc", None) == ERR_NULL


def test_options_from_environment():
    """Each option starts from its KDA_* environment variable, read once; values
    an option does not take are ignored (the default applies)."""
    import subprocess
    import sys
    code = ("import gated_delta_rule_104_amd as k; "
            "print(k.get_option('nc'), k.get_option('split'), k.get_option('check'), k.get_option('log'), "
            "k.get_option('map_skip'))")
    env = dict(os.environ, KDA_NC="2", KDA_SPLIT="1", KDA_CHECK="1", KDA_LOG="yes", KDA_MAP_SKIP="0")
    out = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True, text=True,
                         check=True, timeout=120).stdout.split()
    assert out == ["2", "None", "1", "1", "0"], out
