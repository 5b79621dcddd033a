"""Python binding of libkda (Kimi Delta Attention on MI355X).

Argument marshalling only: every call checks tensor shapes, dtypes and devices,
allocates outputs with torch, and passes raw device pointers plus the current
HIP stream to the C-ABI in ``libkda.so`` (declared in ``include/libkda.h``).
All arithmetic runs in the library's HIP kernels; there is no fallback.  If the
library is missing, loading fails with an error that says how to build it.

Entry points (same names as the C-ABI):
    prefill(q, k, v, log_alpha, beta, S0=None)        -> (o, S_T)
    prefill_noalloc(q, k, v, log_alpha, beta, S0=None)  -> (o, S_T)  (no workspace, allocates nothing)
    prefill_snap(q, k, v, log_alpha, beta, snap_interval, S0=None) -> (o, S_T, S_snap)
    prefill_plan(B, H, T, dk, dv, dtype)               -> (T0, G, Tseg)
    prefill_segments(q, k, v, log_alpha, beta, S_start, Tseg) -> (o, S_T)
    decode_step(q, k, v, log_alpha, beta, S)           -> o          (S updated in place)
    decode_tokens(q, k, v, log_alpha, beta, S, S_out=None, positions=False) -> (o, S_pos or None)
    segment_transfer(k, v, log_alpha, beta, G)         -> (S_zero_end, M)
    segment_merge(S_zero_end, M, S_in=None)            -> (S_start, S_T)
    prefill_backward(q, k, v, log_alpha, beta, S0, dO, dS_T) -> dict of gradients
    set_option(name, value), get_option(name), options(**values) (context manager)
"""
from __future__ import annotations

import contextlib
import ctypes
import os
from typing import Optional, Tuple

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libkda.so")

KDA_F32, KDA_BF16 = 0, 1
_DT = {torch.float32: KDA_F32, torch.bfloat16: KDA_BF16}
# status codes (include/libkda.h)
(KDA_OK, KDA_ERR_NULL, KDA_ERR_SHAPE, KDA_ERR_UNSUPPORTED, KDA_ERR_ALIGN, KDA_ERR_WORKSPACE,
 KDA_ERR_PRECONDITION, KDA_ERR_HIP) = range(8)

_lib = None


class KdaError(RuntimeError):
    """A libkda call returned a status other than KDA_OK (``status`` holds it;
    None for errors the binding itself raises)."""

    def __init__(self, msg: str, status: Optional[int] = None):
        super().__init__(msg)
        self.status = status


def lib_path() -> str:
    return LIB_PATH


def load() -> ctypes.CDLL:
    """Load libkda.so (built by ``python __graft_entry__.py`` / ``build.py``)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise KdaError(f"libkda.so not found at {LIB_PATH}; build it with "
                       "`python gated_delta_rule_104_amd/build.py` (hipcc, gfx950)")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i = ctypes.c_void_p, ctypes.c_int
    lib.kda_chunk_prefill.argtypes = [vp] * 8 + [i] * 6 + [vp, ctypes.c_size_t, vp]
    lib.kda_chunk_prefill_snap.argtypes = [vp] * 9 + [i] * 7 + [vp, ctypes.c_size_t, vp]
    lib.kda_chunk_prefill_noalloc.argtypes = [vp] * 8 + [i] * 6 + [vp]
    lib.kda_prefill_workspace_bytes.argtypes = [i] * 6
    lib.kda_prefill_workspace_bytes.restype = ctypes.c_size_t
    lib.kda_prefill_plan.argtypes = [i] * 6 + [ctypes.POINTER(i)] * 3
    lib.kda_chunk_prefill_segments.argtypes = [vp] * 8 + [i] * 7 + [vp]
    lib.kda_decode_step.argtypes = [vp] * 7 + [i] * 5 + [vp]
    lib.kda_decode_tokens.argtypes = [vp] * 9 + [i] * 6 + [vp]
    lib.kda_segment_transfer.argtypes = [vp] * 6 + [i] * 7 + [vp]
    lib.kda_segment_merge.argtypes = [vp] * 5 + [i] * 5 + [vp]
    lib.kda_backward_workspace_bytes.argtypes = [i] * 6
    lib.kda_backward_workspace_bytes.restype = ctypes.c_size_t
    lib.kda_prefill_backward.argtypes = [vp] * 14 + [i] * 6 + [vp, ctypes.c_size_t, vp]
    for f in (lib.kda_chunk_prefill, lib.kda_chunk_prefill_snap, lib.kda_chunk_prefill_noalloc, lib.kda_prefill_plan, lib.kda_chunk_prefill_segments,
              lib.kda_decode_step, lib.kda_decode_tokens, lib.kda_segment_transfer,
              lib.kda_segment_merge, lib.kda_prefill_backward):
        f.restype = i
    lib.kda_set_option.argtypes = [ctypes.c_char_p, ctypes.c_longlong]
    lib.kda_set_option.restype = i
    lib.kda_get_option.argtypes = [ctypes.c_char_p, ctypes.POINTER(ctypes.c_longlong)]
    lib.kda_get_option.restype = i
    lib.kda_status_string.argtypes = [i]
    lib.kda_status_string.restype = ctypes.c_char_p
    lib.kda_last_error.restype = ctypes.c_char_p
    lib.kda_abi_version.restype = i
    lib.kda_debug_time_main_launches.argtypes = [i]
    lib.kda_debug_time_main_launches.restype = i
    lib.kda_debug_main_launch_ms.argtypes = [ctypes.POINTER(ctypes.c_float), i, ctypes.POINTER(i)]
    lib.kda_debug_main_launch_ms.restype = i
    _lib = lib
    return lib


def _check(rc: int, what: str) -> None:
    if rc != 0:
        lib = load()
        raise KdaError(f"{what}: {lib.kda_status_string(rc).decode()} "
                       f"({lib.kda_last_error().decode()})", rc)


def set_option(name: str, value: Optional[int]) -> None:
    """Set a process-wide library option (kda_set_option); None restores the default."""
    _check(load().kda_set_option(name.encode(), -1 if value is None else int(value)), f"set_option({name})")


def get_option(name: str) -> Optional[int]:
    """The option's value in effect, or None for the library's default."""
    v = ctypes.c_longlong(0)
    _check(load().kda_get_option(name.encode(), ctypes.byref(v)), f"get_option({name})")
    return None if v.value == -1 else int(v.value)


def debug_time_main_launches(count: int) -> None:
    """Arm HIP events around the main launch of the next `count` sequence-split
    prefills (kda_debug_time_main_launches; 0 disarms)."""
    _check(load().kda_debug_time_main_launches(int(count)), "debug_time_main_launches")


def debug_main_launch_ms() -> list:
    """Durations (ms) of the main launches timed since the arming
    (kda_debug_main_launch_ms; waits for them)."""
    lib = load()
    n = ctypes.c_int(0)
    _check(lib.kda_debug_main_launch_ms(None, 0, ctypes.byref(n)), "debug_main_launch_ms")
    buf = (ctypes.c_float * max(n.value, 1))()
    _check(lib.kda_debug_main_launch_ms(buf, n.value, ctypes.byref(n)), "debug_main_launch_ms")
    return [float(buf[i]) for i in range(n.value)]


@contextlib.contextmanager
def options(**values):
    """Set options for the duration of a with-block, then restore the old values."""
    old = {n: get_option(n) for n in values}
    try:
        for n, v in values.items():
            set_option(n, v)
        yield
    finally:
        for n, v in old.items():
            set_option(n, v)


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _io(t: torch.Tensor, name: str, dtype: torch.dtype, shape) -> None:
    if not t.is_cuda:
        raise KdaError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise KdaError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if tuple(t.shape) != tuple(shape):
        raise KdaError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise KdaError(f"{name} must be contiguous")


def prefill_workspace_bytes(B: int, H: int, T: int, dk: int, dv: int, dtype: torch.dtype) -> int:
    """Workspace that lets kda_chunk_prefill use its sequence-split path (0 if unused)."""
    if dtype not in _DT:
        raise KdaError(f"unsupported dtype {dtype}")
    return int(load().kda_prefill_workspace_bytes(B, H, T, dk, dv, _DT[dtype]))


def prefill(q, k, v, log_alpha, beta, S0=None, o=None, S_T=None,
            workspace="auto") -> Tuple[torch.Tensor, torch.Tensor]:
    """Chunked prefill.  q, k, log_alpha [B,H,T,dk]; v [B,H,T,dv]; beta [B,H,T];
    S0 [B,H,dk,dv] fp32 or None.  Returns o [B,H,T,dv] (input dtype) and S_T fp32.
    workspace: "auto" allocates what kda_prefill_workspace_bytes asks for, None
    passes none (single-pass path), or a device uint8 tensor to use."""
    B, H, T, dk = k.shape
    dv = v.shape[-1]
    dt = k.dtype
    if dt not in _DT:
        raise KdaError(f"unsupported dtype {dt}")
    for name, t, shp in (("q", q, (B, H, T, dk)), ("k", k, (B, H, T, dk)), ("v", v, (B, H, T, dv)),
                         ("log_alpha", log_alpha, (B, H, T, dk)), ("beta", beta, (B, H, T))):
        _io(t, name, dt, shp)
    if S0 is not None:
        _io(S0, "S0", torch.float32, (B, H, dk, dv))
    if o is None:
        o = torch.empty(B, H, T, dv, dtype=dt, device=k.device)
    if S_T is None:
        S_T = torch.empty(B, H, dk, dv, dtype=torch.float32, device=k.device)
    _io(o, "o", dt, (B, H, T, dv))
    _io(S_T, "S_T", torch.float32, (B, H, dk, dv))
    if isinstance(workspace, str):
        nbytes = prefill_workspace_bytes(B, H, T, dk, dv, dt)
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=k.device) if nbytes else None
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    rc = load().kda_chunk_prefill(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(S0),
                                  _ptr(o), _ptr(S_T), B, H, T, dk, dv, _DT[dt], _ptr(workspace),
                                  ws_bytes, _stream())
    _check(rc, "kda_chunk_prefill")
    return o, S_T


def prefill_noalloc(q, k, v, log_alpha, beta, S0=None, o=None, S_T=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """prefill() through kda_chunk_prefill_noalloc: the library's own scratch
    array replaces the workspace (calls on one device must not overlap).  o and
    S_T are allocated here when not given; pass them to allocate nothing."""
    B, H, T, dk = k.shape
    dv = v.shape[-1]
    dt = k.dtype
    if dt not in _DT:
        raise KdaError(f"unsupported dtype {dt}")
    for name, t, shp in (("q", q, (B, H, T, dk)), ("k", k, (B, H, T, dk)), ("v", v, (B, H, T, dv)),
                         ("log_alpha", log_alpha, (B, H, T, dk)), ("beta", beta, (B, H, T))):
        _io(t, name, dt, shp)
    if S0 is not None:
        _io(S0, "S0", torch.float32, (B, H, dk, dv))
    if o is None:
        o = torch.empty(B, H, T, dv, dtype=dt, device=k.device)
    if S_T is None:
        S_T = torch.empty(B, H, dk, dv, dtype=torch.float32, device=k.device)
    _io(o, "o", dt, (B, H, T, dv))
    _io(S_T, "S_T", torch.float32, (B, H, dk, dv))
    rc = load().kda_chunk_prefill_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(S0),
                                          _ptr(o), _ptr(S_T), B, H, T, dk, dv, _DT[dt], _stream())
    _check(rc, "kda_chunk_prefill_noalloc")
    return o, S_T


def prefill_snap(q, k, v, log_alpha, beta, snap_interval: int, S0=None, o=None, S_T=None,
                 S_snap=None, workspace="auto"):
    """Chunked prefill that also returns state snapshots for prefix caching:
    S_snap [B, T // snap_interval, H, dk, dv] fp32, entry [b, j, h] being the state
    after the first (j + 1) * snap_interval tokens (snap_interval: a positive
    multiple of 64).  Returns (o, S_T, S_snap); o and S_T are those of prefill()."""
    B, H, T, dk = k.shape
    dv = v.shape[-1]
    dt = k.dtype
    if dt not in _DT:
        raise KdaError(f"unsupported dtype {dt}")
    if snap_interval <= 0 or snap_interval % 64:
        raise KdaError(f"snap_interval must be a positive multiple of 64 (got {snap_interval})")
    for name, t, shp in (("q", q, (B, H, T, dk)), ("k", k, (B, H, T, dk)), ("v", v, (B, H, T, dv)),
                         ("log_alpha", log_alpha, (B, H, T, dk)), ("beta", beta, (B, H, T))):
        _io(t, name, dt, shp)
    if S0 is not None:
        _io(S0, "S0", torch.float32, (B, H, dk, dv))
    nsnap = T // snap_interval
    if o is None:
        o = torch.empty(B, H, T, dv, dtype=dt, device=k.device)
    if S_T is None:
        S_T = torch.empty(B, H, dk, dv, dtype=torch.float32, device=k.device)
    if S_snap is None:
        S_snap = torch.empty(B, nsnap, H, dk, dv, dtype=torch.float32, device=k.device)
    _io(o, "o", dt, (B, H, T, dv))
    _io(S_T, "S_T", torch.float32, (B, H, dk, dv))
    _io(S_snap, "S_snap", torch.float32, (B, nsnap, H, dk, dv))
    if isinstance(workspace, str):
        nbytes = prefill_workspace_bytes(B, H, T, dk, dv, dt)
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=k.device) if nbytes else None
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    rc = load().kda_chunk_prefill_snap(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta),
                                       _ptr(S0), _ptr(o), _ptr(S_T), _ptr(S_snap) if nsnap else None,
                                       snap_interval, B, H, T, dk, dv, _DT[dt], _ptr(workspace),
                                       ws_bytes, _stream())
    _check(rc, "kda_chunk_prefill_snap")
    return o, S_T, S_snap


def prefill_plan(B: int, H: int, T: int, dk: int, dv: int, dtype: torch.dtype) -> Tuple[int, int, int]:
    """(T0, G, Tseg): the cut kda_chunk_prefill uses with its workspace: a first
    part of T0 tokens, then G segments of Tseg tokens (T0 == 0, G == 1: single pass)."""
    if dtype not in _DT:
        raise KdaError(f"unsupported dtype {dtype}")
    T0, G, Tseg = ctypes.c_int(0), ctypes.c_int(0), ctypes.c_int(0)
    _check(load().kda_prefill_plan(B, H, T, dk, dv, _DT[dtype], ctypes.byref(T0), ctypes.byref(G),
                                   ctypes.byref(Tseg)), "kda_prefill_plan")
    return T0.value, G.value, Tseg.value


def prefill_segments(q, k, v, log_alpha, beta, S_start, Tseg: int, o=None, S_T=None):
    """Prefill of the G = ceil(T / Tseg) segments of every head, segment i from
    S_start[i] ([G,B,H,dk,dv] fp32, or None for zero).  Returns (o, S_T of the
    last segment)."""
    B, H, T, dk = k.shape
    dv = v.shape[-1]
    dt = k.dtype
    if dt not in _DT:
        raise KdaError(f"unsupported dtype {dt}")
    if Tseg < 1 or T < 1:
        raise KdaError(f"need T >= 1 and Tseg >= 1 (T={T}, Tseg={Tseg})")
    G = -(-T // Tseg)
    for name, t, shp in (("q", q, (B, H, T, dk)), ("k", k, (B, H, T, dk)), ("v", v, (B, H, T, dv)),
                         ("log_alpha", log_alpha, (B, H, T, dk)), ("beta", beta, (B, H, T))):
        _io(t, name, dt, shp)
    if S_start is not None:
        _io(S_start, "S_start", torch.float32, (G, B, H, dk, dv))
    if o is None:
        o = torch.empty(B, H, T, dv, dtype=dt, device=k.device)
    if S_T is None:
        S_T = torch.empty(B, H, dk, dv, dtype=torch.float32, device=k.device)
    _io(o, "o", dt, (B, H, T, dv))
    _io(S_T, "S_T", torch.float32, (B, H, dk, dv))
    rc = load().kda_chunk_prefill_segments(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta),
                                           _ptr(S_start), _ptr(o), _ptr(S_T), B, H, T, Tseg, dk, dv,
                                           _DT[dt], _stream())
    _check(rc, "kda_chunk_prefill_segments")
    return o, S_T


def decode_step(q, k, v, log_alpha, beta, S, o=None) -> torch.Tensor:
    """One token for N*H heads.  q, k, log_alpha [N,H,dk]; v [N,H,dv]; beta [N,H];
    S [N,H,dk,dv] fp32, updated in place.  Returns o [N,H,dv]."""
    N, H, dk = k.shape
    dv = v.shape[-1]
    dt = k.dtype
    if dt not in _DT:
        raise KdaError(f"unsupported dtype {dt}")
    for name, t, shp in (("q", q, (N, H, dk)), ("k", k, (N, H, dk)), ("v", v, (N, H, dv)),
                         ("log_alpha", log_alpha, (N, H, dk)), ("beta", beta, (N, H))):
        _io(t, name, dt, shp)
    _io(S, "S", torch.float32, (N, H, dk, dv))
    if o is None:
        o = torch.empty(N, H, dv, dtype=dt, device=k.device)
    _io(o, "o", dt, (N, H, dv))
    rc = load().kda_decode_step(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(S),
                                _ptr(o), N, H, dk, dv, _DT[dt], _stream())
    _check(rc, "kda_decode_step")
    return o


def decode_tokens(q, k, v, log_alpha, beta, S, S_out=None, positions: bool = False, o=None, S_pos=None):
    """ntok consecutive tokens per sequence in one pass over the state (speculative
    decoding's verification step).  q, k, log_alpha [N,H,ntok,dk]; v [N,H,ntok,dv];
    beta [N,H,ntok]; S [N,H,dk,dv] fp32.  The state after the tokens goes to S_out
    (default: S itself, in place).  With positions=True (or an S_pos tensor) the
    state after each token is returned too, [N,ntok,H,dk,dv].  Returns (o, S_pos)."""
    N, H, ntok, dk = k.shape
    dv = v.shape[-1]
    dt = k.dtype
    if dt not in _DT:
        raise KdaError(f"unsupported dtype {dt}")
    for name, t, shp in (("q", q, (N, H, ntok, dk)), ("k", k, (N, H, ntok, dk)), ("v", v, (N, H, ntok, dv)),
                         ("log_alpha", log_alpha, (N, H, ntok, dk)), ("beta", beta, (N, H, ntok))):
        _io(t, name, dt, shp)
    _io(S, "S", torch.float32, (N, H, dk, dv))
    if S_out is None:
        S_out = S
    _io(S_out, "S_out", torch.float32, (N, H, dk, dv))
    if o is None:
        o = torch.empty(N, H, ntok, dv, dtype=dt, device=k.device)
    _io(o, "o", dt, (N, H, ntok, dv))
    if S_pos is None and positions:
        S_pos = torch.empty(N, ntok, H, dk, dv, dtype=torch.float32, device=k.device)
    if S_pos is not None:
        _io(S_pos, "S_pos", torch.float32, (N, ntok, H, dk, dv))
    rc = load().kda_decode_tokens(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(S),
                                  _ptr(S_out), _ptr(o), _ptr(S_pos), N, H, ntok, dk, dv, _DT[dt], _stream())
    _check(rc, "kda_decode_tokens")
    return o, S_pos


def segment_transfer(k, v, log_alpha, beta, G: int, S_zero_end=None, M=None):
    """Per-segment zero-start end states [G,B,H,dk,dv] and transfer maps [G,B,H,dk,dk]
    for sequences of T = G * Tseg tokens."""
    B, H, T, dk = k.shape
    dv = v.shape[-1]
    dt = k.dtype
    if dt not in _DT:
        raise KdaError(f"unsupported dtype {dt}")
    if G <= 0 or T % G:
        raise KdaError(f"T={T} is not a positive multiple of G={G}")
    for name, t, shp in (("k", k, (B, H, T, dk)), ("v", v, (B, H, T, dv)),
                         ("log_alpha", log_alpha, (B, H, T, dk)), ("beta", beta, (B, H, T))):
        _io(t, name, dt, shp)
    if S_zero_end is None:
        S_zero_end = torch.empty(G, B, H, dk, dv, dtype=torch.float32, device=k.device)
    if M is None:
        M = torch.empty(G, B, H, dk, dk, dtype=torch.float32, device=k.device)
    _io(S_zero_end, "S_zero_end", torch.float32, (G, B, H, dk, dv))
    _io(M, "M", torch.float32, (G, B, H, dk, dk))
    rc = load().kda_segment_transfer(_ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(S_zero_end),
                                     _ptr(M), B, H, G, T // G, dk, dv, _DT[dt], _stream())
    _check(rc, "kda_segment_transfer")
    return S_zero_end, M


def segment_merge(S_zero_end, M, S_in=None, want_start: bool = True, S_start=None, S_T=None):
    """Sequential merge.  Returns (S_start [G,B,H,dk,dv] or None, S_T [B,H,dk,dv])."""
    G, B, H, dk, dv = S_zero_end.shape
    _io(S_zero_end, "S_zero_end", torch.float32, (G, B, H, dk, dv))
    _io(M, "M", torch.float32, (G, B, H, dk, dk))
    if S_in is not None:
        _io(S_in, "S_in", torch.float32, (B, H, dk, dv))
    if want_start and S_start is None:
        S_start = torch.empty_like(S_zero_end)
    if S_start is not None:
        _io(S_start, "S_start", torch.float32, (G, B, H, dk, dv))
    if S_T is None:
        S_T = torch.empty(B, H, dk, dv, dtype=torch.float32, device=M.device)
    _io(S_T, "S_T", torch.float32, (B, H, dk, dv))
    rc = load().kda_segment_merge(_ptr(S_in), _ptr(S_zero_end), _ptr(M), _ptr(S_start), _ptr(S_T),
                                  B, H, G, dk, dv, _stream())
    _check(rc, "kda_segment_merge")
    return S_start, S_T


def backward_workspace_bytes(B: int, H: int, T: int, dk: int, dv: int, dtype: torch.dtype = torch.bfloat16) -> int:
    """Workspace kda_prefill_backward needs for inputs of this dtype (0 for an unsupported shape)."""
    if dtype not in _DT:
        raise KdaError(f"unsupported dtype {dtype}")
    return int(load().kda_backward_workspace_bytes(B, H, T, dk, dv, _DT[dtype]))


def prefill_backward(q, k, v, log_alpha, beta, S0=None, dO=None, dS_T=None, workspace=None):
    """Gradients of L = sum(dO * o) + sum(dS_T * S_T) of the prefill with respect
    to its inputs.  Returns a dict: dq, dk, dlog_alpha [B,H,T,dk], dv [B,H,T,dv],
    dbeta [B,H,T] in the inputs' dtype, and dS0 [B,H,dk,dv] fp32."""
    B, H, T, dk = k.shape
    dv = v.shape[-1]
    dt = k.dtype
    if dt not in _DT:
        raise KdaError(f"unsupported dtype {dt}")
    for t, n, shp in ((q, "q", (B, H, T, dk)), (k, "k", (B, H, T, dk)), (v, "v", (B, H, T, dv)),
                      (log_alpha, "log_alpha", (B, H, T, dk)), (beta, "beta", (B, H, T))):
        _io(t, n, dt, shp)
    if S0 is not None:
        _io(S0, "S0", torch.float32, (B, H, dk, dv))
    if dO is not None:
        _io(dO, "dO", dt, (B, H, T, dv))
    if dS_T is not None:
        _io(dS_T, "dS_T", torch.float32, (B, H, dk, dv))
    dev = k.device
    io = dict(dtype=dt, device=dev)
    out = dict(dq=torch.empty(B, H, T, dk, **io), dk=torch.empty(B, H, T, dk, **io),
               dv=torch.empty(B, H, T, dv, **io), dlog_alpha=torch.empty(B, H, T, dk, **io),
               dbeta=torch.empty(B, H, T, **io), dS0=torch.empty(B, H, dk, dv, dtype=torch.float32, device=dev))
    need = backward_workspace_bytes(B, H, T, dk, dv, dt)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    if not workspace.is_cuda or workspace.numel() * workspace.element_size() < need:
        raise KdaError(f"workspace must be a device tensor of at least {need} bytes")
    rc = load().kda_prefill_backward(_ptr(q), _ptr(k), _ptr(v), _ptr(log_alpha), _ptr(beta), _ptr(S0), _ptr(dO),
                                     _ptr(dS_T), _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"]),
                                     _ptr(out["dlog_alpha"]), _ptr(out["dbeta"]), _ptr(out["dS0"]), B, H, T, dk, dv,
                                     _DT[dt], _ptr(workspace), workspace.numel() * workspace.element_size(),
                                     _stream())
    _check(rc, "kda_prefill_backward")
    return out
