"""fp64 CPU oracle for Kimi Delta Attention -- TEST INFRASTRUCTURE.

Only tests/, ``__graft_entry__.smoke()`` and bench.py's ``cpu_baseline`` leg may
import this package.  The GPU library never calls it and shares no code with it.

The arithmetic lives in ``kda_oracle.c`` (plain token-by-token fp64 recurrence,
see the comment at its top for the equations and the passages they follow).
This module only marshals numpy/torch arrays into fp64 and calls it.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libkda_oracle.so")

_lib_cache = {}


def load(path: str = LIB_PATH):
    """Load (building first if absent) the oracle library at ``path``."""
    if path in _lib_cache:
        return _lib_cache[path]
    if not os.path.exists(path):
        from . import build_oracle
        build_oracle.build(path)
    lib = ctypes.CDLL(path)
    dp = ctypes.POINTER(ctypes.c_double)
    i = ctypes.c_int
    lib.kda_oracle_prefill.argtypes = [i, i, i, i, i, dp, dp, dp, dp, dp, dp, dp, dp, i]
    lib.kda_oracle_prefill_snap.argtypes = [i, i, i, i, i] + [dp] * 9 + [i, i]
    lib.kda_oracle_segments.argtypes = [i, i, i, i, i, i, dp, dp, dp, dp, dp, dp, i]
    lib.kda_oracle_merge.argtypes = [i, i, i, i, i, dp, dp, dp, dp, dp]
    lib.kda_oracle_decode_step.argtypes = [i, i, i, i, dp, dp, dp, dp, dp, dp, dp, i]
    lib.kda_oracle_backward.argtypes = [i, i, i, i, i] + [dp] * 14 + [i]
    for f in (lib.kda_oracle_prefill, lib.kda_oracle_prefill_snap, lib.kda_oracle_segments, lib.kda_oracle_merge,
              lib.kda_oracle_decode_step, lib.kda_oracle_backward):
        f.restype = ctypes.c_int
    lib.kda_oracle_max_threads.restype = ctypes.c_int
    _lib_cache[path] = lib
    return lib


def _f64(x) -> Optional[np.ndarray]:
    """Exact upcast to a contiguous fp64 numpy array (bf16/fp32 torch tensors or numpy)."""
    if x is None:
        return None
    try:
        import torch
        if isinstance(x, torch.Tensor):
            x = x.detach().to("cpu", torch.float64).numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _p(a: Optional[np.ndarray]):
    if a is None:
        return ctypes.POINTER(ctypes.c_double)()
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def max_threads(lib=None) -> int:
    return int((lib or load()).kda_oracle_max_threads())


def prefill(q, k, v, log_alpha, beta, S0=None, want_o: bool = True, nthreads: int = 0, lib=None):
    """Token recurrence over [B,H,T,*] inputs.  Returns (o [B,H,T,dv] or None, S_T [B,H,dk,dv])."""
    lib = lib or load()
    q, k, v, la, beta, S0 = map(_f64, (q, k, v, log_alpha, beta, S0))
    B, H, T, dk = k.shape
    dv = v.shape[-1]
    assert q.shape == k.shape == la.shape and v.shape == (B, H, T, dv) and beta.shape == (B, H, T)
    if S0 is not None:
        assert S0.shape == (B, H, dk, dv)
    o = np.empty((B, H, T, dv)) if want_o else None
    ST = np.empty((B, H, dk, dv))
    rc = lib.kda_oracle_prefill(B, H, T, dk, dv, _p(q), _p(k), _p(v), _p(la), _p(beta), _p(S0),
                                _p(o), _p(ST), int(nthreads))
    if rc:
        raise RuntimeError(f"kda_oracle_prefill failed ({rc})")
    return o, ST


def prefill_snap(q, k, v, log_alpha, beta, interval: int, S0=None, want_o: bool = True,
                 nthreads: int = 0, lib=None):
    """Token recurrence with state snapshots every `interval` tokens.  Returns
    (o or None, S_T [B,H,dk,dv], snaps [B, T // interval, H, dk, dv]); snapshot j is
    the state after the first (j + 1) * interval tokens."""
    lib = lib or load()
    q, k, v, la, beta, S0 = map(_f64, (q, k, v, log_alpha, beta, S0))
    B, H, T, dk = k.shape
    dv = v.shape[-1]
    assert q.shape == k.shape == la.shape and v.shape == (B, H, T, dv) and beta.shape == (B, H, T)
    assert interval >= 1
    if S0 is not None:
        assert S0.shape == (B, H, dk, dv)
    o = np.empty((B, H, T, dv)) if want_o else None
    ST = np.empty((B, H, dk, dv))
    snaps = np.empty((B, T // interval, H, dk, dv))
    rc = lib.kda_oracle_prefill_snap(B, H, T, dk, dv, _p(q), _p(k), _p(v), _p(la), _p(beta), _p(S0),
                                     _p(o), _p(ST), _p(snaps), int(interval), int(nthreads))
    if rc:
        raise RuntimeError(f"kda_oracle_prefill_snap failed ({rc})")
    return o, ST, snaps


def segments(k, v, log_alpha, beta, G: int, nthreads: int = 0, lib=None):
    """Per-segment zero-start end states [G,B,H,dk,dv] and transfer maps [G,B,H,dk,dk]."""
    lib = lib or load()
    k, v, la, beta = map(_f64, (k, v, log_alpha, beta))
    B, H, T, dk = k.shape
    dv = v.shape[-1]
    assert T % G == 0
    Z = np.empty((G, B, H, dk, dv))
    M = np.empty((G, B, H, dk, dk))
    rc = lib.kda_oracle_segments(B, H, G, T // G, dk, dv, _p(k), _p(v), _p(la), _p(beta), _p(Z),
                                 _p(M), int(nthreads))
    if rc:
        raise RuntimeError(f"kda_oracle_segments failed ({rc})")
    return Z, M


def merge(S_zero_end, M, S_in=None, lib=None):
    """Sequential merge.  Returns (S_start [G,B,H,dk,dv], S_T [B,H,dk,dv])."""
    lib = lib or load()
    Z, M, S_in = map(_f64, (S_zero_end, M, S_in))
    G, B, H, dk, dv = Z.shape
    S_start = np.empty_like(Z)
    ST = np.empty((B, H, dk, dv))
    rc = lib.kda_oracle_merge(B, H, G, dk, dv, _p(S_in), _p(Z), _p(M), _p(S_start), _p(ST))
    if rc:
        raise RuntimeError(f"kda_oracle_merge failed ({rc})")
    return S_start, ST


def decode_step(q, k, v, log_alpha, beta, S, nthreads: int = 0, lib=None):
    """One decode step on [N,H,*] inputs.  Returns (o [N,H,dv], S_new [N,H,dk,dv]); S is not modified."""
    lib = lib or load()
    q, k, v, la, beta = map(_f64, (q, k, v, log_alpha, beta))
    S = _f64(S).copy()
    N, H, dk = k.shape
    dv = v.shape[-1]
    o = np.empty((N, H, dv))
    rc = lib.kda_oracle_decode_step(N, H, dk, dv, _p(q), _p(k), _p(v), _p(la), _p(beta), _p(S),
                                    _p(o), int(nthreads))
    if rc:
        raise RuntimeError(f"kda_oracle_decode_step failed ({rc})")
    return o, S


def backward(q, k, v, log_alpha, beta, S0=None, dO=None, dS_T=None, nthreads: int = 0, lib=None):
    """Gradients of L = sum(dO * o) + sum(dS_T * S_T) for the prefill on [B,H,T,*]
    inputs (dO [B,H,T,dv] and dS_T [B,H,dk,dv], either may be None for zero).
    Returns a dict with dq, dk, dlog_alpha [B,H,T,dk], dv [B,H,T,dv],
    dbeta [B,H,T] and dS0 [B,H,dk,dv]."""
    lib = lib or load()
    q, k, v, la, beta, S0, dO, dS_T = map(_f64, (q, k, v, log_alpha, beta, S0, dO, dS_T))
    B, H, T, dk = k.shape
    dv = v.shape[-1]
    assert q.shape == k.shape == la.shape and v.shape == (B, H, T, dv) and beta.shape == (B, H, T)
    if S0 is not None:
        assert S0.shape == (B, H, dk, dv)
    if dO is not None:
        assert dO.shape == (B, H, T, dv)
    if dS_T is not None:
        assert dS_T.shape == (B, H, dk, dv)
    out = dict(dq=np.empty((B, H, T, dk)), dk=np.empty((B, H, T, dk)), dv=np.empty((B, H, T, dv)),
               dlog_alpha=np.empty((B, H, T, dk)), dbeta=np.empty((B, H, T)), dS0=np.empty((B, H, dk, dv)))
    rc = lib.kda_oracle_backward(B, H, T, dk, dv, _p(q), _p(k), _p(v), _p(la), _p(beta), _p(S0), _p(dO),
                                 _p(dS_T), _p(out["dq"]), _p(out["dk"]), _p(out["dv"]),
                                 _p(out["dlog_alpha"]), _p(out["dbeta"]), _p(out["dS0"]), int(nthreads))
    if rc:
        raise RuntimeError(f"kda_oracle_backward failed ({rc})")
    return out


def rel_l2(x, ref, floor: float = 0.0) -> float:
    """||x - ref||_2 / max(||ref||_2, floor * sqrt(numel)) over the whole array."""
    x = _f64(x)
    ref = _f64(ref)
    den = max(float(np.linalg.norm(ref)), floor * np.sqrt(ref.size))
    num = float(np.linalg.norm(x - ref))
    if den == 0.0:
        return 0.0 if num == 0.0 else float("inf")
    return num / den


def max_rel_l2(x, ref, lead: int = 2, floor: float = 0.0) -> float:
    """Largest rel-L2 over the slices given by the first ``lead`` axes (e.g. per (b,h))."""
    x = _f64(x)
    ref = _f64(ref)
    assert x.shape == ref.shape, (x.shape, ref.shape)
    n = int(np.prod(x.shape[:lead]))
    xs = x.reshape(n, -1)
    rs = ref.reshape(n, -1)
    return max((rel_l2(xs[i], rs[i], floor) for i in range(n)), default=0.0)
