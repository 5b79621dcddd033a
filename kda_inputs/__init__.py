"""Seeded synthetic inputs for Kimi Delta Attention (KDA) workloads.

This module is shared by the fp64 oracle (``oracle/``), the tests, ``bench.py``
and ``__graft_entry__.smoke()``.  It holds only input generation: random draws,
the per-token L2 normalisation of q and k that the workloads prescribe, the
sigmoid maps that produce beta and log-alpha, and rounding to the storage dtype.
None of the method's arithmetic (decay, delta update, outputs) lives here.

Distributions (the same for every workload):
  q, k      ~ N(0, 1), then L2-normalised over the key dimension per (b, h, t)
              in fp32, then rounded (round-to-nearest-even) to the storage dtype
  v         ~ N(0, 1)
  beta      = sigmoid(N(0, 1)), one scalar per (b, h, t)
  log_alpha = -sigmoid(N(0, 1)), one value per key channel per (b, h, t)
  S0        ~ N(0, 0.1^2) in fp32 when requested (variance 0.01), else zero

The gate is passed in log space.  The pages describe the forget gate as
channel-wise and its parameterisation as lower-bounded so that long sequences do
not overflow (blog.csdn.net article on the Kimi K3 report, section 一.1 "KimiDelta
Attention"); -sigmoid(.) lies in (-1, 0), so every drawn log-alpha already meets
the bound log_alpha >= -1 that the GPU kernels take as a precondition.

Every (b, h) slice has its own generator seeded from (seed, b, h), drawn in the
order q, k, v, beta, log_alpha; S0 uses a separate generator per (seed, b, h).
torch's CPU and GPU generators give different streams for one seed, so a test
that compares devices generates once and copies.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Dict, Optional

import torch

__all__ = [
    "PREFILL_CONFIGS",
    "head_seed",
    "gen_prefill",
    "gen_decode_step",
    "gen_decode_state",
    "round_to",
    "VARIANTS",
]

_DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16}

# Stress variants used by parity tests.  Each maps fp32 (beta, log_alpha) draws
# to new values before rounding.  "slow" keeps the start state and the transfer
# maps alive over thousands of tokens, which the plain draws wipe out within a
# few chunks (mean log-alpha is -0.5 per step and channel).
VARIANTS = ("none", "slow", "alpha_one", "alpha_min", "beta_zero", "beta_one")


@dataclass(frozen=True)
class PrefillConfig:
    name: str
    B: int
    H: int
    T: int
    dk: int
    dv: int
    dtype: str
    s0_std: float
    seed: int


# The five workloads, by what they are.  T of 8K / 64K / 1M follows the
# context-extension stages the pages list (blog.csdn.net article, section 二.1).
PREFILL_CONFIGS = {
    "small_f32": PrefillConfig("small_f32", 1, 2, 256, 64, 64, "f32", 0.0, 0),
    "b4_h32_t8k": PrefillConfig("b4_h32_t8k", 4, 32, 8192, 128, 128, "bf16", 0.1, 1),
    "h32_t64k": PrefillConfig("h32_t64k", 1, 32, 65536, 128, 128, "bf16", 0.0, 2),
    "kcp_h32_t1m": PrefillConfig("kcp_h32_t1m", 1, 32, 1048576, 128, 128, "bf16", 0.0, 3),
}
DECODE_CONFIG = dict(name="decode_n256_h32", N=256, H=32, dk=128, dv=128, steps=1024,
                     dtype="bf16", s0_std=0.1, seed=4)


def head_seed(seed: int, *idx: int) -> int:
    """Deterministic 63-bit seed for a slice, from (seed, idx...) by splitmix64."""
    x = (seed * 0x9E3779B97F4A7C15) & 0xFFFFFFFFFFFFFFFF
    for i in idx:
        x = (x + 0x9E3779B97F4A7C15 + (i & 0xFFFFFFFF)) & 0xFFFFFFFFFFFFFFFF
        z = x
        z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & 0xFFFFFFFFFFFFFFFF
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & 0xFFFFFFFFFFFFFFFF
        x = z ^ (z >> 31)
    return x & 0x7FFFFFFFFFFFFFFF


def round_to(x: torch.Tensor, dtype: str) -> torch.Tensor:
    """Round an fp32 tensor to the storage dtype (round-to-nearest-even)."""
    return x.to(_DTYPES[dtype])


def _l2n(x: torch.Tensor) -> torch.Tensor:
    return x / x.norm(dim=-1, keepdim=True).clamp_min(1e-30)


def _apply_variant(beta: torch.Tensor, la: torch.Tensor, variant: str):
    if variant == "none":
        return beta, la
    if variant == "slow":
        return beta * 0.05, la * 1e-3
    if variant == "alpha_one":
        return beta, torch.zeros_like(la)
    if variant == "alpha_min":
        return beta, torch.full_like(la, -1.0)
    if variant == "beta_zero":
        return torch.zeros_like(beta), la
    if variant == "beta_one":
        return torch.ones_like(beta), la
    raise ValueError(f"unknown variant {variant!r}")


def gen_prefill(B: int, H: int, T: int, dk: int, dv: int, dtype: str = "bf16", seed: int = 0,
                device: str | torch.device = "cpu", s0_std: float = 0.0,
                variant: str = "none") -> Dict[str, Optional[torch.Tensor]]:
    """Inputs of one prefill call, contiguous, in layout [B, H, T, D].

    Returns q, k, log_alpha [B,H,T,dk]; v [B,H,T,dv]; beta [B,H,T] in ``dtype``;
    S0 [B,H,dk,dv] fp32 (None when s0_std == 0).
    """
    dt = _DTYPES[dtype]
    dev = torch.device(device)
    q = torch.empty(B, H, T, dk, dtype=dt, device=dev)
    k = torch.empty(B, H, T, dk, dtype=dt, device=dev)
    v = torch.empty(B, H, T, dv, dtype=dt, device=dev)
    la = torch.empty(B, H, T, dk, dtype=dt, device=dev)
    beta = torch.empty(B, H, T, dtype=dt, device=dev)
    S0 = torch.empty(B, H, dk, dv, dtype=torch.float32, device=dev) if s0_std > 0 else None
    for b in range(B):
        for h in range(H):
            g = torch.Generator(device=dev)
            g.manual_seed(head_seed(seed, b, h))
            f32 = dict(dtype=torch.float32, device=dev, generator=g)
            qh = _l2n(torch.randn(T, dk, **f32))
            kh = _l2n(torch.randn(T, dk, **f32))
            vh = torch.randn(T, dv, **f32)
            bh = torch.sigmoid(torch.randn(T, **f32))
            lah = -torch.sigmoid(torch.randn(T, dk, **f32))
            bh, lah = _apply_variant(bh, lah, variant)
            q[b, h] = qh.to(dt)
            k[b, h] = kh.to(dt)
            v[b, h] = vh.to(dt)
            beta[b, h] = bh.to(dt)
            la[b, h] = lah.to(dt)
            if S0 is not None:
                g2 = torch.Generator(device=dev)
                g2.manual_seed(head_seed(seed, b, h, 0x5E))
                S0[b, h] = torch.randn(dk, dv, dtype=torch.float32, device=dev, generator=g2) * s0_std
    return dict(q=q, k=k, v=v, log_alpha=la, beta=beta, S0=S0)


def gen_decode_state(N: int, H: int, dk: int, dv: int, seed: int, s0_std: float = 0.1,
                     device: str | torch.device = "cpu") -> torch.Tensor:
    """Initial fp32 decode states [N, H, dk, dv] ~ N(0, s0_std^2)."""
    dev = torch.device(device)
    g = torch.Generator(device=dev)
    g.manual_seed(head_seed(seed, 0x5E, 0x5E))
    return torch.randn(N, H, dk, dv, dtype=torch.float32, device=dev, generator=g) * s0_std


def gen_decode_step(N: int, H: int, dk: int, dv: int, dtype: str, seed: int, step: int,
                    device: str | torch.device = "cpu",
                    variant: str = "none") -> Dict[str, torch.Tensor]:
    """Per-token inputs of one decode step: q, k, log_alpha [N,H,dk]; v [N,H,dv]; beta [N,H]."""
    dt = _DTYPES[dtype]
    dev = torch.device(device)
    g = torch.Generator(device=dev)
    g.manual_seed(head_seed(seed, 0xDEC, step))
    f32 = dict(dtype=torch.float32, device=dev, generator=g)
    q = _l2n(torch.randn(N, H, dk, **f32))
    k = _l2n(torch.randn(N, H, dk, **f32))
    v = torch.randn(N, H, dv, **f32)
    beta = torch.sigmoid(torch.randn(N, H, **f32))
    la = -torch.sigmoid(torch.randn(N, H, dk, **f32))
    beta, la = _apply_variant(beta, la, variant)
    return dict(q=q.to(dt), k=k.to(dt), v=v.to(dt), log_alpha=la.to(dt), beta=beta.to(dt))


def l2_stats(x: torch.Tensor) -> float:
    """Largest deviation of per-row L2 norms from 1 (used by generator tests)."""
    n = x.float().norm(dim=-1)
    return float((n - 1).abs().max())


def sigma_of(x: torch.Tensor) -> float:
    return float(x.float().std())

