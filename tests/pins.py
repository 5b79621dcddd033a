"""Independent checks ("pins") of the fp64 oracle.

Each function runs the oracle library given as ``lib`` on small inputs and
returns the largest deviation from a result obtained another way: a dense
product-sum of transition matrices, exact rational arithmetic, the single-chunk
closed form solved by numpy, or closed forms of special cases.  None of them
re-calls the oracle's own loop to produce the expected value.

The update being pinned is the gated delta rule per head
    S_t = (I - b_t k_t k_t^T) Diag(a_t) S_{t-1} + b_t k_t v_t^T,  o_t = S_t^T q_t,
the reading taken for the channel-gated delta-rule attention the pages describe
(blog.csdn.net article on the Kimi K3 report, section 一.1).
"""
from __future__ import annotations

import math
from fractions import Fraction

import numpy as np

import oracle


def _rand_inputs(rng, T, dk, dv, unit_keys=True, s0=True):
    q = rng.standard_normal((T, dk))
    k = rng.standard_normal((T, dk))
    if unit_keys:
        k /= np.linalg.norm(k, axis=1, keepdims=True)
        q /= np.linalg.norm(q, axis=1, keepdims=True)
    v = rng.standard_normal((T, dv))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal(T)))
    la = -1.0 / (1.0 + np.exp(-rng.standard_normal((T, dk))))
    S0 = rng.standard_normal((dk, dv)) * 0.5 if s0 else np.zeros((dk, dv))
    return q, k, v, la, beta, S0


def _run(lib, q, k, v, la, beta, S0):
    o, ST = oracle.prefill(q[None, None], k[None, None], v[None, None], la[None, None],
                           beta[None, None], S0[None, None], lib=lib, nthreads=1)
    return o[0, 0], ST[0, 0]


def pin_product_sum(lib, seed=0) -> float:
    """Dense transition matrices A_t = (I - b k k^T) Diag(a); S_t as the unrolled
    product-sum  A_t..A_1 S0 + sum_s A_t..A_{s+1} b_s k_s v_s^T;  o_t = S_t^T q_t."""
    rng = np.random.default_rng(seed)
    worst = 0.0
    for (T, dk, dv) in [(1, 1, 1), (5, 2, 3), (9, 4, 4), (16, 8, 8), (13, 8, 2), (16, 3, 8)]:
        q, k, v, la, beta, S0 = _rand_inputs(rng, T, dk, dv)
        A = [(np.eye(dk) - beta[t] * np.outer(k[t], k[t])) @ np.diag(np.exp(la[t])) for t in range(T)]
        o_ref = np.zeros((T, dv))
        for t in range(T):
            P = np.eye(dk)
            for j in range(t, -1, -1):
                P = P @ A[j]
            S_t = P @ S0
            for s in range(t + 1):
                Ps = np.eye(dk)
                for j in range(t, s, -1):
                    Ps = Ps @ A[j]
                S_t = S_t + Ps @ (beta[s] * np.outer(k[s], v[s]))
            o_ref[t] = S_t.T @ q[t]
        o, ST = _run(lib, q, k, v, la, beta, S0)
        worst = max(worst, np.abs(o - o_ref).max(), np.abs(ST - S_t).max())
    return float(worst)


def pin_exact_rational(lib, seed=1) -> float:
    """Exact Fraction arithmetic on dyadic inputs; the gate enters as log(a) of a
    rational a, so the oracle sees exp(log a) = a to within one rounding."""
    rng = np.random.default_rng(seed)
    worst = 0.0
    for (T, dk, dv) in [(3, 1, 1), (4, 2, 2), (6, 3, 2), (5, 2, 3)]:
        def dy(n, lo=-8, hi=8, den=8):
            return [Fraction(int(x), den) for x in rng.integers(lo, hi + 1, size=n)]
        q = [dy(dk) for _ in range(T)]
        k = [dy(dk) for _ in range(T)]
        v = [dy(dv) for _ in range(T)]
        beta = [Fraction(int(x), 8) for x in rng.integers(0, 9, size=T)]
        a = [[Fraction(int(x), 16) for x in rng.integers(4, 17, size=dk)] for _ in range(T)]
        S = [[Fraction(int(x), 4) for x in rng.integers(-4, 5, size=dv)] for _ in range(dk)]
        S0 = [row[:] for row in S]
        o_ref = []
        for t in range(T):
            D = [[a[t][i] * S[i][j] for j in range(dv)] for i in range(dk)]
            kD = [sum(k[t][i] * D[i][j] for i in range(dk)) for j in range(dv)]
            # (I - b k k^T) D + b k v^T, entry by entry
            S = [[D[i][j] - beta[t] * k[t][i] * kD[j] + beta[t] * k[t][i] * v[t][j]
                  for j in range(dv)] for i in range(dk)]
            o_ref.append([sum(S[i][j] * q[t][i] for i in range(dk)) for j in range(dv)])
        f = lambda m: np.array([[float(x) for x in r] for r in m])
        la = np.array([[math.log(float(x)) for x in r] for r in a])
        o, ST = _run(lib, f(q), f(k), f(v), la, np.array([float(b) for b in beta]), f(S0))
        worst = max(worst, np.abs(o - f(o_ref)).max(), np.abs(ST - f(S)).max())
    return float(worst)


def pin_chunk_closed_form(lib, seed=2) -> float:
    """One chunk in closed form: with g = cumsum(log a), Qh = q e^g, Kh = k e^g,
    A = strict_lower((k e^g)(k e^-g)^T), P = lower((q e^g)(k e^-g)^T):
        (I + diag(b) A) Delta = diag(b) (V - Kh S0)      (numpy.linalg.solve)
        O = Qh S0 + P Delta,   S_T = Diag(e^{g_T}) S0 + (k e^{g_T - g})^T Delta."""
    rng = np.random.default_rng(seed)
    worst = 0.0
    for (T, dk, dv) in [(1, 4, 4), (7, 8, 8), (16, 8, 4), (16, 16, 16), (11, 5, 7)]:
        q, k, v, la, beta, S0 = _rand_inputs(rng, T, dk, dv)
        g = np.cumsum(la, axis=0)
        Qh, Kh, Kb = q * np.exp(g), k * np.exp(g), k * np.exp(-g)
        A = np.tril(Kh @ Kb.T, -1)
        P = np.tril(Qh @ Kb.T, 0)
        Delta = np.linalg.solve(np.eye(T) + np.diag(beta) @ A, np.diag(beta) @ (v - Kh @ S0))
        O = Qh @ S0 + P @ Delta
        ST = np.diag(np.exp(g[-1])) @ S0 + (k * np.exp(g[-1] - g)).T @ Delta
        o, st = _run(lib, q, k, v, la, beta, S0)
        worst = max(worst, np.abs(o - O).max(), np.abs(st - ST).max())
    return float(worst)


def pin_beta_zero(lib, seed=3) -> float:
    """beta = 0: nothing is written, S_t = Diag(prod_{j<=t} a_j) S0 and o_t = S_t^T q_t."""
    rng = np.random.default_rng(seed)
    T, dk, dv = 40, 8, 6
    q, k, v, la, beta, S0 = _rand_inputs(rng, T, dk, dv)
    beta[:] = 0.0
    o, ST = _run(lib, q, k, v, la, beta, S0)
    g = np.cumsum(la, axis=0)
    o_ref = np.stack([(np.exp(g[t])[:, None] * S0).T @ q[t] for t in range(T)])
    S_ref = np.exp(g[-1])[:, None] * S0
    return float(max(np.abs(o - o_ref).max(), np.abs(ST - S_ref).max()))


def pin_replacement(lib, seed=4) -> float:
    """a = 1, b = 1, orthonormal keys: each write replaces the value stored under its
    key, so k_s^T S_T = v_s^T for every s and S_T = (I - K^T K) S0 + K^T V."""
    rng = np.random.default_rng(seed)
    worst = 0.0
    for (T, dk, dv) in [(1, 4, 3), (5, 8, 8), (8, 8, 5), (12, 16, 16)]:
        Qm, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
        k = Qm[:T].copy()
        q = rng.standard_normal((T, dk))
        v = rng.standard_normal((T, dv))
        la = np.zeros((T, dk))
        beta = np.ones(T)
        S0 = rng.standard_normal((dk, dv))
        _, ST = _run(lib, q, k, v, la, beta, S0)
        worst = max(worst, np.abs(k @ ST - v).max(),
                    np.abs(ST - ((np.eye(dk) - k.T @ k) @ S0 + k.T @ v)).max())
    return float(worst)


def pin_scalar(lib) -> float:
    """dk = dv = 1: s_t = a_t (1 - b_t k_t^2) s_{t-1} + b_t k_t v_t, o_t = q_t s_t,
    evaluated exactly with Fractions."""
    a = [Fraction(1, 2), Fraction(3, 4), Fraction(1, 1), Fraction(7, 8)]
    b = [Fraction(1, 2), Fraction(1, 4), Fraction(1, 1), Fraction(0, 1)]
    k = [Fraction(1), Fraction(-1, 2), Fraction(3, 4), Fraction(2)]
    v = [Fraction(2), Fraction(1), Fraction(-3, 2), Fraction(5)]
    q = [Fraction(1), Fraction(2), Fraction(-1), Fraction(1, 2)]
    s = Fraction(1)
    outs = []
    for t in range(4):
        s = a[t] * (1 - b[t] * k[t] ** 2) * s + b[t] * k[t] * v[t]
        outs.append(q[t] * s)
    c = lambda xs: np.array([[float(x)] for x in xs])
    o, ST = _run(lib, c(q), c(k), c(v), np.array([[math.log(float(x))] for x in a]),
                 np.array([float(x) for x in b]), np.array([[1.0]]))
    return float(max(np.abs(o[:, 0] - c(outs)[:, 0]).max(), abs(ST[0, 0] - float(s))))


def pin_affine(lib, seed=5) -> float:
    """The end state is affine in the start state: S_T(S0) = M S0 + S_T(0), where M is
    the end state of the same tokens run from S0 = I with v = 0."""
    rng = np.random.default_rng(seed)
    T, dk, dv = 37, 8, 5
    q, k, v, la, beta, S0 = _rand_inputs(rng, T, dk, dv)
    la *= 0.05
    _, S_full = _run(lib, q, k, v, la, beta, S0)
    _, S_zero = _run(lib, q, k, v, la, beta, np.zeros((dk, dv)))
    _, M = _run(lib, q, k, np.zeros((T, dk)), la, beta, np.eye(dk))
    return float(np.abs(S_full - (M @ S0 + S_zero)).max())


def pin_snap_decay(lib, seed=6) -> float:
    """Snapshots with b = 0: nothing is written, so the snapshot after the first n
    tokens of head (b, h) is Diag(exp(sum_{t<n} log a_t)) S0[b, h], stored at
    [b, n / interval - 1, h]."""
    rng = np.random.default_rng(seed)
    B, H, T, dk, dv, interval = 2, 3, 37, 4, 3, 5
    la = -rng.random((B, H, T, dk))
    S0 = rng.standard_normal((B, H, dk, dv))
    q, k = rng.standard_normal((B, H, T, dk)), rng.standard_normal((B, H, T, dk))
    v = rng.standard_normal((B, H, T, dv))
    _, ST, snaps = oracle.prefill_snap(q, k, v, la, np.zeros((B, H, T)), interval, S0, lib=lib,
                                       nthreads=1)
    nsnap = T // interval
    if snaps.shape != (B, nsnap, H, dk, dv):
        return float("inf")
    worst = 0.0
    for b in range(B):
        for h in range(H):
            for j in range(nsnap):
                n = (j + 1) * interval
                ref = np.exp(la[b, h, :n].sum(axis=0))[:, None] * S0[b, h]
                worst = max(worst, np.abs(snaps[b, j, h] - ref).max())
            worst = max(worst, np.abs(ST[b, h] - np.exp(la[b, h].sum(axis=0))[:, None] * S0[b, h]).max())
    return float(worst)


def pin_snap_overwrite(lib, seed=7) -> float:
    """Snapshots with a = 1, b = 1 and standard basis keys k_t = e_{i_t}: each token
    replaces row i_t of the state by v_t, so every snapshot is S0 with the rows
    written so far replaced by their latest value (tracked here by plain row
    bookkeeping), and o_t = S_t^T q_t."""
    rng = np.random.default_rng(seed)
    worst = 0.0
    for (T, dk, dv, interval) in [(11, 4, 3, 1), (20, 6, 5, 3), (16, 8, 2, 16)]:
        idx = rng.integers(0, dk, size=T)
        k = np.eye(dk)[idx]
        q, v = rng.standard_normal((T, dk)), rng.standard_normal((T, dv))
        S0 = rng.standard_normal((dk, dv))
        o, _, snaps = oracle.prefill_snap(q[None, None], k[None, None], v[None, None],
                                          np.zeros((1, 1, T, dk)), np.ones((1, 1, T)), interval,
                                          S0[None, None], lib=lib, nthreads=1)
        rows = S0.copy()
        for t in range(T):
            rows[idx[t]] = v[t]
            worst = max(worst, np.abs(o[0, 0, t] - rows.T @ q[t]).max())
            if (t + 1) % interval == 0:
                worst = max(worst, np.abs(snaps[0, (t + 1) // interval - 1, 0] - rows).max())
    return float(worst)


def _grad_loss(lib, q, k, v, la, beta, S0, dO, dST):
    o, ST = _run(lib, q, k, v, la, beta, S0)
    return float((o * dO).sum() + (ST * dST).sum())


def pin_grad_finite_difference(lib, seed=8) -> float:
    """Gradients of L = sum(dO * o) + sum(dS_T * S_T) against central differences
    of the forward recurrence (step 1e-6, fp64), for every element of every input,
    on tiny non-square heads.  Returns the largest error relative to max(|grad|, 1)."""
    rng = np.random.default_rng(seed)
    worst = 0.0
    names = (("q", "dq"), ("k", "dk"), ("v", "dv"), ("la", "dlog_alpha"), ("beta", "dbeta"), ("S0", "dS0"))
    for (T, dk, dv, unit) in [(1, 1, 1, True), (7, 3, 4, True), (5, 4, 2, False), (6, 2, 5, True)]:
        q, k, v, la, beta, S0 = _rand_inputs(rng, T, dk, dv, unit_keys=unit)
        dO = rng.standard_normal((T, dv))
        dST = rng.standard_normal((dk, dv))
        E = lambda x: x[None, None]
        g = oracle.backward(E(q), E(k), E(v), E(la), E(beta), E(S0), E(dO), E(dST), lib=lib, nthreads=1)
        args = dict(q=q, k=k, v=v, la=la, beta=beta, S0=S0)
        h = 1e-6
        for n, gn in names:
            x = args[n]
            an = g[gn][0, 0]
            for idx in np.ndindex(x.shape):
                xp = x.copy()
                xm = x.copy()
                xp[idx] += h
                xm[idx] -= h
                lp = _grad_loss(lib, **{**args, n: xp}, dO=dO, dST=dST)
                lm = _grad_loss(lib, **{**args, n: xm}, dO=dO, dST=dST)
                fd = (lp - lm) / (2 * h)
                worst = max(worst, abs(fd - an[idx]) / max(abs(an[idx]), 1.0))
    return float(worst)


def pin_grad_beta_zero(lib, seed=9) -> float:
    """beta = 0: S_t = Diag(e^{g_t}) S0 with g_t = sum_{s<=t} log a_s, so by hand
        dS_t (total) = sum_{s>=t} Diag(e^{g_s - g_t}) q_s dO_s^T + Diag(e^{g_T - g_t}) dS_T
        dq_t = S_t dO_t,   dbeta_t = (dS_t^T k_t) . (v_t - S'_t^T k_t),  S'_t = Diag(e^{g_t}) S0
        dlog_alpha_s[i] = sum_{t>=s} e^{g_t[i]} q_t[i] (S0 dO_t)[i] + e^{g_T[i]} (S0 * dS_T)[i, :].sum()
        dv = dk = 0,  dS0 = sum_t Diag(e^{g_t}) q_t dO_t^T + Diag(e^{g_T}) dS_T."""
    rng = np.random.default_rng(seed)
    worst = 0.0
    for (T, dk, dv) in [(1, 2, 3), (9, 4, 3), (12, 3, 5)]:
        q, k, v, la, _, S0 = _rand_inputs(rng, T, dk, dv)
        beta = np.zeros(T)
        dO = rng.standard_normal((T, dv))
        dST = rng.standard_normal((dk, dv))
        E = lambda x: x[None, None]
        g = oracle.backward(E(q), E(k), E(v), E(la), E(beta), E(S0), E(dO), E(dST), lib=lib, nthreads=1)
        G = np.cumsum(la, axis=0)  # g_t, t = 0..T-1
        gT = G[-1]
        dq = np.stack([(np.exp(G[t])[:, None] * S0) @ dO[t] for t in range(T)])
        dbeta = np.zeros(T)
        for t in range(T):
            dSt = np.exp(gT - G[t])[:, None] * dST
            for s_ in range(t, T):
                dSt = dSt + np.exp(G[s_] - G[t])[:, None] * np.outer(q[s_], dO[s_])
            Sp = np.exp(G[t])[:, None] * S0
            dbeta[t] = (dSt.T @ k[t]) @ (v[t] - Sp.T @ k[t])
        per_t = np.stack([np.exp(G[t]) * q[t] * (S0 @ dO[t]) for t in range(T)])
        fin = np.exp(gT) * (S0 * dST).sum(axis=1)
        dla = np.cumsum(per_t[::-1], axis=0)[::-1] + fin
        dS0 = sum(np.exp(G[t])[:, None] * np.outer(q[t], dO[t]) for t in range(T)) + np.exp(gT)[:, None] * dST
        for got, ref in ((g["dq"][0, 0], dq), (g["dbeta"][0, 0], dbeta), (g["dlog_alpha"][0, 0], dla),
                         (g["dS0"][0, 0], dS0), (g["dv"][0, 0], 0.0), (g["dk"][0, 0], 0.0)):
            worst = max(worst, float(np.abs(got - ref).max()))
    return worst


def pin_grad_transfer_adjoint(lib, seed=10) -> float:
    """With dO = 0 only S_T = M S0 + Z carries the loss, so dS0 = M^T dS_T, with
    M the segment transfer map (the recurrence run from S0 = I with v = 0)."""
    rng = np.random.default_rng(seed)
    worst = 0.0
    for (T, dk, dv) in [(4, 3, 5), (20, 6, 4)]:
        q, k, v, la, beta, S0 = _rand_inputs(rng, T, dk, dv)
        dST = rng.standard_normal((dk, dv))
        E = lambda x: x[None, None]
        g = oracle.backward(E(q), E(k), E(v), E(la), E(beta), E(S0), None, E(dST), lib=lib, nthreads=1)
        _, M = oracle.segments(E(k), E(v), E(la), E(beta), 1, lib=lib, nthreads=1)
        worst = max(worst, float(np.abs(g["dS0"][0, 0] - M[0, 0, 0].T @ dST).max()))
        worst = max(worst, float(np.abs(g["dq"][0, 0]).max()))  # no output term: dq = 0
    return worst


ALL_PINS = {
    "product_sum": (pin_product_sum, 1e-12),
    "exact_rational": (pin_exact_rational, 1e-12),
    "chunk_closed_form": (pin_chunk_closed_form, 1e-10),
    "beta_zero": (pin_beta_zero, 1e-13),
    "replacement": (pin_replacement, 1e-12),
    "scalar": (pin_scalar, 1e-14),
    "affine": (pin_affine, 1e-12),
    "snap_decay": (pin_snap_decay, 1e-13),
    "snap_overwrite": (pin_snap_overwrite, 1e-13),
    "grad_finite_difference": (pin_grad_finite_difference, 1e-7),
    "grad_beta_zero": (pin_grad_beta_zero, 1e-12),
    "grad_transfer_adjoint": (pin_grad_transfer_adjoint, 1e-12),
}
