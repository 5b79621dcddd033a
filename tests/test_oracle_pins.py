"""CPU tests: pin the fp64 oracle to results it does not compute itself."""
import os

import numpy as np
import pytest

import oracle
from oracle import build_oracle

from pins import ALL_PINS, _rand_inputs, _run


@pytest.mark.parametrize("name", sorted(ALL_PINS))
def test_pin(oracle_lib, name):
    fn, tol = ALL_PINS[name]
    err = fn(oracle_lib)
    assert err <= tol, f"{name}: {err:.3e} > {tol:.1e}"


def test_resume_bitwise(oracle_lib):
    """Running T1 tokens, then T2 tokens from the resulting state, gives exactly the
    state and outputs of running T1 + T2 tokens (the state is the checkpoint)."""
    rng = np.random.default_rng(10)
    q, k, v, la, beta, S0 = _rand_inputs(rng, 50, 8, 8)
    o_all, S_all = _run(oracle_lib, q, k, v, la, beta, S0)
    o1, S1 = _run(oracle_lib, q[:23], k[:23], v[:23], la[:23], beta[:23], S0)
    o2, S2 = _run(oracle_lib, q[23:], k[23:], v[23:], la[23:], beta[23:], S1)
    assert np.array_equal(S2, S_all)
    assert np.array_equal(np.concatenate([o1, o2]), o_all)


def test_contraction(oracle_lib):
    """With b in [0,1], ||k|| = 1 and a <= 1 every A_t has spectral norm <= 1, so the
    transfer map M of any segment does too."""
    rng = np.random.default_rng(11)
    for T in (1, 10, 200):
        q, k, v, la, beta, _ = _rand_inputs(rng, T, 16, 16)
        la *= 0.01
        _, M = _run(oracle_lib, q, k, np.zeros((T, 16)), la, beta, np.eye(16))
        assert np.linalg.norm(M, 2) <= 1.0 + 1e-12


def test_decode_step_matches_prefill(oracle_lib):
    rng = np.random.default_rng(12)
    N, H, dk, dv = 3, 2, 8, 4
    S = rng.standard_normal((N, H, dk, dv))
    q, k = rng.standard_normal((N, H, dk)), rng.standard_normal((N, H, dk))
    v, la = rng.standard_normal((N, H, dv)), -rng.random((N, H, dk))
    beta = rng.random((N, H))
    o, S1 = oracle.decode_step(q, k, v, la, beta, S, lib=oracle_lib)
    o2, S2 = oracle.prefill(q[:, :, None], k[:, :, None], v[:, :, None], la[:, :, None],
                            beta[:, :, None], S, lib=oracle_lib)
    assert np.array_equal(o, o2[:, :, 0]) and np.array_equal(S1, S2)


@pytest.mark.parametrize("G", [1, 3, 4])
def test_segments_merge_match_prefill(oracle_lib, G):
    """Segment decomposition: per-segment zero-start states and transfer maps, merged
    in order, reproduce the start state of every segment and the final state."""
    rng = np.random.default_rng(13 + G)
    B, H, Tseg, dk, dv = 1, 2, 12, 6, 5
    T = G * Tseg
    q = rng.standard_normal((B, H, T, dk))
    k = rng.standard_normal((B, H, T, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, H, T, dv))
    la = -0.05 * rng.random((B, H, T, dk))
    beta = rng.random((B, H, T))
    S0 = rng.standard_normal((B, H, dk, dv))
    Z, M = oracle.segments(k, v, la, beta, G, lib=oracle_lib)
    S_start, ST = oracle.merge(Z, M, S0, lib=oracle_lib)
    _, ST_ref = oracle.prefill(q, k, v, la, beta, S0, lib=oracle_lib)
    assert np.abs(ST - ST_ref).max() < 1e-12
    for gi in range(G):
        _, Sg = oracle.prefill(q[:, :, :gi * Tseg], k[:, :, :gi * Tseg], v[:, :, :gi * Tseg],
                               la[:, :, :gi * Tseg], beta[:, :, :gi * Tseg], S0, lib=oracle_lib)
        assert np.abs(S_start[gi] - Sg).max() < 1e-12


def test_empty_sequence(oracle_lib):
    """T = 0 leaves the state untouched."""
    rng = np.random.default_rng(14)
    S0 = rng.standard_normal((1, 1, 4, 3))
    z = np.zeros((1, 1, 0, 4))
    o, ST = oracle.prefill(z, z, np.zeros((1, 1, 0, 3)), z, np.zeros((1, 1, 0)), S0, lib=oracle_lib)
    assert o.shape == (1, 1, 0, 3) and np.array_equal(ST, S0)


def test_snapshots_match_prefix_runs(oracle_lib):
    """Snapshot j equals the end state of the same recurrence run on the first
    (j + 1) * interval tokens alone; with T a multiple of the interval the last
    snapshot is S_T."""
    rng = np.random.default_rng(15)
    B, H, T, dk, dv, interval = 2, 2, 24, 5, 4, 6
    q, k = rng.standard_normal((B, H, T, dk)), rng.standard_normal((B, H, T, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, H, T, dv))
    la = -0.2 * rng.random((B, H, T, dk))
    beta = rng.random((B, H, T))
    S0 = rng.standard_normal((B, H, dk, dv))
    o, ST, snaps = oracle.prefill_snap(q, k, v, la, beta, interval, S0, lib=oracle_lib)
    o_ref, ST_ref = oracle.prefill(q, k, v, la, beta, S0, lib=oracle_lib)
    assert np.array_equal(o, o_ref) and np.array_equal(ST, ST_ref)
    assert np.array_equal(snaps[:, -1], ST)
    for j in range(T // interval):
        n = (j + 1) * interval
        _, Sj = oracle.prefill(q[:, :, :n], k[:, :, :n], v[:, :, :n], la[:, :, :n], beta[:, :, :n],
                               S0, lib=oracle_lib)
        assert np.array_equal(snaps[:, j], Sj)
    _, _, none = oracle.prefill_snap(q[:, :, :5], k[:, :, :5], v[:, :, :5], la[:, :, :5],
                                     beta[:, :, :5], interval, S0, lib=oracle_lib)
    assert none.shape == (B, 0, H, dk, dv)


@pytest.mark.parametrize("mutant", [1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11])
def test_planted_mistakes_are_caught(tmp_path, mutant):
    """Each planted mistake (dropped decay, flipped delta sign, pre-update output,
    k in place of q, decay after the write, transposed state read, snapshot one
    token late; in the gradients: the output's term dropped, du's sign flipped,
    dlog_alpha from the undecayed state, dD passed back without the decay)
    makes at least one pin fail."""
    path = build_oracle.build(str(tmp_path / f"mut{mutant}.so"), mutant=mutant)
    lib = oracle.load(path)
    failed = []
    for name, (fn, tol) in ALL_PINS.items():
        try:
            err = fn(lib)
        except Exception:  # a crash also counts as caught
            err = float("inf")
        if not err <= tol:
            failed.append(name)
    assert failed, f"mutant {mutant} passed every pin"
