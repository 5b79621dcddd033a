"""CPU tests of the seeded input generators and the stored oracle fixture."""
import json
import os

import numpy as np
import pytest
import torch

import kda_inputs as ki
import oracle

HERE = os.path.dirname(os.path.abspath(__file__))


def test_deterministic_per_seed():
    a = ki.gen_prefill(1, 3, 40, 16, 8, "bf16", seed=5, s0_std=0.1)
    b = ki.gen_prefill(1, 3, 40, 16, 8, "bf16", seed=5, s0_std=0.1)
    c = ki.gen_prefill(1, 3, 40, 16, 8, "bf16", seed=6, s0_std=0.1)
    for key in ("q", "k", "v", "log_alpha", "beta", "S0"):
        assert torch.equal(a[key], b[key])
        assert not torch.equal(a[key], c[key])


def test_heads_are_independent_streams():
    """Head (b,h) draws only from its own generator: a larger batch contains the
    smaller one's heads unchanged."""
    small = ki.gen_prefill(1, 2, 32, 16, 16, "bf16", seed=3)
    big = ki.gen_prefill(2, 4, 32, 16, 16, "bf16", seed=3)
    for key in ("q", "k", "v", "log_alpha", "beta"):
        assert torch.equal(small[key][0, :2], big[key][0, :2])


def test_distributions():
    d = ki.gen_prefill(1, 2, 4096, 128, 128, "bf16", seed=1, s0_std=0.1)
    # L2-normalised q, k: bf16 rounding keeps the norm within a few 2^-9
    assert ki.l2_stats(d["q"]) < 4e-3 and ki.l2_stats(d["k"]) < 4e-3
    la = d["log_alpha"].float()
    assert float(la.max()) < 0 and float(la.min()) >= -1.0
    assert abs(float(la.mean()) + 0.5) < 0.01
    b = d["beta"].float()
    assert 0 < float(b.min()) and float(b.max()) < 1 and abs(float(b.mean()) - 0.5) < 0.01
    assert abs(ki.sigma_of(d["v"]) - 1.0) < 0.01
    assert abs(ki.sigma_of(d["S0"]) - 0.1) < 0.002


def test_bf16_round_to_nearest_even():
    x = torch.tensor([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -9, -1.0 - 2 ** -8], dtype=torch.float32)
    y = ki.round_to(x, "bf16").float()
    # ties go to the even mantissa; 1 + 2^-9 is below the tie and rounds down
    assert y.tolist() == [1.0, 1.0 + 4 * 2 ** -8, 1.0, -1.0]


@pytest.mark.parametrize("variant", ki.VARIANTS)
def test_variants(variant):
    d = ki.gen_prefill(1, 1, 64, 8, 8, "f32", seed=2, variant=variant)
    la, b = d["log_alpha"], d["beta"]
    if variant == "alpha_one":
        assert float(la.abs().max()) == 0.0
    if variant == "alpha_min":
        assert torch.all(la == -1.0)
    if variant == "beta_zero":
        assert float(b.abs().max()) == 0.0
    if variant == "beta_one":
        assert torch.all(b == 1.0)
    if variant == "slow":
        assert float(la.min()) > -1e-3 and float(b.max()) < 0.05


def test_decode_inputs_shapes():
    s = ki.gen_decode_step(4, 3, 16, 8, "bf16", seed=4, step=0)
    assert s["q"].shape == (4, 3, 16) and s["v"].shape == (4, 3, 8) and s["beta"].shape == (4, 3)
    s2 = ki.gen_decode_step(4, 3, 16, 8, "bf16", seed=4, step=1)
    assert not torch.equal(s["q"], s2["q"])
    S = ki.gen_decode_state(4, 3, 16, 8, seed=4)
    assert S.shape == (4, 3, 16, 8) and S.dtype == torch.float32


def test_golden_fixture_reproduced(oracle_lib):
    """The stored fixture (inputs + oracle outputs) is reproduced: the generator and
    the oracle's arithmetic are unchanged since the fixture was written."""
    with open(os.path.join(HERE, "golden", "oracle_small.json")) as f:
        gold = json.load(f)
    d = ki.gen_prefill(1, 2, 20, 8, 8, "f32", seed=7, s0_std=0.1)
    for key, val in gold["inputs"].items():
        assert np.array_equal(d[key].double().numpy(), np.array(val))
    inp = {k: np.array(v) for k, v in gold["inputs"].items()}
    o, ST = oracle.prefill(inp["q"], inp["k"], inp["v"], inp["log_alpha"], inp["beta"], inp["S0"],
                           lib=oracle_lib)
    assert np.abs(o - np.array(gold["o"])).max() < 1e-14
    assert np.abs(ST - np.array(gold["S_T"])).max() < 1e-14
