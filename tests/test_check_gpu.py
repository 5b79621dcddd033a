"""GPU tests of the precondition check mode (option "check").

The kernels rely on log alpha in [-1, 0], the pages' lower-bounded decay
(blog.csdn.net article on the Kimi K3 report, section 一.1), and on beta in
[0, 1].  With the option set, every call that reads log_alpha and beta reduces
them on the device first and returns KDA_ERR_PRECONDITION, writing nothing,
when a value is out of range or not finite.  In-range inputs give the same
results bit for bit as without the check.
"""
import pytest
import torch

import gated_delta_rule_104_amd as kda
import kda_inputs as ki

pytestmark = pytest.mark.gpu


def dev():
    assert torch.cuda.is_available()
    return torch.device("cuda:0")


def inputs(T=200, D=128, dtype="bf16", seed=60):
    d = ki.gen_prefill(1, 2, T, D, D, dtype, seed=seed, s0_std=0.1)
    return {n: (x.to(dev()) if x is not None else None) for n, x in d.items()}


def prefill_call(g, la=None, beta=None, o=None):
    return kda.prefill(g["q"], g["k"], g["v"], g["log_alpha"] if la is None else la,
                       g["beta"] if beta is None else beta, g["S0"], o=o)


def expect_precondition(fn, what):
    with pytest.raises(kda.KdaError) as e:
        fn()
    assert e.value.status == kda.KDA_ERR_PRECONDITION, str(e.value)
    assert what in str(e.value), str(e.value)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_check_passes_valid_inputs_unchanged(dtype, kda_opts):
    g = inputs(dtype=dtype)
    o0, S0 = prefill_call(g)
    kda_opts("check", 1)
    o1, S1 = prefill_call(g)
    torch.cuda.synchronize()
    assert torch.equal(o0, o1) and torch.equal(S0, S1)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("bad", [-2.0, 0.5, float("nan"), float("-inf")])
def test_check_rejects_gate_out_of_range(dtype, bad, kda_opts):
    """One channel of one token with log alpha = bad: KDA_ERR_PRECONDITION, and
    the output buffer is left as it was."""
    print(f"[case] check log_alpha={bad} {dtype}", flush=True)
    g = inputs(dtype=dtype)
    la = g["log_alpha"].clone()
    la[0, 1, 77, 5] = bad
    kda_opts("check", 1)
    o = torch.full_like(g["v"], 7.0)
    expect_precondition(lambda: prefill_call(g, la=la, o=o), "log_alpha")
    torch.cuda.synchronize()
    assert bool((o == 7.0).all())


@pytest.mark.parametrize("bad", [1.5, -0.25, float("nan")])
def test_check_rejects_beta_out_of_range(bad, kda_opts):
    g = inputs()
    beta = g["beta"].clone()
    beta[0, 0, 199] = bad
    kda_opts("check", 1)
    expect_precondition(lambda: prefill_call(g, beta=beta), "beta")


def test_check_covers_every_call(kda_opts):
    """Segment transfer, segmented prefill, decode (one and several tokens) and
    the gradients check their gates too; the sequence-split prefill checks
    before its first launch."""
    g = inputs(T=256)
    la = g["log_alpha"].clone()
    la[0, 0, 3, 100] = -2.0
    kda_opts("check", 1)
    expect_precondition(lambda: kda.segment_transfer(g["k"], g["v"], la, g["beta"], 2), "log_alpha")
    expect_precondition(lambda: kda.prefill_segments(g["q"], g["k"], g["v"], la, g["beta"], None, 64), "log_alpha")
    step = {n: g[n][:, :, 3].contiguous() for n in ("q", "k", "v", "beta")}
    S = torch.zeros(1, 2, 128, 128, device=dev())
    expect_precondition(lambda: kda.decode_step(step["q"], step["k"], step["v"], la[:, :, 3].contiguous(),
                                                step["beta"], S), "log_alpha")
    expect_precondition(lambda: kda.decode_tokens(g["q"][:, :, :5].contiguous(), g["k"][:, :, :5].contiguous(),
                                                  g["v"][:, :, :5].contiguous(), la[:, :, :5].contiguous(),
                                                  g["beta"][:, :, :5].contiguous(), S), "log_alpha")
    expect_precondition(lambda: kda.prefill_backward(g["q"], g["k"], g["v"], la, g["beta"], g["S0"],
                                                     torch.ones_like(g["v"]), None), "log_alpha")
    # the sequence-split path
    kda_opts("split", 3)
    big = inputs(T=4096)
    la2 = big["log_alpha"].clone()
    la2[0, 1, 4000, 0] = -1.5
    expect_precondition(lambda: prefill_call(big, la=la2), "log_alpha")
    assert torch.equal(S, torch.zeros_like(S))
