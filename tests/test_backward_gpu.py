"""GPU parity of the prefill gradients (kda_prefill_backward, through the
C-ABI) against the fp64 oracle's reverse-mode gradients.

The loss is L = sum(dO * o) + sum(dS_T * S_T) with seeded random dO and dS_T.
Errors are the largest relative L2 error over (b, h) slices, per gradient; the
bars are those of the forward outputs: 1e-4 for fp32 inputs (the token-step
kernel, every step in fp32) and 2e-2 for bf16 inputs (the chunked form on the
matrix cores: bf16 operands, fp32 accumulation, like the forward).
"""
import numpy as np
import pytest
import torch

import gated_delta_rule_104_amd as kda
import kda_inputs as ki
import oracle

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}
NAMES = ("dq", "dk", "dv", "dlog_alpha", "dbeta", "dS0")


def dev():
    assert torch.cuda.is_available()
    return torch.device("cuda:0")


def grads_case(B, H, T, D, dtype, seed, s0_std=0.1, variant="none", with_dO=True, with_dST=True, edit=None):
    print(f"[case] backward B={B} H={H} T={T} D={D} {dtype} {variant} dO={with_dO} dS_T={with_dST}",
          flush=True)
    d = ki.gen_prefill(B, H, T, D, D, dtype, seed=seed, s0_std=s0_std, variant=variant)
    if edit is not None:
        edit(d)
    gen = torch.Generator().manual_seed(1000 + seed)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    dO = torch.randn(B, H, T, D, generator=gen).to(tdt) if with_dO else None
    dST = torch.randn(B, H, D, D, generator=gen) if with_dST else None
    g = {n: (x.to(dev()) if x is not None else None) for n, x in d.items()}
    out = kda.prefill_backward(g["q"], g["k"], g["v"], g["log_alpha"], g["beta"], g["S0"],
                               dO.to(dev()) if dO is not None else None,
                               dST.to(dev()) if dST is not None else None)
    torch.cuda.synchronize()
    ref = oracle.backward(d["q"], d["k"], d["v"], d["log_alpha"], d["beta"], d["S0"], dO, dST)
    err = {}
    for n in NAMES:
        got = out[n].cpu()
        assert torch.isfinite(got).all(), n
        lead = 2 if n != "dbeta" else 1
        err[n] = oracle.max_rel_l2(got, ref[n], lead, floor=1e-6) if got.numel() else 0.0
    print("    " + "  ".join(f"{k} {v:.2e}" for k, v in err.items()), flush=True)
    return err


@pytest.mark.parametrize("T", [1, 63, 64, 65, 130])
def test_backward_f32_d64(T):
    err = grads_case(1, 2, T, 64, "f32", 70 + T)
    assert max(err.values()) <= TOL["f32"], err


@pytest.mark.parametrize("T,variant", [(130, "none"), (200, "slow"), (64, "beta_one")])
def test_backward_bf16_d128(T, variant):
    err = grads_case(2, 2, T, 128, "bf16", 80 + T, variant=variant)
    assert max(err.values()) <= TOL["bf16"], err


def test_backward_bf16_d64_batch():
    err = grads_case(2, 3, 100, 64, "bf16", 91, variant="slow")
    assert max(err.values()) <= TOL["bf16"], err


def test_backward_f32_d128():
    err = grads_case(1, 2, 96, 128, "f32", 92, variant="slow")
    assert max(err.values()) <= TOL["f32"], err


def test_backward_small_f32_workload():
    """The small fp32 workload's shape: B=1, H=2, T=256, d=64."""
    err = grads_case(1, 2, 256, 64, "f32", 0, s0_std=0.0)
    assert max(err.values()) <= TOL["f32"], err


@pytest.mark.parametrize("variant", ["alpha_one", "alpha_min", "beta_zero"])
def test_backward_gate_extremes(variant):
    """No decay (alpha = 1), the lower bound (log alpha = -1), and beta = 0."""
    err = grads_case(1, 2, 100, 64, "f32", 96, variant=variant)
    assert max(err.values()) <= TOL["f32"], err


def test_backward_many_intervals():
    """1000 tokens: 15 full 64-token intervals and a ragged one of 40."""
    err = grads_case(1, 2, 1000, 64, "bf16", 97, variant="slow")
    assert max(err.values()) <= TOL["bf16"], err


@pytest.mark.parametrize("split", ["1", "2"])
@pytest.mark.parametrize("dtype,D,T", [("f32", 128, 130), ("f32", 64, 100)])
def test_backward_split_choice(split, dtype, D, T, kda_opts):
    """fp32 token-step kernel: one workgroup per head, or two each owning half
    of the state's columns (their row sums added by a second kernel): both match
    the oracle."""
    kda_opts("bw_split", int(split))
    err = grads_case(1, 3, T, D, dtype, 98, variant="slow")
    assert max(err.values()) <= TOL[dtype], err


def test_backward_only_end_state_gradient():
    """dO = 0: only S_T carries the loss; dq is zero and dS0 = M^T dS_T."""
    err = grads_case(1, 2, 150, 128, "bf16", 93, variant="slow", with_dO=False)
    assert max(err.values()) <= TOL["bf16"], err


def test_backward_only_output_gradient():
    err = grads_case(1, 2, 90, 64, "f32", 94, with_dST=False)
    assert max(err.values()) <= TOL["f32"], err


def test_backward_zero_tokens():
    """T = 0: the end state is the start state, so dS0 = dS_T exactly."""
    B, H, D = 1, 2, 64
    e = torch.empty(B, H, 0, D, dtype=torch.float32, device=dev())
    beta = torch.empty(B, H, 0, dtype=torch.float32, device=dev())
    S0 = torch.randn(B, H, D, D, device=dev())
    dST = torch.randn(B, H, D, D, device=dev())
    out = kda.prefill_backward(e, e, e, e, beta, S0, None, dST)
    torch.cuda.synchronize()
    assert torch.equal(out["dS0"], dST)


def test_backward_deterministic():
    d = ki.gen_prefill(1, 2, 100, 128, 128, "bf16", seed=95, s0_std=0.1)
    g = {n: (x.to(dev()) if x is not None else None) for n, x in d.items()}
    dO = torch.randn(1, 2, 100, 128, generator=torch.Generator().manual_seed(5)).to(torch.bfloat16).to(dev())
    a = kda.prefill_backward(g["q"], g["k"], g["v"], g["log_alpha"], g["beta"], g["S0"], dO, None)
    b = kda.prefill_backward(g["q"], g["k"], g["v"], g["log_alpha"], g["beta"], g["S0"], dO, None)
    torch.cuda.synchronize()
    for n in NAMES:
        assert torch.equal(a[n], b[n]), n


def test_backward_full_b4_h32_t8k():
    """The bench's launch (B=4, H=32, T=8192, d=128, bf16, with S0, dO and dS_T,
    drawn on the device as the bench draws them) on every head; the oracle
    checks two sampled heads, read back from the device (heads are independent)."""
    B, H, T, D = 4, 32, 8192, 128
    print(f"[case] backward full B={B} H={H} T={T} D={D} bf16", flush=True)
    g = ki.gen_prefill(B, H, T, D, D, "bf16", seed=1, s0_std=0.1, device=dev())
    gen = torch.Generator(device=dev()).manual_seed(6)
    dO = torch.randn(B, H, T, D, generator=gen, device=dev()).to(torch.bfloat16)
    dST = torch.randn(B, H, D, D, generator=gen, device=dev())
    out = kda.prefill_backward(g["q"], g["k"], g["v"], g["log_alpha"], g["beta"], g["S0"], dO, dST)
    torch.cuda.synchronize()
    for (b, h) in ((0, 0), (3, 31)):
        sl = lambda x: x[b:b + 1, h:h + 1].cpu()
        ref = oracle.backward(sl(g["q"]), sl(g["k"]), sl(g["v"]), sl(g["log_alpha"]), sl(g["beta"]),
                              sl(g["S0"]), sl(dO), sl(dST))
        err = {}
        for n in NAMES:
            got = sl(out[n])
            assert torch.isfinite(got).all(), n
            err[n] = oracle.max_rel_l2(got, ref[n], 2 if n != "dbeta" else 1, floor=1e-6)
        print(f"    head ({b},{h}) " + "  ".join(f"{k} {v:.2e}" for k, v in err.items()), flush=True)
        assert max(err.values()) <= TOL["bf16"], err


# ----------------------------------------------------------------- chunked form (bf16)

@pytest.mark.parametrize("T", [1, 63, 64, 65, 127, 128, 200, 1000])
@pytest.mark.parametrize("D", [64, 128])
def test_backward_chunked_tails(T, D):
    """Ragged last chunks, one to sixteen chunks, both head sizes."""
    err = grads_case(1, 2, T, D, "bf16", 300 + T, variant="slow")
    assert max(err.values()) <= TOL["bf16"], err


@pytest.mark.parametrize("variant", ["none", "alpha_one", "alpha_min", "beta_zero", "beta_one"])
def test_backward_chunked_gates(variant):
    """The workloads' gates, no decay, the lower bound log alpha = -1, beta = 0
    (dk and dv are then exactly zero) and beta = 1."""
    err = grads_case(2, 2, 300, 128, "bf16", 310, variant=variant)
    assert max(err.values()) <= TOL["bf16"], err


def test_backward_chunked_tiny_beta_rows():
    """Tokens with beta = 0 or beta = 1e-12 (below 2^-30) among ordinary ones:
    their dbeta comes from the rows of Xbar, W and Kh Kb^T the chain kernels
    keep for them; every other token's from dv and Delta."""
    def edit(d):
        beta = d["beta"]
        t = torch.arange(beta.shape[-1])
        beta[..., t % 7 == 3] = 0.0
        beta[..., t % 11 == 5] = 1e-12
        beta[..., t % 13 == 1] = 1e-6
    err = grads_case(1, 2, 200, 128, "bf16", 340, variant="slow", edit=edit)
    assert max(err.values()) <= TOL["bf16"], err


@pytest.mark.parametrize("with_dO,with_dST", [(True, False), (False, True)])
def test_backward_chunked_one_loss_term(with_dO, with_dST):
    """Only the outputs, or only the end state, carry the loss (dO or dS_T NULL)."""
    err = grads_case(1, 3, 260, 128, "bf16", 320, variant="slow", with_dO=with_dO, with_dST=with_dST)
    assert max(err.values()) <= TOL["bf16"], err


@pytest.mark.parametrize("T,D,tiny", [(1024, 128, False), (4100, 128, True), (2000, 64, False)])
def test_backward_chunked_overlap_bitwise(T, D, tiny, kda_opts):
    """From 16 chunks per head the reverse chain runs as two launches (the
    later half of the chunks, then the earlier half, dS carried in fp32) and
    the later half's per-chunk gradients beside the earlier half's chain:
    every output equals, bit for bit, the one of the chain run whole followed
    by every chunk's gradients (option bw_overlap 0).  Ragged last chunk, both
    head sizes, and tokens with tiny beta (their rows of W, Xbar and Kh Kb^T
    are indexed by the chunk of the whole sequence)."""
    B, H = 1, 3
    print(f"[case] backward overlap B={B} H={H} T={T} D={D} tiny={tiny}", flush=True)
    g = ki.gen_prefill(B, H, T, D, D, "bf16", seed=360 + T, s0_std=0.1, variant="slow", device=dev())
    if tiny:
        t = torch.arange(T, device=dev())
        g["beta"][..., t % 7 == 3] = 0.0
        g["beta"][..., t % 11 == 5] = 1e-12
    gen = torch.Generator(device=dev()).manual_seed(361 + T)
    dO = torch.randn(B, H, T, D, generator=gen, device=dev()).to(torch.bfloat16)
    dST = torch.randn(B, H, D, D, generator=gen, device=dev())
    out = {}
    for ov in (0, 1):
        kda_opts("bw_overlap", ov)
        out[ov] = kda.prefill_backward(g["q"], g["k"], g["v"], g["log_alpha"], g["beta"], g["S0"], dO, dST)
        torch.cuda.synchronize()
    for n in NAMES:
        assert torch.isfinite(out[1][n]).all(), n
        assert torch.equal(out[0][n], out[1][n]), n


def test_backward_chunked_single_long_head():
    """One head over 4100 tokens (65 chunks, the last one ragged): one
    workgroup per chain beside 130 gradient workgroups."""
    err = grads_case(1, 1, 4100, 128, "bf16", 350, variant="slow")
    assert max(err.values()) <= TOL["bf16"], err


def test_backward_chunked_d64_many_heads():
    """d = 64 with 64 heads over 2048 tokens: the chains' d = 64 variants and
    2048 gradient workgroups; sampled heads against the oracle."""
    B, H, T, D = 2, 32, 2048, 64
    print(f"[case] backward d64 B={B} H={H} T={T}", flush=True)
    d = ki.gen_prefill(B, H, T, D, D, "bf16", seed=352, s0_std=0.1, variant="slow")
    gen = torch.Generator().manual_seed(353)
    dO = torch.randn(B, H, T, D, generator=gen).to(torch.bfloat16)
    dST = torch.randn(B, H, D, D, generator=gen)
    g = {n: (x.to(dev()) if x is not None else None) for n, x in d.items()}
    out = kda.prefill_backward(g["q"], g["k"], g["v"], g["log_alpha"], g["beta"], g["S0"], dO.to(dev()),
                               dST.to(dev()))
    torch.cuda.synchronize()
    for (b, h) in ((0, 0), (1, 31), (0, 17)):
        sl = lambda x: x[b:b + 1, h:h + 1]
        ref = oracle.backward(sl(d["q"]), sl(d["k"]), sl(d["v"]), sl(d["log_alpha"]), sl(d["beta"]),
                              sl(d["S0"]), sl(dO), sl(dST))
        err = {n: oracle.max_rel_l2(sl(out[n]).cpu(), ref[n], 2 if n != "dbeta" else 1, floor=1e-6)
               for n in NAMES}
        print(f"    head ({b},{h}) " + "  ".join(f"{k} {v:.2e}" for k, v in err.items()), flush=True)
        assert max(err.values()) <= TOL["bf16"], err


def test_backward_chunked_no_loss():
    """dO and dS_T both NULL: the loss is zero and so is every gradient."""
    d = ki.gen_prefill(2, 2, 150, 128, 128, "bf16", seed=351, s0_std=0.1, variant="slow")
    g = {n: (x.to(dev()) if x is not None else None) for n, x in d.items()}
    out = kda.prefill_backward(g["q"], g["k"], g["v"], g["log_alpha"], g["beta"], g["S0"], None, None)
    torch.cuda.synchronize()
    for n in NAMES:
        assert torch.count_nonzero(out[n]).item() == 0, n


def test_backward_chunked_zero_tokens():
    """T = 0 on the chunked path: dS0 = dS_T exactly."""
    B, H, D = 2, 2, 128
    e = torch.empty(B, H, 0, D, dtype=torch.bfloat16, device=dev())
    beta = torch.empty(B, H, 0, dtype=torch.bfloat16, device=dev())
    dST = torch.randn(B, H, D, D, device=dev())
    out = kda.prefill_backward(e, e, e, e, beta, None, None, dST)
    torch.cuda.synchronize()
    assert torch.equal(out["dS0"], dST)


@pytest.mark.parametrize("nc", [1, 2, 4])
def test_backward_chunked_column_split_invariant(nc, kda_opts):
    """The reverse chain's consumer-wave count (state columns per workgroup)
    changes the launch, not the result."""
    d = ki.gen_prefill(1, 2, 200, 128, 128, "bf16", seed=330, s0_std=0.1, variant="slow")
    g = {n: (x.to(dev()) if x is not None else None) for n, x in d.items()}
    dO = torch.randn(1, 2, 200, 128, generator=torch.Generator().manual_seed(3)).to(torch.bfloat16).to(dev())
    dST = torch.randn(1, 2, 128, 128, generator=torch.Generator().manual_seed(4)).to(dev())
    args = (g["q"], g["k"], g["v"], g["log_alpha"], g["beta"], g["S0"], dO, dST)
    kda_opts("nc", nc)
    a = kda.prefill_backward(*args)
    kda_opts("nc", None)
    b = kda.prefill_backward(*args)
    torch.cuda.synchronize()
    for n in NAMES:
        assert torch.equal(a[n], b[n]), n
