"""GPU test of kda_chunk_prefill_noalloc, the prefill entry point that
allocates nothing (its sequence-split path uses the library's scratch array).

Two calls in a row through the C-ABI, the second with a smaller input (and a
different split plan), each checked bit for bit against kda_chunk_prefill with
a caller workspace (the same kernels and plan), and on sampled heads against
the fp64 oracle at the bf16 bar.  A plan larger than the scratch array is
refused with KDA_ERR_WORKSPACE before anything is launched.
"""
import pytest
import torch

import gated_delta_rule_104_amd as kda
import kda_inputs as ki
import oracle

pytestmark = pytest.mark.gpu

TOL = 2e-2


def dev():
    assert torch.cuda.is_available()
    return torch.device("cuda:0")


@pytest.mark.parametrize("B,H,T,variant", [(1, 32, 16384, "slow"), (1, 8, 4096, "none")])
def test_noalloc_matches_prefill(B, H, T, variant):
    D = 128
    T0, G, Tseg = kda.prefill_plan(B, H, T, D, D, torch.bfloat16)
    print(f"[case] noalloc B={B} H={H} T={T} {variant} plan ({T0}, {G}, {Tseg})", flush=True)
    assert G > 1  # both calls take the split path, which uses the scratch array
    g = ki.gen_prefill(B, H, T, D, D, "bf16", seed=70 + H, device=dev(), s0_std=0.1, variant=variant)
    args = (g["q"], g["k"], g["v"], g["log_alpha"], g["beta"], g["S0"])
    o_ref, S_ref = kda.prefill(*args)
    o = torch.full_like(o_ref, 3.0)
    S_T = torch.full_like(S_ref, 3.0)
    kda.prefill_noalloc(*args, o=o, S_T=S_T)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(S_T, S_ref)
    for h in (0, H - 1):
        sl = [g[n][:, h:h + 1].cpu() for n in ("q", "k", "v", "log_alpha", "beta")]
        o_or, S_or = oracle.prefill(*sl, g["S0"][:, h:h + 1].cpu())
        eo = oracle.rel_l2(o[0, h].cpu(), o_or[0, 0])
        es = oracle.rel_l2(S_T[0, h].cpu(), S_or[0, 0])
        print(f"    head {h}: o {eo:.3e}  S_T {es:.3e}", flush=True)
        assert eo <= TOL and es <= TOL


def test_noalloc_single_pass_and_fp32():
    """Shapes that never split (many heads; fp32) use no scratch and match too."""
    for (B, H, T, D, dt) in ((4, 32, 640, 128, "bf16"), (1, 2, 300, 128, "f32")):
        g = ki.gen_prefill(B, H, T, D, D, dt, seed=75, device=dev(), s0_std=0.1)
        args = (g["q"], g["k"], g["v"], g["log_alpha"], g["beta"], g["S0"])
        o_ref, S_ref = kda.prefill(*args)
        o, S_T = kda.prefill_noalloc(*args)
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref) and torch.equal(S_T, S_ref)


def test_noalloc_refuses_plans_beyond_the_scratch(kda_opts):
    """64 segments of 32 heads need (3 * 64 - 1) * 32 fp32 128 x 128 states,
    382 MiB, more than the 64 MiB scratch array: refused, nothing written."""
    B, H, T, D = 1, 32, 8192, 128
    g = ki.gen_prefill(B, H, T, D, D, "bf16", seed=76, device=dev())
    kda_opts("split", 64)
    assert kda.prefill_plan(B, H, T, D, D, torch.bfloat16)[1] == 64
    o = torch.full((B, H, T, D), 5.0, dtype=torch.bfloat16, device=dev())
    with pytest.raises(kda.KdaError) as e:
        kda.prefill_noalloc(g["q"], g["k"], g["v"], g["log_alpha"], g["beta"], None, o=o)
    assert e.value.status == kda.KDA_ERR_WORKSPACE, str(e.value)
    assert "scratch" in str(e.value)
    torch.cuda.synchronize()
    assert bool((o == 5.0).all())
