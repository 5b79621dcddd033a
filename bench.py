"""Benchmark of the libkda hot path on one MI355X.

One step = one kda_chunk_prefill call over B=1, H=32, T=65536, dk=dv=128, bf16
inputs (seeded synthetic data already resident in HBM, S0 = 0).  `value` is
sequence tokens per second of that step.  The same run also measures, outside
the timed steps:
  * the per-kernel durations of the sequence-split path, through the public
    calls it is made of (the roofline line is the slowest of them);
  * the same prefill with a state snapshot every 512 tokens;
  * the same prefill shape with slowly decaying gates, where no transfer-map
    column of the segment pass reaches zero;
  * the batched prefill B=4, H=32, T=8192 with an fp32 start state;
  * the gradients of that batched prefill (kda_prefill_backward);
  * decode: 1024 consecutive kda_decode_step calls on 256 sequences x 32 heads
    (fp32 state 512 MiB in place), reported as % of HBM bandwidth;
  * decode_tokens: 4 draft tokens per sequence in one call, with and without
    the per-token states;
  * kcp: kda_segment_transfer + kda_segment_merge on T = 1,048,576 in 8
    segments of 131,072 (H = 32), reported as time and effective bandwidth,
    then kda_chunk_prefill_segments from the merged start states (outputs);
  * calibration: a large bf16 torch matmul and a device copy, the rates this
    box reaches beside the spec peaks;
  * cpu_baseline: the fp64 oracle on a bounded sample of the prefill workload.
Kernel durations come from HIP events recorded on the stream the kernels are
launched on.  Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import statistics
import sys
import time

import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import gated_delta_rule_104_amd as kda  # noqa: E402
import kda_inputs as ki  # noqa: E402

METRIC = "KDA chunked-prefill tokens/sec (H=32,d=128,T=64K) + % MFMA peak; decode % HBM BW"
PEAK_HBM_GBS = 8000.0
PEAK_BF16_TFLOPS = 2500.0
CH = 64


# HBM bytes per launch measured with rocprofv3 FETCH_SIZE / WRITE_SIZE on this
# workload, each scaled by the counter's reading for a device copy of known size
# (fetch x 2.0000, write x 1.0000).  Valid only for the kernel sources they were
# taken on: KERNEL_SOURCES_SHA is the first 16 hex digits of the SHA-256 of the
# sources listed in kernel_sources_sha(); any change makes `traffic` null.
TRAFFIC = {
    "sources_sha": "c29bc817e698ec8d",
    # the kernels of one kda_chunk_prefill call at h32_t64k: the two segment-pass
    # launches (the head walk, and the pass over segments whose map did not
    # vanish, whose workgroups all exit here), the prefill of every segment from
    # zero, the merge, the corrected heads
    "segment_pass_launches": 0.03354e9,
    "zero_start_segments": 2.15312e9 + 0.55366e9,
    "segment_merge": 0.00219e9 + 0.00210e9,
    "corrected_heads": 0.07440e9 + 0.01468e9,
    "decode_step": 0.5455e9 + 0.5390e9,
    # the backward's three kernels at B=4, H=32, T=8192, d=128: forward
    # checkpoint pass, reverse chain, per-chunk gradients
    "backward": (0.8164e9 + 0.8137e9) + (1.0849e9 + 0.8137e9) + (2.6868e9 + 0.8075e9),
}


# the kernels one kda_chunk_prefill call launches at the headline workload
TRAFFIC_PATH = ("segment_pass_launches", "zero_start_segments", "segment_merge", "corrected_heads")


def kernel_sources_sha():
    import hashlib
    h = hashlib.sha256()
    for f in ("kda_api.hip", "kda_chunk.hip", "kda_decode.hip", "kda_device.hpp", "kda_launch.hpp",
              "kda_merge.hip", "kda_bwgrad.hip"):
        with open(os.path.join(ROOT, "gated_delta_rule_104_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def prefill_bytes(B, H, T, D):
    """Algorithmic HBM bytes of one bf16 prefill: q, k, log_alpha, v read and o
    written once (2 B each per channel), beta read once, S_T written (fp32)."""
    per_token_head = 2 * (3 * D + D + D) + 2
    return B * H * T * per_token_head + B * H * D * D * 4


def prefill_flops(B, H, T, D, triangle=False):
    """Matrix flops per chunk-head of the chunked form (dense 16x16 tiles or
    triangle-aware): scores A and P, the UT/WY products, the state chain."""
    C, K, V = CH, D, D
    if triangle:
        per_chunk = 2 * C * C * K + C * C * (K + V) + 6 * C * K * V + C * C * V + C * C * C // 3
    else:
        per_chunk = 2 * (2 * C * C * K) + 2 * C * C * (K + V) + 6 * C * K * V + 2 * C * C * V \
            + 2 * C * C * C // 3
    nchunks = -(-T // C)
    return B * H * nchunks * per_chunk


MIN_TIMED = 20  # every figure is the median of at least this many event-timed launches


def time_launches(fn, n, exact=False):
    """Median and list of per-launch durations (ms) from events on the current
    stream, each launch between its own pair of events: n launches if exact (the
    headline's K steps), else at least MIN_TIMED."""
    n = n if exact else max(n, MIN_TIMED)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for a, b in evs:
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    ts = [a.elapsed_time(b) for a, b in evs]
    return statistics.median(ts), ts


def segment_pass_bytes(B, H, T, D, G):
    """Algorithmic bytes of the segment transfer pass: k, log_alpha, v and beta read
    once; a zero-start end state and a transfer map (fp32, D x D) written per
    segment and head."""
    return B * H * T * (2 * 3 * D + 2) + 2 * G * B * H * D * D * 4


def merge_bytes(B, H, D, G):
    """Merge: read every segment's end state and map, write every start state and S_T."""
    return G * B * H * D * D * 4 * 3 + B * H * D * D * 4


def segment_prefill_bytes(B, H, T, D, G):
    """Segmented prefill: q, k, log_alpha, v, beta read and o written once, a start
    state read per segment and head, S_T written."""
    return B * H * T * (2 * 5 * D + 2) + G * B * H * D * D * 4 + B * H * D * D * 4


def direct_part_bytes(B, H, T0, D):
    """Direct prefill of the first T0 tokens: q, k, log_alpha, v, beta read and o
    written once, its end state written (from a zero start, nothing read)."""
    return B * H * T0 * (2 * 5 * D + 2) + B * H * D * D * 4


HEAD_CHUNKS = 4  # the library's default for option head_chunks


def bench_decomposition(pf, args):
    """Per-kernel durations of the sequence-split prefill, through the public calls
    it is made of, with the same launch shapes as kda_chunk_prefill."""
    g = pf["g"]
    B, H, T, D = pf["B"], pf["H"], pf["T"], pf["D"]
    T0, G, Tseg = kda.prefill_plan(B, H, T, D, D, torch.bfloat16)
    if G == 1:
        return None
    if T0 == 0:
        return bench_decomposition_heads(pf, args, G, Tseg)
    dev = g["k"].device
    T1 = T0 + (G - 1) * Tseg
    names = ("q", "k", "v", "log_alpha", "beta")
    head = {n: g[n][:, :, :T0].contiguous() for n in names}
    mid = {n: g[n][:, :, T0:T1].contiguous() for n in names[1:]}
    tail = {n: g[n][:, :, T0:].contiguous() for n in names}
    Z = torch.empty(G - 1, B, H, D, D, dtype=torch.float32, device=dev)
    M = torch.empty_like(Z)
    S1 = torch.empty(B, H, D, D, dtype=torch.float32, device=dev)
    S_start = torch.empty(G, B, H, D, D, dtype=torch.float32, device=dev)
    S_T = torch.empty(B, H, D, D, dtype=torch.float32, device=dev)
    o0 = torch.empty(B, H, T0, D, dtype=torch.bfloat16, device=dev)
    o1 = torch.empty(B, H, T - T0, D, dtype=torch.bfloat16, device=dev)

    def direct():
        # the call's own choice for this part: 4 consumer waves, one workgroup per head
        with kda.options(nc=4):
            kda.prefill(head["q"], head["k"], head["v"], head["log_alpha"], head["beta"], None, o=o0, S_T=S1,
                        workspace=None)

    parts = {
        "direct_part": (direct, direct_part_bytes(B, H, T0, D)),
        "segment_transfer": (lambda: kda.segment_transfer(mid["k"], mid["v"], mid["log_alpha"], mid["beta"],
                                                          G - 1, S_zero_end=Z, M=M),
                             segment_pass_bytes(B, H, T1 - T0, D, G - 1)),
        "segment_merge": (lambda: kda.segment_merge(Z, M, S1, S_start=S_start[: G - 1], S_T=S_start[G - 1]),
                          merge_bytes(B, H, D, G - 1) + B * H * D * D * 4),
        "segment_prefill": (lambda: kda.prefill_segments(tail["q"], tail["k"], tail["v"], tail["log_alpha"],
                                                         tail["beta"], S_start, Tseg, o=o1, S_T=S_T),
                            segment_prefill_bytes(B, H, T - T0, D, G)),
    }
    for fn, _ in parts.values():
        fn()
    torch.cuda.synchronize()
    res = {"T0": T0, "G": G, "Tseg": Tseg}
    n = max(5, args.steps)
    for name, (fn, nbytes) in parts.items():
        # each launch alone between events on the stream it runs on
        ms, _ = time_launches(fn, n)
        res[name] = {"ms": ms, "algorithmic_bytes": nbytes, "GBs": nbytes / (ms * 1e-3) / 1e9}
    del head, mid, tail
    return res


def bench_decomposition_heads(pf, args, G, Tseg):
    """The default split pipeline (segments from zero, heads corrected), piece by
    piece through public calls with the launch shapes it uses:
    - head_walk: the segment pass over the first HEAD_CHUNKS chunks of segments
      1 .. G-1 (224 workgroups here); inside the call only the map columns run,
      so the public call, which also carries the state columns, bounds it above;
    - zero_start_segments: the prefill of all G segments from zero (one
      workgroup per segment and head), the dominant kernel; inside the call it
      also writes every segment's end state;
    - segment_merge: the merge over segments 1 .. G-1; inside the call the maps
      that vanished are neither read nor applied, so this bounds it above;
    - corrected_heads: the prefill of the first HEAD_CHUNKS chunks of segments
      1 .. G-1 from their start states.
    With the workloads' gates every map vanishes within the head, so the
    segment pass over the other segments does no work (its workgroups exit)."""
    g = pf["g"]
    B, H, T, D = pf["B"], pf["H"], pf["T"], pf["D"]
    dev = g["k"].device
    Lh = HEAD_CHUNKS * CH
    starts = [i * Tseg for i in range(1, G)]
    if any(s + Lh > T for s in starts):
        return None
    names = ("q", "k", "v", "log_alpha", "beta")
    heads = {n: torch.cat([g[n][:, :, s:s + Lh] for s in starts], dim=2).contiguous() for n in names}
    Zh = torch.empty(G - 1, B, H, D, D, dtype=torch.float32, device=dev)
    Mh = torch.empty_like(Zh)
    S_start = torch.empty_like(Zh)
    S_T = torch.empty(B, H, D, D, dtype=torch.float32, device=dev)
    S_T2 = torch.empty_like(S_T)
    o_all = torch.empty(B, H, T, D, dtype=torch.bfloat16, device=dev)
    o_heads = torch.empty(B, H, (G - 1) * Lh, D, dtype=torch.bfloat16, device=dev)
    Ztot = torch.randn(G - 1, B, H, D, D, device=dev)
    Mtot = torch.randn(G - 1, B, H, D, D, device=dev) * 0.01
    S1 = torch.randn(B, H, D, D, device=dev)

    def corrected():
        # the call's launch shape for this piece: 4 consumer waves, one workgroup per segment
        with kda.options(nc=4):
            kda.prefill_segments(heads["q"], heads["k"], heads["v"], heads["log_alpha"], heads["beta"], S_start,
                                 Lh, o=o_heads, S_T=S_T2)

    parts = {
        "head_walk": (lambda: kda.segment_transfer(heads["k"], heads["v"], heads["log_alpha"], heads["beta"],
                                                   G - 1, S_zero_end=Zh, M=Mh),
                      segment_pass_bytes(B, H, (G - 1) * Lh, D, G - 1)),
        "zero_start_segments": (lambda: kda.prefill_segments(g["q"], g["k"], g["v"], g["log_alpha"], g["beta"],
                                                             None, Tseg, o=o_all, S_T=S_T),
                                zero_start_bytes(B, H, T, D, G)),
        "segment_merge": (lambda: kda.segment_merge(Ztot, Mtot, S1, S_start=S_start, S_T=S_T2),
                          merge_bytes(B, H, D, G - 1)),
        "corrected_heads": (corrected, segment_prefill_bytes(B, H, (G - 1) * Lh, D, G - 1)),
    }
    for fn, _ in parts.values():
        fn()
    torch.cuda.synchronize()
    res = {"T0": 0, "G": G, "Tseg": Tseg, "head_chunks": HEAD_CHUNKS}
    n = max(5, args.steps)
    for name, (fn, nbytes) in parts.items():
        ms, _ = time_launches(fn, n)
        res[name] = {"ms": ms, "algorithmic_bytes": nbytes, "GBs": nbytes / (ms * 1e-3) / 1e9}
    del heads, o_all, o_heads
    return res


def zero_start_bytes(B, H, T, D, G):
    """Prefill of every segment from zero: q, k, log_alpha, v, beta read and o
    written once, an end state written per segment and head."""
    return B * H * T * (2 * 5 * D + 2) + G * B * H * D * D * 4


STAMP_FIRST, STAMP_STEPS, STAMP_WAVES = 32, 16, 8  # the profiling build's recording window


def phase_stamps(dev, which="prefill"):
    """Where a pipeline step of a chunk kernel goes, from the profiling build's
    per-wave shader-clock stamps of steps 32 .. 47 on every workgroup: median
    cycles of each phase for consumer waves (the chain) and producer waves (the
    elementwise phase), the waits at the two barriers, and the step period
    (start to the next step's start, earliest wave).  which: "prefill", the
    h32_t64k prefill's main kernel (every segment from zero); "ckpt" or
    "reverse", the checkpoint pass or the reverse chain of the b4_h32_t8k
    prefill gradients."""
    import ctypes
    import numpy as np
    kda.LIB_PATH = os.path.join(ROOT, "gated_delta_rule_104_amd", "libkda_stamps.so")
    lib = kda.load()
    if which == "prefill":
        B, H, T, D = 1, 32, 65536, 128
        T0, G, Tseg = kda.prefill_plan(B, H, T, D, D, torch.bfloat16)
        assert T0 == 0 and G > 1, "the phase split is recorded on the split prefill's main launch"
        nwg = B * H * G
        g = ki.gen_prefill(B, H, T, D, D, "bf16", seed=2, device=dev)
        call = lambda: kda.prefill(g["q"], g["k"], g["v"], g["log_alpha"], g["beta"], None)
    else:
        B, H, T, D = 4, 32, 8192, 128
        nwg = B * H  # one workgroup per head (both chains, side by side, fill the chip once)
        g = ki.gen_prefill(B, H, T, D, D, "bf16", seed=1, s0_std=0.1, device=dev)
        gen = torch.Generator(device=dev).manual_seed(6)
        dO = torch.randn(B, H, T, D, generator=gen, device=dev).to(torch.bfloat16)
        dST = torch.randn(B, H, D, D, generator=gen, device=dev)
        ws = torch.empty(kda.backward_workspace_bytes(B, H, T, D, D, torch.bfloat16), dtype=torch.uint8, device=dev)
        call = lambda: kda.prefill_backward(g["q"], g["k"], g["v"], g["log_alpha"], g["beta"], g["S0"], dO, dST,
                                            workspace=ws)
    st = torch.zeros(nwg * STAMP_STEPS * STAMP_WAVES * 5, dtype=torch.int64, device=dev)
    for _ in range(30 if which == "prefill" else 10):
        call()
    torch.cuda.synchronize()
    os.environ["KDA_STAMP_TARGET"] = which
    kda._check(lib.kda_debug_phase_stamps(ctypes.c_void_p(st.data_ptr()), ctypes.c_size_t(st.numel())),
               "kda_debug_phase_stamps")
    call()
    torch.cuda.synchronize()
    kda._check(lib.kda_debug_phase_stamps(None, ctypes.c_size_t(0)), "kda_debug_phase_stamps")
    s = st.cpu().numpy().reshape(nwg, STAMP_STEPS, STAMP_WAVES, 5).astype(np.float64)
    s = s[(s[:, :, :, 0] > 0).all(axis=(1, 2))]  # workgroups that ran these steps (an exited one records none)
    assert len(s), "no workgroup recorded its steps"
    nc = 4  # consumer waves (the rest produce)
    cons, prod = s[:, :-1, :nc], s[:, :-1, nc:]
    med = lambda x: float(np.median(x))
    out = {"launch": which, "workgroups": len(s), "steps": f"{STAMP_FIRST}..{STAMP_FIRST + STAMP_STEPS - 1}",
           "unit": "cycles", "period": med(s[:, 1:, :, 0].min(axis=2) - s[:, :-1, :, 0].min(axis=2))}
    for name, w, first in (("consumers", cons, "chain"), ("producers", prod, "elementwise")):
        out[name] = {first: med(w[..., 1] - w[..., 0]), "wait_barrier_1": med(w[..., 2] - w[..., 1]),
                     "score_tiles": med(w[..., 3] - w[..., 2]), "wait_barrier_2": med(w[..., 4] - w[..., 3])}
    return out


def bench_prefill(args, dev):
    B, H, T, D = 1, 32, 65536, 128
    print(f"[bench] generating prefill inputs B={B} H={H} T={T} D={D} bf16", file=sys.stderr, flush=True)
    g = ki.gen_prefill(B, H, T, D, D, "bf16", seed=2, device=dev)
    o = torch.empty(B, H, T, D, dtype=torch.bfloat16, device=dev)
    S_T = torch.empty(B, H, D, D, dtype=torch.float32, device=dev)
    nws = kda.prefill_workspace_bytes(B, H, T, D, D, torch.bfloat16)
    ws = torch.empty(nws, dtype=torch.uint8, device=dev) if nws else None

    def step():
        kda.prefill(g["q"], g["k"], g["v"], g["log_alpha"], g["beta"], None, o=o, S_T=S_T, workspace=ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # the main launch of every timed step (the prefill of every segment from
    # zero), timed by the library with events on this stream around it
    T0, G, _ = kda.prefill_plan(B, H, T, D, D, torch.bfloat16)
    timed = T0 == 0 and G > 1 and args.steps <= 256
    if timed:
        kda.debug_time_main_launches(args.steps)
    t0 = time.perf_counter()
    med_ms, per = time_launches(step, args.steps, exact=True)
    t1 = time.perf_counter()
    wall_ms = (t1 - t0) * 1e3 / len(per)
    main_ms = kda.debug_main_launch_ms() if timed else []
    if timed:
        kda.debug_time_main_launches(0)
    return dict(B=B, H=H, T=T, D=D, median_ms=med_ms, mean_ms=sum(per) / len(per), wall_ms=wall_ms,
                per=per, g=g, ws_bytes=nws, main_ms=main_ms)


def bench_prefill_batched(args, dev):
    """The batched prefill workload B=4, H=32, T=8192, d=128 (bf16 inputs, fp32
    start state): time per call, tokens/s and the fractions of the MFMA and HBM
    roofs, measured after the headline steps."""
    B, H, T, D = 4, 32, 8192, 128
    print(f"[bench] generating prefill inputs B={B} H={H} T={T} D={D} bf16", file=sys.stderr, flush=True)
    g = ki.gen_prefill(B, H, T, D, D, "bf16", seed=1, s0_std=0.1, device=dev)
    o = torch.empty(B, H, T, D, dtype=torch.bfloat16, device=dev)
    S_T = torch.empty(B, H, D, D, dtype=torch.float32, device=dev)
    nws = kda.prefill_workspace_bytes(B, H, T, D, D, torch.bfloat16)
    ws = torch.empty(nws, dtype=torch.uint8, device=dev) if nws else None

    def call():
        kda.prefill(g["q"], g["k"], g["v"], g["log_alpha"], g["beta"], g["S0"], o=o, S_T=S_T, workspace=ws)

    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    ms, _ = time_launches(call, max(5, args.steps))
    nbytes = prefill_bytes(B, H, T, D) + B * H * D * D * 4  # + the start state read
    fl = prefill_flops(B, H, T, D)
    del g, o, ws
    return {"B": B, "H": H, "T": T, "D": D, "ms": ms, "tokens_per_s": B * T / (ms * 1e-3),
            "hbm_frac": nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
            "mfma_dense_tile_frac": fl / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
            "plan": list(kda.prefill_plan(B, H, T, D, D, torch.bfloat16))}


def bench_prefill_slow_decay(args, dev):
    """The headline prefill shape with slowly decaying gates (log_alpha x 1e-3,
    beta x 0.05, the stress variant of the parity tests).  Under these gates the
    segment pass's transfer-map columns never reach zero, so none of its waves
    stop early: this is the split path's cost when nothing decays away."""
    B, H, T, D = 1, 32, 65536, 128
    print(f"[bench] generating slow-decay prefill inputs B={B} H={H} T={T} D={D} bf16", file=sys.stderr,
          flush=True)
    g = ki.gen_prefill(B, H, T, D, D, "bf16", seed=2, device=dev, variant="slow")
    o = torch.empty(B, H, T, D, dtype=torch.bfloat16, device=dev)
    S_T = torch.empty(B, H, D, D, dtype=torch.float32, device=dev)
    nws = kda.prefill_workspace_bytes(B, H, T, D, D, torch.bfloat16)
    ws = torch.empty(nws, dtype=torch.uint8, device=dev) if nws else None

    def call():
        kda.prefill(g["q"], g["k"], g["v"], g["log_alpha"], g["beta"], None, o=o, S_T=S_T, workspace=ws)

    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    ms, _ = time_launches(call, max(5, args.steps))
    del g, o, ws
    return {"B": B, "H": H, "T": T, "D": D, "gates": "log_alpha x 1e-3, beta x 0.05", "ms": ms,
            "tokens_per_s": B * T / (ms * 1e-3),
            "mfma_dense_tile_frac": prefill_flops(B, H, T, D) / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS}


def backward_bytes(B, H, T, D):
    """Algorithmic bytes of kda_prefill_backward with bf16 inputs: q, k, v,
    log_alpha, dO (2 B x D each) and beta read once per token-head; dq, dk, dv,
    dlog_alpha (2 B x D each, the inputs' dtype) and dbeta written once; S0 and
    dS_T read and dS0 written (fp32) per head.  The checkpoints the three
    kernels pass to each other through the workspace are not counted."""
    return B * H * T * (2 * 5 * D + 2 + 2 * 4 * D + 2) + 3 * B * H * D * D * 4


def backward_path_bytes(B, H, T, D, C=CH, halves=False):
    """HBM bytes the kernels of the bf16 backward move by design, per
    chunk-head (2-byte elements unless noted):
      forward checkpoint pass: reads k, v, log_alpha, beta; writes the chunk's
        start state S (D x D) and Delta (C x D);
      reverse chain: reads q, k, log_alpha, dO, beta; writes dv and dU (D x D);
      per-chunk gradients: reads q, k, log_alpha, dO, dv, beta and S, dU,
        Delta; writes dq, dk, dlog_alpha, dbeta;
    plus S0, dS_T read and dS0 and the forward pass's (unused) end state
    written once per head (fp32); with the reverse chain in two halves (option
    bw_overlap, 16 chunks per head and more), dS at their boundary written and
    read once more.
    The rows the chain kernels keep only for tokens with beta below 2^-30 (none
    in the benchmark's inputs) are not counted."""
    tok = C * 2 * D                     # one [C][D] bf16 tile
    k1 = 3 * tok + 2 * C + D * D * 2 + tok
    k2 = 4 * tok + 2 * C + tok + D * D * 2
    k3 = 5 * tok + 2 * C + 2 * D * D * 2 + tok + 3 * tok + 2 * C
    nchunks = -(-T // C)
    extra = 2 if halves and nchunks >= 16 else 0
    return B * H * nchunks * (k1 + k2 + k3) + (4 + extra) * B * H * D * D * 4


def backward_flops(B, H, T, D, C=CH):
    """Matrix flops the chunked backward issues per call, on dense 16x16 tiles
    (triangles and the 16-row diagonal blocks counted whole):
      forward checkpoint pass per chunk-head: scores Kh Kb^T (2C^2K), Kh S and
        Kb^T Delta (2CKV each), the 16-row block solve (C^2 V);
      reverse chain: scores L and P (2C^2K each), Kb dU, Qh^T dO and Kh^T Xbar
        (2CKV each), P^T dO (2C^2V), the block solve (C^2 V);
      per-chunk gradients: the four 64x64 products dP, dP^T, Abar, Abar^T
        (2C^2D each), dO S^T, Xbar S^T and Delta dU^T (2CKV each), and the four
        products with the 64x64 gradients, each run twice on split operands
        (8 x 2C^2K)."""
    K = V = D
    fwd = 2 * C * C * K + 2 * (2 * C * K * V) + C * C * V
    chain = 2 * (2 * C * C * K) + 3 * (2 * C * K * V) + 2 * C * C * V + C * C * V
    grads = 4 * (2 * C * C * D) + 3 * (2 * C * K * V) + 8 * (2 * C * C * K)
    nchunks = -(-T // C)
    return B * H * nchunks * (fwd + chain + grads)


def bench_backward(args, dev):
    """Gradients of the batched prefill workload B=4, H=32, T=8192, d=128 (bf16
    inputs, fp32 start state, dO and dS_T given): time per call and tokens/s."""
    B, H, T, D = 4, 32, 8192, 128
    print(f"[bench] generating backward inputs B={B} H={H} T={T} D={D} bf16", file=sys.stderr, flush=True)
    g = ki.gen_prefill(B, H, T, D, D, "bf16", seed=1, s0_std=0.1, device=dev)
    gen = torch.Generator(device=dev).manual_seed(6)
    dO = torch.randn(B, H, T, D, generator=gen, device=dev).to(torch.bfloat16)
    dST = torch.randn(B, H, D, D, generator=gen, device=dev)
    ws = torch.empty(kda.backward_workspace_bytes(B, H, T, D, D, torch.bfloat16), dtype=torch.uint8, device=dev)

    def call():
        kda.prefill_backward(g["q"], g["k"], g["v"], g["log_alpha"], g["beta"], g["S0"], dO, dST, workspace=ws)

    for _ in range(3):
        call()
    torch.cuda.synchronize()
    ms, _ = time_launches(call, MIN_TIMED)
    nbytes = backward_bytes(B, H, T, D)
    pbytes = backward_path_bytes(B, H, T, D)
    fl = backward_flops(B, H, T, D)
    traffic = TRAFFIC["backward"] if kernel_sources_sha() == TRAFFIC["sources_sha"] else None
    del g, dO, ws
    return {"B": B, "H": H, "T": T, "D": D, "ms": ms, "tokens_per_s": B * T / (ms * 1e-3),
            "algorithmic_bytes": nbytes, "hbm_frac": nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
            # the bound: HBM over the bytes the three kernels move with their checkpoints
            "bound": "hbm", "path_bytes": pbytes, "path_GBs": pbytes / (ms * 1e-3) / 1e9,
            "path_hbm_frac": pbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, "traffic": traffic,
            "issued_mfma_tflops": fl / (ms * 1e-3) / 1e12,
            "mfma_frac": fl / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, "mfma_peak_tflops": PEAK_BF16_TFLOPS,
            "kernels": "forward checkpoint pass beside the reverse chain, then per-chunk gradients"}


def bench_snapshots(pf, args, interval=512):
    """The same prefill with a state snapshot every `interval` tokens (prefix
    caching): time per call, the snapshot bytes written, and the cost over the
    plain call measured in the same run."""
    g = pf["g"]
    B, H, T, D = pf["B"], pf["H"], pf["T"], pf["D"]
    dev = g["k"].device
    nsnap = T // interval
    o = torch.empty(B, H, T, D, dtype=torch.bfloat16, device=dev)
    S_T = torch.empty(B, H, D, D, dtype=torch.float32, device=dev)
    snaps = torch.empty(B, nsnap, H, D, D, dtype=torch.float32, device=dev)
    ws = torch.empty(pf["ws_bytes"], dtype=torch.uint8, device=dev) if pf["ws_bytes"] else None

    def snap():
        kda.prefill_snap(g["q"], g["k"], g["v"], g["log_alpha"], g["beta"], interval, None, o=o, S_T=S_T,
                         S_snap=snaps, workspace=ws)

    def plain():
        kda.prefill(g["q"], g["k"], g["v"], g["log_alpha"], g["beta"], None, o=o, S_T=S_T, workspace=ws)

    snap(); plain()
    torch.cuda.synchronize()
    n = max(5, args.steps)
    ms, _ = time_launches(snap, n)
    base, _ = time_launches(plain, n)
    del snaps
    return {"interval": interval, "snapshots_per_head": nsnap, "ms": ms, "plain_ms": base,
            "overhead": ms / base - 1.0, "snapshot_bytes": B * H * nsnap * D * D * 4}


def bench_decode(args, dev):
    N, H, D, steps = 256, 32, 128, args.decode_steps
    print(f"[bench] generating decode inputs N={N} H={H} D={D} steps={steps}", file=sys.stderr, flush=True)
    S = ki.gen_decode_state(N, H, D, D, seed=4, device=dev)
    pool = [ki.gen_decode_step(N, H, D, D, "bf16", seed=4, step=t, device=dev) for t in range(steps)]
    o = torch.empty(N, H, D, dtype=torch.bfloat16, device=dev)
    for t in range(8):
        x = pool[t]
        kda.decode_step(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], S, o=o)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for t in range(steps):
        x = pool[t]
        kda.decode_step(x["q"], x["k"], x["v"], x["log_alpha"], x["beta"], S, o=o)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b)
    per_step_bytes = N * H * (2 * D * D * 4 + 2 * (3 * D + D + D) + 2)
    step_ms = ms / steps
    gbs = per_step_bytes / (step_ms * 1e-3) / 1e9
    del pool
    traffic = TRAFFIC["decode_step"] if kernel_sources_sha() == TRAFFIC["sources_sha"] else None
    return dict(N=N, H=H, D=D, steps=steps, ms_total=ms, us_per_step=step_ms * 1e3,
                tokens_per_s=N * steps / (ms * 1e-3), achieved_GBs=gbs, hbm_frac=gbs / PEAK_HBM_GBS,
                bytes_per_step=per_step_bytes, traffic_per_step=traffic)


def bench_decode_tokens(args, dev, ntok=4):
    """Speculative-decoding verification: ntok draft tokens for each of 256
    sequences x 32 heads in one call (state read and written once), with and
    without the per-token rollback states."""
    N, H, D = 256, 32, 128
    # token t's inputs are decode step t's draws (one generator per token, over all heads)
    steps = [ki.gen_decode_step(N, H, D, D, "bf16", seed=5, step=t, device=dev) for t in range(ntok)]
    g = {n: torch.stack([x[n] for x in steps], dim=2).contiguous() for n in steps[0]}
    S = ki.gen_decode_state(N, H, D, D, seed=5, device=dev)
    S_out = torch.empty_like(S)
    o = torch.empty(N, H, ntok, D, dtype=torch.bfloat16, device=dev)
    S_pos = torch.empty(N, ntok, H, D, D, dtype=torch.float32, device=dev)

    def call(pos):
        kda.decode_tokens(g["q"], g["k"], g["v"], g["log_alpha"], g["beta"], S, S_out=S_out, o=o,
                          S_pos=S_pos if pos else None)

    call(False); call(True)
    torch.cuda.synchronize()
    n = max(10, args.steps)
    ms, _ = time_launches(lambda: call(False), n)
    ms_pos, _ = time_launches(lambda: call(True), n)
    nbytes = N * H * (2 * D * D * 4 + ntok * (2 * (3 * D + D + D) + 2))
    pos_bytes = N * H * ntok * D * D * 4
    del g, S_pos
    return {"N": N, "H": H, "D": D, "ntok": ntok, "ms": ms, "tokens_per_s": N * ntok / (ms * 1e-3),
            "algorithmic_bytes": nbytes, "hbm_frac": nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
            "with_positions_ms": ms_pos,
            "with_positions_hbm_frac": (nbytes + pos_bytes) / (ms_pos * 1e-3) / 1e9 / PEAK_HBM_GBS}


def bench_kcp(args, dev):
    """The context-parallel decomposition on one GPU at T = 1,048,576 in 8
    segments of 131,072 tokens (H = 32): the segment pass (each segment's
    zero-start end state and transfer map), the sequential merge (every
    segment's true start state), and the prefill of every segment from its start
    state, which produces the outputs.  Beside them, kda_chunk_prefill on the
    same sequence (its plan cuts the same 8 segments; it prefills them from
    zero and corrects their heads)."""
    B, H, G, Tseg, D = 1, 32, 8, 131072, 128
    T = G * Tseg
    print(f"[bench] generating kcp inputs H={H} T={T} G={G}", file=sys.stderr, flush=True)
    g = ki.gen_prefill(B, H, T, D, D, "bf16", seed=3, device=dev)
    Z = torch.empty(G, B, H, D, D, dtype=torch.float32, device=dev)
    M = torch.empty(G, B, H, D, D, dtype=torch.float32, device=dev)
    S_start = torch.empty_like(Z)
    S_T = torch.empty(B, H, D, D, dtype=torch.float32, device=dev)
    S_T2 = torch.empty_like(S_T)
    o = torch.empty(B, H, T, D, dtype=torch.bfloat16, device=dev)

    def transfer():
        kda.segment_transfer(g["k"], g["v"], g["log_alpha"], g["beta"], G, S_zero_end=Z, M=M)

    def merge():
        kda.segment_merge(Z, M, None, S_start=S_start, S_T=S_T)

    def prefill():
        kda.prefill_segments(g["q"], g["k"], g["v"], g["log_alpha"], g["beta"], S_start, Tseg, o=o, S_T=S_T2)

    ws = torch.empty(kda.prefill_workspace_bytes(B, H, T, D, D, torch.bfloat16), dtype=torch.uint8, device=dev)

    def call():
        kda.prefill(g["q"], g["k"], g["v"], g["log_alpha"], g["beta"], None, o=o, S_T=S_T2, workspace=ws)

    transfer(); merge(); prefill(); call()
    torch.cuda.synchronize()
    t_ms, _ = time_launches(transfer, MIN_TIMED)
    m_ms, _ = time_launches(merge, MIN_TIMED)
    p_ms, _ = time_launches(prefill, MIN_TIMED)
    c_ms, _ = time_launches(call, MIN_TIMED)
    plan = list(kda.prefill_plan(B, H, T, D, D, torch.bfloat16))
    nbytes = B * H * T * (2 * (2 * D + D) + 2) + 2 * G * B * H * D * D * 4
    pbytes = segment_prefill_bytes(B, H, T, D, G)
    del g, o, ws
    return dict(H=H, T=T, G=G, Tseg=Tseg, transfer_ms=t_ms, merge_ms=m_ms,
                tokens_per_s=T / ((t_ms + m_ms) * 1e-3),
                transfer_GBs=nbytes / (t_ms * 1e-3) / 1e9,
                segment_prefill_ms=p_ms, segment_prefill_GBs=pbytes / (p_ms * 1e-3) / 1e9,
                with_outputs_ms=t_ms + m_ms + p_ms,
                with_outputs_tokens_per_s=T / ((t_ms + m_ms + p_ms) * 1e-3),
                prefill_call_ms=c_ms, prefill_call_plan=plan, prefill_call_tokens_per_s=T / (c_ms * 1e-3))


def bench_calibration(dev):
    """What this machine reaches beside the spec peaks the fractions are taken
    against: a large bf16 matrix product through torch (hipBLASLt) and a plain
    device-to-device copy (read + write), each timed with events."""
    n = 8192
    a = torch.randn(n, n, device=dev, dtype=torch.bfloat16)
    b = torch.randn(n, n, device=dev, dtype=torch.bfloat16)
    for _ in range(3):
        torch.matmul(a, b)
    torch.cuda.synchronize()
    mm_ms, _ = time_launches(lambda: torch.matmul(a, b), 10)
    del a, b
    nbytes = 1 << 30
    src = torch.ones(nbytes, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    cp_ms, _ = time_launches(lambda: dst.copy_(src), 10)
    del src, dst
    return {"bf16_gemm_8192_tflops": 2 * n ** 3 / (mm_ms * 1e-3) / 1e12,
            "copy_1GiB_GBs": 2 * nbytes / (cp_ms * 1e-3) / 1e9,
            "spec_bf16_tflops": PEAK_BF16_TFLOPS, "spec_hbm_GBs": PEAK_HBM_GBS}


def cpu_model():
    """The host CPU's model name (from /proc/cpuinfo where present)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def cpu_baseline(pf, budget_s):
    """fp64 oracle on a bounded sample of the same prefill inputs: all heads and
    tokens if that fits in about `budget_s` seconds, else the first `nh` heads and
    the first `tt` tokens, sized from a short calibration run."""
    import oracle
    g = pf["g"]
    H, T = pf["H"], pf["T"]
    nthreads = oracle.max_threads()
    nh = min(H, max(1, nthreads))
    sl = lambda x, nh, tt: x[:, :nh, :tt].cpu()
    tt = 1024
    t0 = time.perf_counter()
    oracle.prefill(*(sl(g[n], nh, tt) for n in ("q", "k", "v", "log_alpha", "beta")))
    per_tok = (time.perf_counter() - t0) / tt  # seconds per token over nh heads
    if per_tok * T * (-(-H // nh)) <= budget_s:
        nh, tt = H, T
    else:
        tt = int(min(T, max(1024, budget_s / max(per_tok, 1e-9))))
        tt = max(CH, tt - tt % CH)
    args = [sl(g[n], nh, tt) for n in ("q", "k", "v", "log_alpha", "beta")]
    t0 = time.perf_counter()
    oracle.prefill(*args, want_o=True)
    el = time.perf_counter() - t0
    token_heads_per_s = nh * tt / el
    what = "the whole workload" if (nh, tt) == (H, T) else \
        f"{nh} of {H} heads x first {tt} tokens of the same inputs"
    return {"value": token_heads_per_s / H, "unit": "tokens/s", "cores": nthreads, "kind": "oracle",
            "cpu_model": cpu_model(), "host_cpus": os.cpu_count(),
            "sample": f"{what} ({el:.1f} s, fp64, outputs and end states); tokens/s over all {H} heads"}


def summarize_profiles(paths):
    """Summaries of rocprofv3 CSV output (no GPU needed): the `--stats` table
    (`*_kernel_stats.csv`) per kernel name; a kernel trace
    (`*_kernel_trace.csv`) grouped by kernel name and grid size, with dispatch
    count and mean / median / quartiles / min / max duration in microseconds
    (the quartiles separate two launches of one shape that take different
    times, such as the split prefill's two segment-pass launches); a counter
    collection (`*_counter_collection.csv`) grouped the same way, each counter
    summed over its dimensions per dispatch, then averaged over dispatches."""
    import collections
    import csv

    def short(name):
        return name.replace("void ", "")[:110]

    for path in paths:
        with open(path, newline="") as fh:
            rows = list(csv.DictReader(fh))
        print(f"## {os.path.basename(path)} ({len(rows)} rows)")
        if not rows:
            continue
        if "AverageNs" in rows[0]:  # the --stats summary, per kernel name
            for r in rows:
                print(f"  {short(r['Name'])} | n={r['Calls']} mean {float(r['AverageNs']) / 1e3:.1f} us  "
                      f"min {float(r['MinNs']) / 1e3:.1f}  max {float(r['MaxNs']) / 1e3:.1f}  "
                      f"share {float(r['Percentage']):.2f}%")
        elif "Counter_Name" in rows[0]:
            agg = collections.defaultdict(lambda: collections.defaultdict(lambda: collections.defaultdict(float)))
            for r in rows:
                key = (short(r["Kernel_Name"]), r["Grid_Size"])
                agg[key][r["Counter_Name"]][r["Dispatch_Id"]] += float(r["Counter_Value"])
            for (kname, grid), cs in sorted(agg.items()):
                parts = [f"{c}={statistics.mean(per.values()):.6g} (n={len(per)})" for c, per in sorted(cs.items())]
                print(f"  {kname} | grid {grid} | " + " ".join(parts))
        else:
            agg = collections.defaultdict(list)
            meta = {}
            for r in rows:
                key = (short(r["Kernel_Name"]), r.get("Grid_Size", r.get("Grid_Size_X", "")))
                agg[key].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1000.0)
                meta[key] = (r.get("Workgroup_Size", r.get("Workgroup_Size_X", "")),
                             r.get("LDS_Block_Size", r.get("Lds_Size", "")), r.get("Scratch_Size", ""),
                             r.get("Arch_VGPR_Count", r.get("VGPR_Count", "")))
            for key, ds in sorted(agg.items(), key=lambda kv: -sum(kv[1])):
                wg, lds, scr, vgpr = meta[key]
                q1, _, q3 = statistics.quantiles(ds, n=4) if len(ds) > 1 else (ds[0], ds[0], ds[0])
                print(f"  {key[0]} | grid {key[1]} wg {wg} lds {lds} scratch {scr} vgpr column {vgpr} | n={len(ds)} "
                      f"mean {statistics.mean(ds):.1f} us  median {statistics.median(ds):.1f}  "
                      f"quartiles {q1:.1f} / {q3:.1f}  min {min(ds):.1f}  max {max(ds):.1f}")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--decode-steps", type=int, default=1024,
                    help="consecutive decode steps timed (the workload is 1024)")
    ap.add_argument("--no-kcp", action="store_true")
    ap.add_argument("--no-snap", action="store_true")
    ap.add_argument("--no-batched", action="store_true", help="skip the B=4 T=8192 prefill")
    ap.add_argument("--no-slow", action="store_true", help="skip the slow-decay prefill")
    ap.add_argument("--no-backward", action="store_true", help="skip the prefill gradients")
    ap.add_argument("--no-tokens", action="store_true", help="skip the several-token decode")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-calib", action="store_true", help="skip the GEMM and copy reference rates")
    ap.add_argument("--phase-stamps", nargs="?", const="prefill", default=None,
                    choices=["prefill", "ckpt", "reverse"],
                    help="with the profiling build (build.py --stamps): the phase split of the h32_t64k "
                         "prefill's main kernel (or of the b4_h32_t8k gradients' checkpoint pass or reverse "
                         "chain), from per-wave timestamps, instead of the bench line")
    ap.add_argument("--no-decomp", action="store_true",
                    help="skip timing the split prefill's pieces through the public calls (the roofline "
                         "then takes the whole call)")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--copy-calib", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB three times (the "
                         "known-size reference for HBM traffic counters) and exit")
    ap.add_argument("--summarize", nargs="+", metavar="CSV",
                    help="only summarise rocprofv3 kernel-trace / counter-collection CSV files and exit")
    args = ap.parse_args()
    if args.summarize:
        summarize_profiles(args.summarize)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: the KDA hot path here is single-GPU "
              f"(--gpus {args.gpus} requested)", file=sys.stderr)
        sys.exit(2)
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    if args.copy_calib:
        n = args.copy_calib << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calib_bytes": n, "launches": 3}), flush=True)
        return
    if args.phase_stamps:
        print(json.dumps({"phase_stamps": phase_stamps(dev, args.phase_stamps)}), flush=True)
        return
    kda.load()

    pf = bench_prefill(args, dev)
    B, H, T, D = pf["B"], pf["H"], pf["T"], pf["D"]
    ms = pf["median_ms"]
    tok_s = B * T / (ms * 1e-3)
    nbytes = prefill_bytes(B, H, T, D)
    gbs = nbytes / (ms * 1e-3) / 1e9
    fl_dense = prefill_flops(B, H, T, D)
    fl_tri = prefill_flops(B, H, T, D, triangle=True)
    dec = None if args.no_decomp else bench_decomposition(pf, args)
    if dec is not None and dec["T0"] == 0:
        names = ("head_walk", "zero_start_segments", "segment_merge", "corrected_heads")
        kern = {"head_walk": "kda_chunk_kernel<bf16,128,8,segment> (first chunks of segments 1..G-1)",
                "zero_start_segments": "kda_chunk_kernel<bf16,128,4,prefill> (every segment from zero)",
                "segment_merge": "kda_merge_kernel<128>",
                "corrected_heads": "kda_chunk_kernel<bf16,128,4,prefill> (first chunks from the start states)"}
    elif dec is not None:
        names = ("direct_part", "segment_transfer", "segment_merge", "segment_prefill")
        kern = {"direct_part": "kda_chunk_kernel<bf16,128,4,prefill> (first part, one workgroup per head)",
                "segment_transfer": "kda_chunk_kernel<bf16,128,8,segment>",
                "segment_merge": "kda_merge_kernel<128>",
                "segment_prefill": "kda_chunk_kernel<bf16,128,4,prefill>"}
    if dec is not None:
        dom = max(names, key=lambda n: dec[n]["ms"])
        r = dec[dom]
        # the dominant kernel's duration inside the timed steps (events around
        # its launch in each call), when that kernel is the call's main launch;
        # the standalone figure (its public call alone, back to back) is kept
        in_call = pf["main_ms"] if dom == "zero_start_segments" and len(pf["main_ms"]) == args.steps else []
        k_ms = sum(in_call) / len(in_call) if in_call else r["ms"]
        k_gbs = r["algorithmic_bytes"] / (k_ms * 1e-3) / 1e9
        counters_valid = kernel_sources_sha() == TRAFFIC["sources_sha"]
        traffic = TRAFFIC.get(dom) if counters_valid else None
        # counters are kept for the default pipeline's kernels only
        path_names = TRAFFIC_PATH if dec["T0"] == 0 else names
        path_counter = (sum(TRAFFIC[n] for n in path_names)
                        if counters_valid and all(n in TRAFFIC for n in path_names) else None)
        roofline = {"bound": "hbm", "achieved": k_gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                    "frac": k_gbs / PEAK_HBM_GBS, "traffic": traffic, "kernel": kern[dom],
                    "kernel_ms": k_ms,
                    "kernel_timing": ("mean over the timed steps, events around its launch in each call"
                                      if in_call else "median of its public call alone, back to back"),
                    "kernel_ms_median": statistics.median(in_call) if in_call else r["ms"],
                    "standalone_kernel_ms": r["ms"], "standalone_GBs": r["GBs"],
                    "standalone_frac": r["GBs"] / PEAK_HBM_GBS,
                    "algorithmic_bytes": r["algorithmic_bytes"],
                    "path_GBs": gbs, "path_frac": gbs / PEAK_HBM_GBS,
                    # whole call: its kernels' counter bytes against the single-pass
                    # algorithmic bytes
                    "path_traffic": {"counter_bytes": path_counter, "algorithmic_bytes": nbytes,
                                     "ratio": path_counter / nbytes if path_counter else None}}
    else:
        dec = None
        roofline = {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                    "frac": gbs / PEAK_HBM_GBS, "traffic": None, "kernel": "kda_chunk_kernel (single pass)",
                    "kernel_ms": ms, "algorithmic_bytes": nbytes}
    out = {
        "metric": METRIC,
        "value": tok_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": pf["wall_ms"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "kda_prefill_b1_h32_t65536_d128_bf16", "B": B, "H": H, "T": T,
                   "dk": D, "dv": D, "chunk": CH, "S0": "zero"},
        "roofline": roofline,
        "mfma": {"dense_tile_tflops": fl_dense / (ms * 1e-3) / 1e12,
                 "dense_tile_frac": fl_dense / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                 "triangle_tflops": fl_tri / (ms * 1e-3) / 1e12,
                 "triangle_frac": fl_tri / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                 "peak_tflops": PEAK_BF16_TFLOPS},
    }
    if dec is not None:
        out["prefill_kernels"] = dec
    if not args.no_snap:
        out["snapshots"] = bench_snapshots(pf, args)
        torch.cuda.empty_cache()
    if not args.no_slow:
        out["prefill_slow_decay"] = bench_prefill_slow_decay(args, dev)
        torch.cuda.empty_cache()
    if not args.no_batched:
        out["prefill_b4_h32_t8k"] = bench_prefill_batched(args, dev)
        torch.cuda.empty_cache()
    if not args.no_backward:
        out["backward_b4_h32_t8k"] = bench_backward(args, dev)
        torch.cuda.empty_cache()
    if not args.no_decode:
        out["decode"] = bench_decode(args, dev)
        torch.cuda.empty_cache()
    if not args.no_decode and not args.no_tokens:
        out["decode_tokens"] = bench_decode_tokens(args, dev)
        torch.cuda.empty_cache()
    if not args.no_kcp:
        out["kcp"] = bench_kcp(args, dev)
        torch.cuda.empty_cache()
    if not args.no_calib:
        out["calibration"] = bench_calibration(dev)
        torch.cuda.empty_cache()
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(pf, args.cpu_budget)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
