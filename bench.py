"""Benchmark: Gated DeltaNet prefill tokens/s (T=8192, bf16) + decode state-update HBM GB/s.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--skip-cpu-baseline]

One step = one pass of the prefill hot path over the T=8192 workload
(B=1, 16 key heads repeated to 32 value heads, Dk=Dv=128, bf16 q/k/v/a/b,
fp32 state/output): gating and the chunked rule as one gdn_chunk_fwd_gated
call (chunk preparation with the gating folded in, then the per-sequence
state recurrence). Inputs are resident in HBM before timing starts. About
half a second of untimed steps lets clocks settle, then W untimed warm-up
steps, then exactly K timed steps bracketed by torch.cuda.synchronize().
HIP events on the launch stream then time K more calls for the roofline
figure (warm: calls back to back), and up to 20 calls each preceded by a
1 GiB write outside the event pair (cold: the call's inputs are no longer
in the 256 MB memory-side cache).

The decode figures run one decode step of the 256-sequence workload (conv
update, gating, recurrent update of the 512 MiB fp32 state in place) and the
fused single-launch decode step, and report algorithmic bytes / event-timed
duration.

The CPU baseline times the fp64 oracle on the host on every workload (the
long prefill on its first 8192 tokens), with the CPU model, the cores this
process may use and the threads each timing used; it is a reported baseline,
not a target.

roofline.traffic is the HBM traffic of one call, from the rocprofv3
FETCH_SIZE / WRITE_SIZE summary committed under profiles/ (written by
bench_profile.py, calibrated on a plain 1 GiB copy); it is null when the
kernel sources differ from the ones the counters were taken on.

Prints one JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_HBM_GBPS = 8000.0        # MI355X HBM3E
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "hbm_traffic_prefill_t8k_decode_256seq.md")
CSRC = os.path.join(ROOT, "gated_deltanet_gdn_amd", "csrc")
# kernel sources each measured figure depends on
SOURCES = {"chunk": ["k_chunk.hip", "gdn_device.hpp"], "recurrent": ["k_recurrent.hip", "gdn_device.hpp"],
           "fused": ["k_recurrent.hip", "gdn_device.hpp"], "mtp": ["k_recurrent.hip", "gdn_device.hpp"]}


def source_hash(part):
    h = hashlib.sha256()
    for f in SOURCES[part]:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(part, key="bytes_per_call"):
    """A per-call counter figure (HBM bytes, or executed MFMA flops with key
    "mfma_flops_per_call") from the committed counter summary, or None if
    absent or stale."""
    try:
        with open(TRAFFIC_SUMMARY) as fh:
            for line in fh:
                if line.startswith("traffic_json:"):
                    rec = json.loads(line.split(":", 1)[1])[part]
                    return rec[key] if rec["source_hash"] == source_hash(part) else None
    except (OSError, KeyError, ValueError):
        pass
    return None


def chunk_flops_per_token_head(C=64, dk=128, dv=128, r=2):
    """Algorithmic flops of the chunked rule per token per value head.

    Grams Q K^T and K K^T (shared by r value heads), W = T K, U = T V and the
    intra-chunk P U product (C x C x D each per chunk), and the three state
    products W S, Q S, K^T U (Dk x Dv per token). Triangular products are
    counted dense; hi/lo precision passes are not counted.
    """
    return 2 * ((2 / r) * C * dk + C * (dk + 2 * dv) + 3 * dk * dv)


def chunk_bytes(T, nk, nv, dk=128, dv=128, n_seqs=1, in_bytes=2, o_bytes=4, state_in=False, gate_bytes=8):
    """Algorithmic HBM bytes of one chunk_fwd call (inputs read once, outputs written once); gate_bytes per
    (token, head): 8 for fp32 g and beta, 4 for bf16 a and b when the gating is folded in."""
    b = T * nk * dk * in_bytes * 2 + T * nv * dv * in_bytes      # q, k, v
    b += T * nv * gate_bytes                                     # g, beta (or a, b)
    b += T * nv * dv * o_bytes                                   # o
    b += n_seqs * nv * dk * dv * 4 * (2 if state_in else 1)      # final (+ initial) state
    return b


def recurrent_bytes(n, nk, nv, dk=128, dv=128, in_bytes=2):
    b = 2 * n * nv * dk * dv * 4                                 # state read + write
    b += n * nk * dk * in_bytes * 2 + n * nv * dv * in_bytes      # q, k, v
    b += n * nv * 4 * 2 + n * nv * dv * 4                        # g, beta, o
    return b


def fused_decode_bytes(n_tok, n_seqs, nk, nv, dk=128, dv=128, state_len=3, K=4, io_bytes=2):
    """Algorithmic bytes of one fused decode step: recurrent and conv states read and written once,
    x, a, b read, o written (fp32), conv weights read."""
    C = 2 * nk * dk + nv * dv
    return (2 * n_seqs * nv * dk * dv * 4 + 2 * n_seqs * C * state_len * io_bytes + n_tok * C * io_bytes
            + 2 * n_tok * nv * io_bytes + n_tok * nv * dv * 4 + C * K * 4)


def time_fused_decode(gdn, W, name, steps, warmup, stream, dev, tokens_per_seq=None):
    """Fused decode step (one launch): HIP events around every launch on its stream, and wall time."""
    import torch
    wl = W.WORKLOADS[name]
    n = wl.n_seqs
    if tokens_per_seq is None:
        x = {k: v.to(dev) for k, v in W.decode_inputs(wl).items()}
        cu, n_tok = None, n
    else:
        x = {k: v.to(dev) for k, v in W.decode_mtp_inputs(wl, [tokens_per_seq] * n).items()}
        cu, n_tok = x["cu_seqlens"], n * tokens_per_seq
    o = torch.empty((n_tok, wl.nv, wl.dv), device=dev, dtype=torch.float32)

    def fstep(ev=None):
        if ev is not None:
            ev[0].record(stream)
        gdn.gdn_decode_step_fused(x["x"], x["conv_state"], x["conv_w"], x["a"], x["b"], x["A_log"], x["dt_bias"],
                                  x["state"], wl.nk, cu_seqlens=cu, o=o, stream=stream)
        if ev is not None:
            ev[1].record(stream)

    for _ in range(warmup):
        fstep()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        fstep()
    torch.cuda.synchronize()
    step_ms = (time.perf_counter() - t0) * 1e3 / steps
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for i in range(steps):
        fstep(evs[i])
    torch.cuda.synchronize()
    k_ms = sum(a.elapsed_time(b) for a, b in evs) / steps
    nbytes = fused_decode_bytes(n_tok, n, wl.nk, wl.nv, state_len=wl.state_len)
    gbps = nbytes / (k_ms * 1e-3) / 1e9
    return dict(workload=f"{name}: {n} seqs x {tokens_per_seq or 1} token(s), {wl.nk}->{wl.nv} heads, "
                         f"conv update + gating + recurrent in one launch, states in place",
                step_ms=round(step_ms, 4), tokens_per_s=round(n_tok / (step_ms * 1e-3), 1),
                roofline=dict(bound="hbm", kernel="decode_fused_kernel", achieved=round(gbps, 1),
                              peak=PEAK_HBM_GBPS, unit="GB/s", frac=round(gbps / PEAK_HBM_GBPS, 4),
                              traffic=measured_traffic("fused" if tokens_per_seq is None else "mtp"),
                              avg_ms=round(k_ms, 4), algorithmic_bytes=nbytes))


def _timed(fn, reps, warmup, stream, graph=False):
    """Average ms per call of fn(): one pair of HIP events on its stream around reps back-to-back calls
    (warm-up calls first), so that a short kernel is not charged the per-event overhead. With graph=True
    the reps calls are captured once in a device graph and replayed between the events, so that a kernel
    shorter than its host-side launch is timed on the GPU, not at the launch rate."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    if graph:
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.stream(side), torch.cuda.graph(gr, stream=side):
            for _ in range(reps):
                fn(side)
        stream.wait_stream(side)
        torch.cuda.synchronize()
        gr.replay()                     # first replay outside the timed pair
        torch.cuda.synchronize()
        e0.record(stream)
        gr.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps
    e0.record(stream)
    for _ in range(reps):
        fn()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def _hbm_row(workload, ms, nbytes, kernel):
    gbps = nbytes / (ms * 1e-3) / 1e9
    return dict(workload=workload, kernel=kernel, bound="hbm", avg_ms=round(ms, 4), algorithmic_bytes=int(nbytes),
                achieved=round(gbps, 1), peak=PEAK_HBM_GBPS, unit="GB/s", frac=round(gbps / PEAK_HBM_GBPS, 4))


def time_rows(gdn, W, stream, dev, reps=5, warmup=3):
    """The neighbours of the core on their own workloads at full size: causal conv + SiLU, gating,
    the chunked rule and gated RMSNorm on the long prefill (T=262144, 16 -> 64 heads), conv update
    on the 256-sequence decode batch. HIP events around each launch; algorithmic bytes each."""
    import torch
    rows = {}
    wl = W.WORKLOADS["long_fused_t256k"]
    x = W.fused_inputs(wl, device=dev)
    T, C = x["x"].shape
    kd = wl.nk * wl.dk
    ms = _timed(lambda: gdn.gdn_causal_conv1d(x["x"], x["conv_w"], state_len=wl.state_len, stream=stream),
                reps, warmup, stream)
    rows["causal_conv1d"] = _hbm_row(f"long_fused_t256k: x [{T}, {C}] bf16 -> y, SiLU, conv state out", ms,
                                     2 * T * C * 2 + C * wl.conv_k * 4 + C * wl.state_len * 2, "causal_conv1d_kernel")
    y, _ = gdn.gdn_causal_conv1d(x["x"], x["conv_w"], state_len=wl.state_len, stream=stream)
    g = torch.empty((T, wl.nv), device=dev)
    beta = torch.empty_like(g)
    ms = _timed(lambda st=stream: gdn.gdn_gating(x["a"], x["b"], x["A_log"], x["dt_bias"], g=g, beta=beta,
                                                 stream=st),
                4 * reps, warmup, stream, graph=True)
    rows["gating"] = _hbm_row(f"long_fused_t256k: a, b [{T}, {wl.nv}] bf16 -> g, beta fp32", ms,
                              T * wl.nv * 12 + wl.nv * 8, "gating_kernel")
    q, k, v = y[:, :kd].view(T, wl.nk, wl.dk), y[:, kd:2 * kd].view(T, wl.nk, wl.dk), y[:, 2 * kd:].view(T, wl.nv, wl.dv)
    o = torch.empty((T, wl.nv, wl.dv), device=dev)
    st = torch.empty((1, wl.nv, wl.dk, wl.dv), device=dev)
    ws = torch.empty(gdn.gdn_chunk_fwd_workspace_size(T, 1, wl.nk, wl.nv), device=dev, dtype=torch.uint8)
    ms = _timed(lambda: gdn.gdn_chunk_fwd(q, k, v, g, beta, final_state=st, o=o, workspace=ws, stream=stream),
                max(2, reps // 2), 1, stream)
    r = wl.nv // wl.nk
    flops = chunk_flops_per_token_head(r=r) * T * wl.nv
    cb = chunk_bytes(T, wl.nk, wl.nv)
    tf = flops / (ms * 1e-3) / 1e12
    rows["chunk_fwd"] = dict(workload=f"long_fused_t256k core: T={T}, {wl.nk}->{wl.nv} heads, q/k/v views of the "
                                      f"conv output, zero initial state", kernel="chunk_prep + chunk_state",
                             bound="mfma", avg_ms=round(ms, 4), algorithmic_flops=flops, achieved=round(tf, 2),
                             peak=PEAK_BF16_TFLOPS, unit="TFLOP/s", frac=round(tf / PEAK_BF16_TFLOPS, 4),
                             algorithmic_bytes=cb, hbm_gbps_algorithmic=round(cb / (ms * 1e-3) / 1e9, 1),
                             tokens_per_s=round(T / (ms * 1e-3), 1))
    # the same core with the conv and the gating folded in (one call), against conv + gated chunk launches
    cso = torch.empty((1, C, wl.state_len), device=dev, dtype=x["x"].dtype)
    ms_f = _timed(lambda: gdn.gdn_prefill_fused(x["x"], x["conv_w"], x["a"], x["b"], x["A_log"], x["dt_bias"], wl.nk,
                                                wl.nv, state_len=wl.state_len, conv_state_out=cso, final_state=st, o=o,
                                                workspace=ws, stream=stream),
                  max(2, reps // 2), 1, stream)
    ms_s = _timed(lambda: (gdn.gdn_causal_conv1d(x["x"], x["conv_w"], state_len=wl.state_len, y=y, conv_state_out=cso,
                                                 stream=stream),
                           gdn.gdn_chunk_fwd_gated(q, k, v, x["a"], x["b"], x["A_log"], x["dt_bias"], final_state=st,
                                                   o=o, workspace=ws, stream=stream)),
                  max(2, reps // 2), 1, stream)
    fb = T * C * 2 + T * wl.nv * 2 * 2 + T * wl.nv * wl.dv * 4 + wl.nv * wl.dk * wl.dv * 4 + C * wl.state_len * 2
    tf = flops / (ms_f * 1e-3) / 1e12
    rows["prefill_fused"] = dict(
        workload=f"long_fused_t256k: x [{T}, {C}] bf16 through conv + SiLU, gating and the chunked rule in one call",
        kernel="chunk_prep (conv on q, k) + chunk_state (conv on v) + conv state out", bound="mfma",
        avg_ms=round(ms_f, 4), avg_ms_separate_conv_then_gated_chunk=round(ms_s, 4), algorithmic_flops=flops,
        achieved=round(tf, 2), peak=PEAK_BF16_TFLOPS, unit="TFLOP/s", frac=round(tf / PEAK_BF16_TFLOPS, 4),
        algorithmic_bytes=fb, hbm_gbps_algorithmic=round(fb / (ms_f * 1e-3) / 1e9, 1),
        tokens_per_s=round(T / (ms_f * 1e-3), 1))
    del ws, y, q, k, v, g, beta, cso
    # the varlen prefill batch: 8 packed sequences with nonzero initial states, gating folded in
    vw = W.WORKLOADS["varlen_prefill_8seq"]
    vx = {kk: (vv.to(dev) if isinstance(vv, torch.Tensor) else vv) for kk, vv in W.chunk_inputs(vw).items()}
    Tv, nseq = int(vx["cu_seqlens"][-1].item()), len(vx["lengths"])
    vo = torch.empty((Tv, vw.nv, vw.dv), device=dev)
    vst = torch.empty((nseq, vw.nv, vw.dk, vw.dv), device=dev)
    vws = torch.empty(gdn.gdn_chunk_fwd_workspace_size(Tv, nseq, vw.nk, vw.nv), device=dev, dtype=torch.uint8)
    ms = _timed(lambda: gdn.gdn_chunk_fwd_gated(vx["q"], vx["k"], vx["v"], vx["a"], vx["b"], vx["A_log"], vx["dt_bias"],
                                                cu_seqlens=vx["cu_seqlens"], initial_state=vx["S0"], final_state=vst,
                                                o=vo, workspace=vws, stream=stream),
                reps, warmup, stream)
    vflops = chunk_flops_per_token_head(r=vw.nv // vw.nk) * Tv * vw.nv
    vb = chunk_bytes(Tv, vw.nk, vw.nv, n_seqs=nseq, state_in=True, gate_bytes=4)
    tf = vflops / (ms * 1e-3) / 1e12
    rows["chunk_fwd_varlen"] = dict(
        workload=f"varlen_prefill_8seq: {nseq} sequences, lengths {[int(l) for l in vx['lengths']]} ({Tv} tokens), "
                 f"{vw.nk}->{vw.nv} heads, initial states, gating folded in",
        kernel="chunk_offsets + chunk_prep + chunk_state", bound="mfma", avg_ms=round(ms, 4),
        algorithmic_flops=vflops, achieved=round(tf, 2), peak=PEAK_BF16_TFLOPS, unit="TFLOP/s",
        frac=round(tf / PEAK_BF16_TFLOPS, 4), algorithmic_bytes=vb, hbm_gbps_algorithmic=round(vb / (ms * 1e-3) / 1e9, 1),
        tokens_per_s=round(Tv / (ms * 1e-3), 1))
    del vx, vo, vst, vws
    # one sequence with few heads (one GPU's share of the prefill workload under an 8-way head split): the
    # segment-parallel prefill (the library's choice for this shape) against the unsplit call
    sw = W.WORKLOADS["prefill_head_share_t8k"]
    sx = W.chunk_inputs(sw, device=dev)
    so = torch.empty((sw.T, sw.nv, sw.dv), device=dev)
    sst = torch.empty((1, sw.nv, sw.dk, sw.dv), device=dev)
    sws = torch.empty(gdn.gdn_chunk_fwd_workspace_size(sw.T, 1, sw.nk, sw.nv), device=dev, dtype=torch.uint8)
    seg_call = lambda: gdn.gdn_chunk_fwd_gated(sx["q"], sx["k"], sx["v"], sx["a"], sx["b"], sx["A_log"],
                                               sx["dt_bias"], final_state=sst, o=so, workspace=sws, stream=stream)
    ms = _timed(seg_call, 4 * reps, 4 * warmup, stream)
    old_seg = os.environ.get("GDN_SEGMENTS")
    os.environ["GDN_SEGMENTS"] = "1"
    try:
        ms_u = _timed(seg_call, 4 * reps, 4 * warmup, stream)
    finally:
        if old_seg is None:
            del os.environ["GDN_SEGMENTS"]
        else:
            os.environ["GDN_SEGMENTS"] = old_seg
    sflops = chunk_flops_per_token_head(r=sw.nv // sw.nk) * sw.T * sw.nv
    tf = sflops / (ms * 1e-3) / 1e12
    rows["chunk_fwd_segments"] = dict(
        workload=f"prefill_head_share_t8k: T={sw.T}, {sw.nk}->{sw.nv} heads, zero initial state, gating folded in "
                 f"(one GPU's share of prefill_chunk_t8k under an 8-way head split)",
        kernel="segment_table + chunk_prep + chunk_state (8 segments: local states and transitions) + "
               "segment_combine + chunk_state (rerun from the incoming states)", bound="mfma",
        avg_ms=round(ms, 4), avg_ms_unsplit=round(ms_u, 4), speedup_vs_unsplit=round(ms_u / ms, 3),
        algorithmic_flops=sflops, achieved=round(tf, 2), peak=PEAK_BF16_TFLOPS, unit="TFLOP/s",
        frac=round(tf / PEAK_BF16_TFLOPS, 4), tokens_per_s=round(sw.T / (ms * 1e-3), 1))
    del sx, so, sst, sws
    out = torch.empty((T, wl.nv, wl.dv), device=dev)
    ms = _timed(lambda: gdn.gdn_gated_rmsnorm(o, x["z"], x["norm_w"], eps=1e-6, y=out, stream=stream),
                reps, warmup, stream)
    rows["gated_rmsnorm"] = _hbm_row(f"long_fused_t256k: {T * wl.nv} rows of {wl.dv}, x fp32, z bf16 -> y fp32", ms,
                                     T * wl.nv * wl.dv * (4 + 2 + 4) + wl.dv * 4, "gated_rmsnorm_kernel")
    # the whole long pipeline: conv, gating, chunk rule and the gated RMSNorm epilogue in one call (the norm
    # inside the state kernel), and beside it the fused prefill followed by the norm launch
    ws2 = torch.empty(gdn.gdn_chunk_fwd_workspace_size(T, 1, wl.nk, wl.nv), device=dev, dtype=torch.uint8)
    ms = _timed(lambda: gdn.gdn_prefill_fused_norm(x["x"], x["conv_w"], x["a"], x["b"], x["A_log"], x["dt_bias"],
                                                   wl.nk, wl.nv, x["z"], x["norm_w"], eps=1e-6,
                                                   state_len=wl.state_len, final_state=st, y=out, workspace=ws2,
                                                   output_conv_state=False, stream=stream),
                max(2, reps // 2), 1, stream)
    ms2 = _timed(lambda: (gdn.gdn_prefill_fused(x["x"], x["conv_w"], x["a"], x["b"], x["A_log"], x["dt_bias"], wl.nk,
                                                wl.nv, state_len=wl.state_len, final_state=st, o=o, workspace=ws2,
                                                output_conv_state=False, stream=stream),
                          gdn.gdn_gated_rmsnorm(o, x["z"], x["norm_w"], eps=1e-6, y=out, stream=stream)),
                 max(2, reps // 2), 1, stream)
    rows["long_prefill_pipeline"] = dict(
        workload=f"long_fused_t256k: conv + SiLU, gating, chunk rule and gated RMSNorm (one call), T={T}",
        kernel="gdn_prefill_fused_norm", avg_ms=round(ms, 4), tokens_per_s=round(T / (ms * 1e-3), 1),
        avg_ms_two_launches=round(ms2, 4), speedup_vs_two_launches=round(ms2 / ms, 3))
    del ws2
    del x, o, out, st
    dw = W.WORKLOADS["decode_256seq"]
    dx = {kk: vv.to(dev) for kk, vv in W.decode_inputs(dw).items()}
    yd = torch.empty_like(dx["x"])
    n, Cd = dx["x"].shape
    ms = _timed(lambda st=stream: gdn.gdn_causal_conv1d_update(dx["x"], dx["conv_state"], dx["conv_w"], y=yd,
                                                                stream=st),
                20 * reps, warmup, stream, graph=True)
    rows["causal_conv1d_update"] = _hbm_row(f"decode_256seq: x [{n}, {Cd}] bf16, conv state [{n}, {Cd}, 3] in place",
                                            ms, n * Cd * (2 + 2 * 3 * 2 + 2) + Cd * 4 * 4, "conv_update_kernel")
    torch.cuda.empty_cache()
    return rows


def cpu_info():
    """CPU model, cores available to this process, and the thread cap: the cores this
    process may run on, capped by OMP_NUM_THREADS when it is set (the machine's CPU share)."""
    model = None
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    avail = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    omp = int(os.environ.get("OMP_NUM_THREADS", "0") or 0)
    return model, avail, (min(avail, omp) if omp > 0 else avail)


def _repeat(fn, min_s):
    """Run fn() until at least min_s seconds of wall time have passed; returns (reps, seconds)."""
    reps, t0 = 0, time.perf_counter()
    while True:
        fn()
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= min_s:
            return reps, dt


def cpu_baseline(W, cap, min_s=2.0):
    """The fp64 oracle on the host cores, for every workload (a reported baseline, not the target).

    Threads per workload = the thread cap (cores of this process, OMP_NUM_THREADS when set) capped at
    the number of independent (sequence, value head) units. Each timing repeats its sample until
    min_s seconds have passed. The long prefill is timed on its first 8192 tokens (all 64 heads, the
    whole conv + gating + chunk + gated RMSNorm pipeline), since the whole workload would take minutes.
    """
    import numpy as np
    import oracle
    f = lambda t: t.detach().to("cpu").double().numpy()
    out = {}

    def chunk_rate(name, sample=None):
        wl = W.WORKLOADS[name]
        x = W.chunk_inputs(wl)
        cu = x["cu_seqlens"].numpy()
        n_units = len(x["lengths"]) * wl.nv
        th = max(1, min(cap, n_units))
        a, b, A, dt = f(x["a"]), f(x["b"]), f(x["A_log"]), f(x["dt_bias"])
        q, k, v = f(x["q"]), f(x["k"]), f(x["v"])
        S0 = None if x["S0"] is None else f(x["S0"])
        T = q.shape[0]

        def run():
            g, beta = oracle.gating(a, b, A, dt)
            oracle.delta_rule(q, k, v, g, beta, cu_seqlens=cu, initial_state=S0, threads=th)
        reps, sec = _repeat(run, min_s)
        return dict(value=round(reps * T / sec, 1), unit="tokens/s", threads=th,
                    sample=f"whole workload ({T} tokens, {wl.nv} value heads), gating + token recurrence, "
                           f"{reps} runs in {sec:.2f} s")

    out["tiny_chunk_f32"] = chunk_rate("tiny_chunk_f32")
    out["prefill_chunk_t8k"] = chunk_rate("prefill_chunk_t8k")
    out["varlen_prefill_8seq"] = chunk_rate("varlen_prefill_8seq")

    wl = W.WORKLOADS["decode_256seq"]
    x = W.decode_inputs(wl)
    n, kd = wl.n_seqs, wl.nk * wl.dk
    th = max(1, min(cap, n * wl.nv))
    xx, cs, cw, a, b, A, dt, st = (f(x[kk]) for kk in ("x", "conv_state", "conv_w", "a", "b", "A_log",
                                                       "dt_bias", "state"))

    def dec():
        y, _ = oracle.causal_conv1d_update(xx, cs, cw)
        g, beta = oracle.gating(a, b, A, dt)
        oracle.delta_rule(y[:, :kd].reshape(n, wl.nk, wl.dk), y[:, kd:2 * kd].reshape(n, wl.nk, wl.dk),
                          y[:, 2 * kd:].reshape(n, wl.nv, wl.dv), g, beta,
                          cu_seqlens=np.arange(n + 1), initial_state=st, threads=th)
    reps, sec = _repeat(dec, min_s)
    out["decode_256seq"] = dict(value=round(reps * n * wl.nv / sec, 1), unit="state updates/s", threads=th,
                                sample=f"whole decode step (conv update, gating, {n} x {wl.nv} state updates), "
                                       f"{reps} runs in {sec:.2f} s")

    wl = W.WORKLOADS["long_fused_t256k"]
    Ts = 8192
    x = W.fused_inputs(wl, T=Ts)
    th = max(1, min(cap, wl.nv))
    xx, cw, a, b, A, dt, z, nw = (f(x[kk]) for kk in ("x", "conv_w", "a", "b", "A_log", "dt_bias", "z",
                                                      "norm_w"))
    kd = wl.nk * wl.dk

    def longp():
        y, _ = oracle.causal_conv1d(xx, cw, state_len=wl.state_len)
        g, beta = oracle.gating(a, b, A, dt)
        o, _ = oracle.delta_rule(y[:, :kd].reshape(Ts, wl.nk, wl.dk), y[:, kd:2 * kd].reshape(Ts, wl.nk, wl.dk),
                                 y[:, 2 * kd:].reshape(Ts, wl.nv, wl.dv), g, beta, threads=th)
        oracle.gated_rmsnorm(o, z, nw)
    reps, sec = _repeat(longp, min_s)
    out["long_fused_t256k"] = dict(value=round(reps * Ts / sec, 1), unit="tokens/s", threads=th,
                                   sample=f"first {Ts} of {wl.T} tokens, all {wl.nv} value heads, conv + SiLU, "
                                          f"gating, token recurrence and gated RMSNorm, {reps} runs in {sec:.2f} s")
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--skip-cpu-baseline", action="store_true")
    ap.add_argument("--settle-s", type=float, default=0.5,
                    help="seconds of untimed steps before the warm-up steps, so that clocks settle")
    ap.add_argument("--skip-decode", action="store_true")
    ap.add_argument("--skip-mtp", action="store_true", help="skip the 1 + 3 token fused decode measurement")
    ap.add_argument("--skip-rows", action="store_true", help="skip the per-row kernels on their own workloads")
    ap.add_argument("--rows-only", action="store_true",
                    help="only the per-row kernels (one JSON line with them; used for their kernel trace)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="finish with one plain 1 GiB device copy (counter calibration runs only)")
    ap.add_argument("--mtp-only", action="store_true",
                    help="only the 1 + 3 token fused decode step (one JSON line; used for its counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the GDN core shards by head or sequence with no "
              "collective, so there is no multi-GPU step to time (run with --gpus 1).", file=sys.stderr)
        sys.exit(2)

    import torch
    import gated_deltanet_gdn_amd as gdn
    import workloads as W

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    if args.rows_only:
        print(json.dumps({"rows": time_rows(gdn, W, stream, dev)}), flush=True)
        return
    if args.mtp_only:
        mtp = time_fused_decode(gdn, W, "decode_mtp_256x4", args.steps, max(args.warmup, 50), stream, dev,
                                tokens_per_seq=W.WORKLOADS["decode_mtp_256x4"].extra["tokens_per_seq"])
        if args.calibrate_copy:
            src = torch.ones(1 << 28, device=dev, dtype=torch.float32)
            torch.empty_like(src).copy_(src)
            torch.cuda.synchronize()
        print(json.dumps({"decode_mtp_fused": mtp}), flush=True)
        return

    # ---------------------------------------------------------------- prefill step
    wl = W.WORKLOADS["prefill_chunk_t8k"]
    x = W.chunk_inputs(wl)
    d = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in x.items()}
    T = wl.T
    g = torch.empty((T, wl.nv), device=dev, dtype=torch.float32)
    beta = torch.empty_like(g)
    o = torch.empty((T, wl.nv, wl.dv), device=dev, dtype=torch.float32)
    st = torch.empty((1, wl.nv, wl.dk, wl.dv), device=dev, dtype=torch.float32)
    ws = torch.empty(gdn.gdn_chunk_fwd_workspace_size(T, 1, wl.nk, wl.nv), device=dev, dtype=torch.uint8)

    # one step = gating + the chunked rule, as one call with the gating folded into the chunk preparation
    # (bit for bit the same as gdn_gating followed by gdn_chunk_fwd, which is timed below for reference)
    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        gdn.gdn_chunk_fwd_gated(d["q"], d["k"], d["v"], d["a"], d["b"], d["A_log"], d["dt_bias"], final_state=st,
                                o=o, workspace=ws, stream=stream)
        if ev is not None:
            ev[1].record(stream)

    def step_separate():
        gdn.gdn_gating(d["a"], d["b"], d["A_log"], d["dt_bias"], g=g, beta=beta, stream=stream)
        gdn.gdn_chunk_fwd(d["q"], d["k"], d["v"], g, beta, final_state=st, o=o, workspace=ws, stream=stream)

    # clocks settle under load first (untimed), then W warm-up steps, then the timed region:
    # K steps between synchronisations, nothing else in the stream
    settle, t_settle = 0, time.perf_counter()
    while time.perf_counter() - t_settle < args.settle_s:
        for _ in range(10):
            step()
        torch.cuda.synchronize()
        settle += 10
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    ms_step = elapsed * 1e3 / args.steps
    # the kernel time: HIP events on the launch stream around every call of K more steps (the event
    # records add a few microseconds of stream gaps, so they stay out of the timed region above)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    chunk_ms = sum(a.elapsed_time(b) for a, b in evs) / args.steps
    # cold-cache figure: a 1 GiB write between calls, outside the event pair, evicts the call's inputs
    # and workspace from the 256 MB memory-side cache (the warm figure above runs calls back to back)
    flush = torch.empty(1 << 28, device=dev, dtype=torch.float32)
    n_cold = min(args.steps, 20)
    cevs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n_cold)]
    for i in range(n_cold):
        flush.fill_(float(i))
        step(cevs[i])
    torch.cuda.synchronize()
    cold_ms = sum(a.elapsed_time(b) for a, b in cevs) / n_cold
    del flush

    # the same step as two calls (gating, then the chunk rule), for reference
    for _ in range(max(10, args.warmup // 4)):
        step_separate()
    torch.cuda.synchronize()
    t_sep = time.perf_counter()
    for _ in range(args.steps):
        step_separate()
    torch.cuda.synchronize()
    ms_separate = (time.perf_counter() - t_sep) * 1e3 / args.steps

    r = wl.nv // wl.nk
    flops = chunk_flops_per_token_head(r=r) * T * wl.nv
    cbytes = chunk_bytes(T, wl.nk, wl.nv, gate_bytes=4)
    achieved_tflops = flops / (chunk_ms * 1e-3) / 1e12
    roofline = dict(bound="mfma", kernel="gdn_chunk_fwd_gated (chunk_prep with the gating + chunk_state launches)",
                    achieved=round(achieved_tflops, 2), peak=PEAK_BF16_TFLOPS, unit="TFLOP/s",
                    frac=round(achieved_tflops / PEAK_BF16_TFLOPS, 4), traffic=measured_traffic("chunk"),
                    avg_ms=round(chunk_ms, 4), cold_avg_ms=round(cold_ms, 4),
                    cold_frac=round(flops / (cold_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                    algorithmic_flops=flops, algorithmic_bytes=cbytes,
                    hbm_gbps_algorithmic=round(cbytes / (chunk_ms * 1e-3) / 1e9, 1))
    # MFMA work as the hardware counted it (hi/lo precision passes included):
    # SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512 per call, from the same counter summary
    executed = measured_traffic("chunk", "mfma_flops_per_call")
    roofline["mfma_executed_flops"] = executed
    roofline["mfma_counter_frac"] = (round(executed / (chunk_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)
                                     if executed else None)

    # ---------------------------------------------------------------- decode step
    decode = None
    if not args.skip_decode:
        dw = W.WORKLOADS["decode_256seq"]
        dx = {k: v.to(dev) for k, v in W.decode_inputs(dw).items()}
        n = dw.n_seqs
        kd = dw.nk * dw.dk
        y = torch.empty_like(dx["x"])
        dg = torch.empty((n, dw.nv), device=dev, dtype=torch.float32)
        db = torch.empty_like(dg)
        do = torch.empty((n, dw.nv, dw.dv), device=dev, dtype=torch.float32)
        qv = y[:, :kd].view(n, dw.nk, dw.dk)
        kv = y[:, kd:2 * kd].view(n, dw.nk, dw.dk)
        vv = y[:, 2 * kd:].view(n, dw.nv, dw.dv)

        def dstep(ev=None):
            gdn.gdn_causal_conv1d_update(dx["x"], dx["conv_state"], dx["conv_w"], y=y, stream=stream)
            gdn.gdn_gating(dx["a"], dx["b"], dx["A_log"], dx["dt_bias"], g=dg, beta=db, stream=stream)
            if ev is not None:
                ev[0].record(stream)
            gdn.gdn_recurrent_fwd(qv, kv, vv, dg, db, dx["state"], o=do, stream=stream)
            if ev is not None:
                ev[1].record(stream)

        for _ in range(max(args.warmup, 50)):   # steady clocks, as for the fused decode legs below
            dstep()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            dstep()
        torch.cuda.synchronize()
        dstep_ms = (time.perf_counter() - t0) * 1e3 / args.steps
        devs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                for _ in range(args.steps)]
        for i in range(args.steps):
            dstep(devs[i])
        torch.cuda.synchronize()
        rec_ms = sum(a.elapsed_time(b) for a, b in devs) / args.steps
        rbytes = recurrent_bytes(n, dw.nk, dw.nv)
        gbps = rbytes / (rec_ms * 1e-3) / 1e9
        decode = dict(workload="decode_256seq: 256 seqs x 1 token, 16->32 heads, 512 MiB fp32 state in place",
                      step_ms=round(dstep_ms, 4),
                      roofline=dict(bound="hbm", kernel="recurrent_kernel", achieved=round(gbps, 1),
                                    peak=PEAK_HBM_GBPS, unit="GB/s", frac=round(gbps / PEAK_HBM_GBPS, 4),
                                    traffic=measured_traffic("recurrent"), avg_ms=round(rec_ms, 4),
                                    algorithmic_bytes=rbytes))

    decode_fused = decode_mtp = None
    if not args.skip_decode:
        # (the decode steps are ~0.2 ms each: at least 50 untimed steps bring the clocks to their steady
        # state whatever --warmup says, as the settle loop does for the chunk call)
        dwarm = max(args.warmup, 50)
        decode_fused = time_fused_decode(gdn, W, "decode_256seq", args.steps, dwarm, stream, dev)
        decode_fused["separate_launches_step_ms"] = decode["step_ms"]
        if not args.skip_mtp:
            decode_mtp = time_fused_decode(gdn, W, "decode_mtp_256x4", args.steps, dwarm, stream, dev,
                                           tokens_per_seq=W.WORKLOADS["decode_mtp_256x4"].extra["tokens_per_seq"])

    rows = None if args.skip_rows else time_rows(gdn, W, stream, dev)

    if args.calibrate_copy:   # known-size reference for the FETCH_SIZE / WRITE_SIZE counters
        src = torch.ones(1 << 28, device=dev, dtype=torch.float32)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    cpu = None
    if not args.skip_cpu_baseline:
        model, avail, cap = cpu_info()
        per = cpu_baseline(W, cap)
        head = per["prefill_chunk_t8k"]
        cpu = dict(value=head["value"], unit=head["unit"], cores=head["threads"], kind="oracle",
                   sample=head["sample"], cpu_model=model, cores_available=avail, thread_cap=cap,
                   thread_policy="min(cores of this process capped by OMP_NUM_THREADS, independent units)",
                   per_config=per)

    out = {
        "metric": "GDN prefill tokens/s (T=8K, bf16) + decode state-update HBM GB/s",
        "value": round(T / (ms_step * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_steps": settle,
        "ms_per_step": round(ms_step, 4),
        "ms_per_step_separate_gating": round(ms_separate, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; q,k,v,a,b ~ N(0,1) bf16, A_log = log U[1,16], dt_bias ~ N(0,0.1))",
        "config": {"workload": "prefill_chunk_t8k: B=1, T=8192, 16 key heads -> 32 value heads, Dk=Dv=128, "
                               "chunk 64, zero initial state, gating + chunked rule, fp32 output + final state",
                   "global_batch": 1, "seq_len": T, "parallelism": "single GPU"},
        "roofline": roofline,
        "decode": decode,
        "decode_fused": decode_fused,
        "decode_mtp_fused": decode_mtp,
        "rows": rows,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
