"""GPU tests of the segment-parallel chunk prefill (one sequence, at most eight value heads).

One sequence whose 16-column slices are few (nv * 8 <= 64) is split into P
segments of whole chunks: a first pass runs every segment from a zero state
and from the identity with v = 0, a small kernel chains the incoming states
S_in[p + 1] = M_p S_in[p] + D_p, and a second pass reruns every segment from
its incoming state. The segment count depends on the shape only
(eight segments of at least four chunks up to four value heads, four from
five to eight heads for sequences of at least 256 chunks); GDN_SEGMENTS=<P>
forces one (1 = unsplit). Its rounding differs from the unsplit call, so
each case is compared with the fp64 oracle at the bf16 bar and with the
unsplit call at the sum of the two bars. The fused prefill (conv inside the
chunk kernels) splits the same way and must equal its separate launches bit
for bit. Cases: one GPU's share of the
prefill workload under an 8-way head split (T = 8192, 2 -> 4 heads), eight
value heads over 16384 tokens, ragged
lengths, initial states, cu_seqlens given (same bits as without), bf16
output, g and beta given, a slow decay in which the incoming states carry
across segments, and segments of a single chunk. Each test prints its case
before touching the GPU.
"""
import contextlib
import os

import numpy as np
import pytest
import torch

import gated_deltanet_gdn_amd as gdn
import oracle
import test_gpu_prefill_fused as PF
import workloads as W
from gpu_common import TOL, assert_close, dev, f64

pytestmark = pytest.mark.gpu
THREADS = min(16, os.cpu_count() or 1)


def _say(*a):
    print("[case]", *a, flush=True)


@contextlib.contextmanager
def _segments(p):
    old = os.environ.get("GDN_SEGMENTS")
    if p is None:
        os.environ.pop("GDN_SEGMENTS", None)
    else:
        os.environ["GDN_SEGMENTS"] = str(p)
    try:
        yield
    finally:
        if old is None:
            os.environ.pop("GDN_SEGMENTS", None)
        else:
            os.environ["GDN_SEGMENTS"] = old


def _inputs(T, nk, nv, seed, s0_std):
    wl = W.Workload("t", seed, "chunk", "bf16", nk=nk, nv=nv, s0_std=s0_std)
    return W.chunk_inputs(wl, lengths=[T])


def _dev(x):
    return {k: (v.to(dev()) if isinstance(v, torch.Tensor) else v) for k, v in x.items()}


def _gated(d, with_s0, o_dtype=torch.float32, with_cu=False):
    return gdn.gdn_chunk_fwd_gated(d["q"], d["k"], d["v"], d["a"], d["b"], d["A_log"], d["dt_bias"],
                                   cu_seqlens=d["cu_seqlens"] if with_cu else None,
                                   initial_state=d["S0"] if with_s0 else None, o_dtype=o_dtype)


def _oracle(x, with_s0):
    g_ref, b_ref = oracle.gating(f64(x["a"]), f64(x["b"]), f64(x["A_log"]), f64(x["dt_bias"]))
    return oracle.delta_rule(f64(x["q"]), f64(x["k"]), f64(x["v"]), g_ref, b_ref,
                             cu_seqlens=x["cu_seqlens"].numpy(),
                             initial_state=f64(x["S0"]) if with_s0 else None, threads=THREADS)


def _check(x, with_s0, P, what, o_dtype=torch.float32):
    d = _dev(x)
    with _segments(P):
        o_s, s_s = _gated(d, with_s0, o_dtype)
    with _segments(1):
        o_u, s_u = _gated(d, with_s0, o_dtype)
    torch.cuda.synchronize()
    o_ref, s_ref = _oracle(x, with_s0)
    rms = np.sqrt(np.mean(o_ref ** 2))
    if o_dtype == torch.float32:
        assert_close(o_s, o_ref, TOL["bf16"], f"{what} segmented o")
        assert_close(o_s, f64(o_u), 2 * TOL["bf16"], f"{what} segmented vs unsplit o")
    else:   # one rounding of the output on top of each bar
        assert np.all(np.abs(f64(o_s) - o_ref) <= TOL["bf16"] * rms + np.abs(o_ref) * 2.0 ** -8 + 1e-30)
        assert np.all(np.abs(f64(o_s) - f64(o_u)) <= 2 * TOL["bf16"] * rms + np.abs(o_ref) * 2.0 ** -7 + 1e-30)
    assert_close(s_s, s_ref, TOL["bf16"], f"{what} segmented final state")
    assert_close(s_s, f64(s_u), 2 * TOL["bf16"], f"{what} segmented vs unsplit final state")
    return o_s, s_s


def test_segments_head_share_of_prefill():
    """prefill_head_share_t8k (T = 8192 with 2 -> 4 heads, one GPU's share of the prefill workload under an
    8-way head split) at the default segment count (8)."""
    wl = W.WORKLOADS["prefill_head_share_t8k"]
    _say("segments:", wl.name, "default count")
    _check(W.chunk_inputs(wl), False, None, "head share")


CASES = [
    dict(name="ragged_s0_r2_P3", T=5000, nk=1, nv=2, s0=True, P=3),
    dict(name="r1_P16_two_chunks_each", T=2000, nk=1, nv=1, s0=True, P=16),
    dict(name="r4_P5_bf16_out", T=1500, nk=1, nv=4, s0=True, P=5, o_dtype="bf16"),
    dict(name="two_chunks_P2", T=65, nk=1, nv=2, s0=True, P=2),
    dict(name="default_count_nv2", T=3000, nk=2, nv=2, s0=False, P=None),
]


@pytest.mark.parametrize("ci", range(len(CASES)), ids=[c["name"] for c in CASES])
def test_segments_cases(ci):
    c = CASES[ci]
    _say("segments", c)
    x = _inputs(c["T"], c["nk"], c["nv"], 20 + ci, 0.3 if c["s0"] else 0.0)
    o_dtype = torch.bfloat16 if c.get("o_dtype") == "bf16" else torch.float32
    _check(x, c["s0"], c["P"], c["name"], o_dtype)


def test_segments_eight_heads_long():
    """Eight value heads (2 -> 8) and T = 16384: four segments by default (sequences of 256 chunks or more)."""
    _say("segments: T=16384, 2->8 heads, default count")
    x = _inputs(16384, 2, 8, 61, 0.3)
    _check(x, True, None, "eight heads")


def test_segments_slow_decay():
    """A_log = 0 and a ~ N(-6, 1): g ~ -0.0025 per token, so a segment's incoming state still weighs about
    e^-1 at its end and errors in the transitions would show."""
    _say("segments: slow decay, T=4096, 1->2 heads, P=8")
    x = _inputs(4096, 1, 2, 31, 0.3)
    x["A_log"] = torch.zeros_like(x["A_log"])
    x["a"] = (x["a"].float() - 6.0).to(torch.bfloat16)
    _check(x, True, 8, "slow decay")


def test_segments_cu_seqlens_same_bits():
    """One sequence given with cu_seqlens = [0, T] runs the same segments as without: equal bits."""
    _say("segments: cu_seqlens given, T=3000, 1->2 heads")
    x = _inputs(3000, 1, 2, 41, 0.3)
    d = _dev(x)
    with _segments(None):
        o_a, s_a = _gated(d, True, with_cu=False)
        o_b, s_b = _gated(d, True, with_cu=True)
    torch.cuda.synchronize()
    assert torch.equal(o_a, o_b) and torch.equal(s_a, s_b)


def test_segments_sequence_shorter_than_the_buffer():
    """cu_seqlens = [0, 2300] over buffers of 4096 tokens: the segments are cut from the sequence's own length
    (those past its end are empty), and the tokens it holds match the oracle and the unsplit call."""
    _say("segments: one sequence of 2300 tokens in buffers of 4096, 1->2 heads, P=8")
    x = _inputs(4096, 1, 2, 43, 0.3)
    Ts = 2300
    d = _dev(x)
    cu = torch.tensor([0, Ts], dtype=torch.int32, device=dev())
    call = lambda: gdn.gdn_chunk_fwd_gated(d["q"], d["k"], d["v"], d["a"], d["b"], d["A_log"], d["dt_bias"],
                                           cu_seqlens=cu, initial_state=d["S0"])
    with _segments(8):
        o_s, s_s = call()
    with _segments(1):
        o_u, s_u = call()
    torch.cuda.synchronize()
    xs = {k: (v[:Ts] if isinstance(v, torch.Tensor) and k in ("q", "k", "v", "a", "b") else v) for k, v in x.items()}
    xs["cu_seqlens"] = torch.tensor([0, Ts], dtype=torch.int32)
    o_ref, s_ref = _oracle(xs, True)
    assert_close(o_s[:Ts], o_ref, TOL["bf16"], "short sequence: segmented o")
    assert_close(s_s, s_ref, TOL["bf16"], "short sequence: segmented final state")
    assert_close(o_s[:Ts], f64(o_u[:Ts]), 2 * TOL["bf16"], "short sequence: segmented vs unsplit o")
    assert_close(s_s, f64(s_u), 2 * TOL["bf16"], "short sequence: segmented vs unsplit final state")


def test_segments_given_g_beta():
    """gdn_chunk_fwd (g and beta given), segmented, against the oracle."""
    _say("segments: g and beta given, T=2500, 2->4 heads, P=6")
    x = _inputs(2500, 2, 4, 51, 0.3)
    d = _dev(x)
    g, beta = gdn.gdn_gating(d["a"], d["b"], d["A_log"], d["dt_bias"])
    with _segments(6):
        o, st = gdn.gdn_chunk_fwd(d["q"], d["k"], d["v"], g, beta, initial_state=d["S0"])
    torch.cuda.synchronize()
    o_ref, s_ref = oracle.delta_rule(f64(x["q"]), f64(x["k"]), f64(x["v"]), f64(g), f64(beta),
                                     cu_seqlens=x["cu_seqlens"].numpy(), initial_state=f64(x["S0"]),
                                     threads=THREADS)
    assert_close(o, o_ref, TOL["bf16"], "given g, beta: o")
    assert_close(st, s_ref, TOL["bf16"], "given g, beta: final state")


FUSED_CASES = [
    dict(name="fused_ragged_bias_history_P4", T=5000, nk=1, nv=2, bias=True, conv_state=True, s0=True, P=4),
    dict(name="fused_history5_P3_bf16_out", T=1000, nk=2, nv=4, conv_state=True, state_len=5, o_dtype="bf16", P=3),
    dict(name="fused_eight_heads_default_count", T=16384, nk=2, nv=8, conv_state=True, P=None),
    dict(name="fused_strided_x_f32_gating_P8", T=3000, nk=1, nv=4, bias=True, s0=True, ab="f32", pad=64, P=8),
]


@pytest.mark.parametrize("ci", range(len(FUSED_CASES)), ids=[c["name"] for c in FUSED_CASES])
def test_segments_fused_prefill(ci):
    """gdn_prefill_fused split into segments: the conv inputs before a segment's first token are x rows (the
    conv state only before the first segment), and a transition run stages zero values. It must equal the
    separate conv, gating and (equally split) chunk launches bit for bit, write the same conv state as the
    unsplit call, and match the unsplit call's o and final state at the sum of the two bars."""
    c = FUSED_CASES[ci]
    _say("segments, fused prefill", c)
    d = PF._inputs(c, 80 + ci)
    with _segments(c["P"]):
        o_s, st_s, cs_s = PF._separate(d, c["nk"], c["nv"])
        o_f, st_f, cs_f = PF._fused(d, c["nk"], c["nv"])
    with _segments(1):
        o_u, st_u, cs_u = PF._fused(d, c["nk"], c["nv"])
    torch.cuda.synchronize()
    PF._same(o_f, o_s, "o")
    PF._same(st_f, st_s, "final state")
    PF._same(cs_f, cs_s, "conv state out")
    assert torch.equal(cs_f, cs_u), "conv state out differs from the unsplit call"
    if d["o_dtype"] == torch.float32:
        assert_close(o_f, f64(o_u), 2 * TOL["bf16"], f"{c['name']} segmented vs unsplit o")
    else:
        ref = f64(o_u)
        rms = np.sqrt(np.mean(ref ** 2))
        assert np.all(np.abs(f64(o_f) - ref) <= 2 * TOL["bf16"] * rms + np.abs(ref) * 2.0 ** -7 + 1e-30)
    assert_close(st_f, f64(st_u), 2 * TOL["bf16"], f"{c['name']} segmented vs unsplit final state")
