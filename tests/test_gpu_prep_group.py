"""GPU tests of the grouped chunk preparation.

With enough (chunk, key head) items the preparation runs one workgroup per
(chunk, key head), forming the K and Q tiles (and their conv), the Grams and
the norms once and then each value head's decays, inverse and tiles in turn;
otherwise one workgroup per (chunk, value head). The per-element arithmetic
is the same, so both must give the same bits: these tests force each with
GDN_PREP_GROUP=0|1 and compare o, the final state and (for the fused
prefill) the conv state, over varlen batches with head groupings r = 1, 2
and 4, fp32 and bf16 inputs, bf16 gating inputs folded in, the conv inside
the chunk kernels, and the full varlen workload. Each test prints its case
before touching the GPU.
"""
import contextlib
import os

import pytest
import torch

import gated_deltanet_gdn_amd as gdn
import test_gpu_prefill_fused as PF
import workloads as W
from gpu_common import dev

pytestmark = pytest.mark.gpu


def _say(*a):
    print("[case]", *a, flush=True)


@contextlib.contextmanager
def _group(v):
    old = os.environ.get("GDN_PREP_GROUP")
    os.environ["GDN_PREP_GROUP"] = v
    try:
        yield
    finally:
        if old is None:
            del os.environ["GDN_PREP_GROUP"]
        else:
            os.environ["GDN_PREP_GROUP"] = old


def _both(fn):
    with _group("0"):
        a = fn()
    with _group("1"):
        b = fn()
    torch.cuda.synchronize()
    return a, b


def _same(a, b, what):
    diff = (a.double() - b.double()).abs().max().item() if a.numel() else 0.0
    print(f"[exact] {what}: max |grouped - per head| = {diff:.3e}", flush=True)
    assert torch.equal(a, b), f"{what}: the grouped preparation differs"


CASES = [
    dict(name="varlen_r2_bf16", lengths=[1, 63, 64, 65, 130, 0, 7], nk=2, nv=4, dtype="bf16"),
    dict(name="one_sequence_r4_bf16", lengths=[300], nk=1, nv=4, dtype="bf16"),
    dict(name="r1_bf16", lengths=[100, 37], nk=2, nv=2, dtype="bf16"),
    dict(name="varlen_r2_f32", lengths=[5, 70, 129], nk=1, nv=2, dtype="f32"),
]


@pytest.mark.parametrize("ci", range(len(CASES)), ids=[c["name"] for c in CASES])
def test_grouped_prep_equals_per_head(ci):
    c = CASES[ci]
    _say("prep grouping", c)
    wl = W.Workload("t", 900 + ci, "chunk", c["dtype"], nk=c["nk"], nv=c["nv"], s0_std=0.3)
    x = W.chunk_inputs(wl, lengths=c["lengths"])
    d = {k: (v.to(dev()) if isinstance(v, torch.Tensor) else v) for k, v in x.items()}
    run = lambda: gdn.gdn_chunk_fwd_gated(d["q"], d["k"], d["v"], d["a"], d["b"], d["A_log"], d["dt_bias"],
                                          cu_seqlens=d["cu_seqlens"], initial_state=d["S0"])
    (o0, s0), (o1, s1) = _both(run)
    _same(o1, o0, "o")
    _same(s1, s0, "final state")


@pytest.mark.parametrize("ci", range(len(PF.CASES)), ids=[c["name"] for c in PF.CASES])
def test_grouped_prep_fused_prefill(ci):
    c = PF.CASES[ci]
    _say("prep grouping, fused prefill", c)
    d = PF._inputs(c, 950 + ci)
    (o0, s0, cs0), (o1, s1, cs1) = _both(lambda: PF._fused(d, c["nk"], c["nv"]))
    _same(o1, o0, "o")
    _same(s1, s0, "final state")
    _same(cs1, cs0, "conv state out")


def test_grouped_prep_full_varlen_workload():
    wl = W.WORKLOADS["varlen_prefill_8seq"]
    _say("prep grouping, full workload", wl.name)
    x = W.chunk_inputs(wl, device=dev())
    run = lambda: gdn.gdn_chunk_fwd_gated(x["q"], x["k"], x["v"], x["a"], x["b"], x["A_log"], x["dt_bias"],
                                          cu_seqlens=x["cu_seqlens"], initial_state=x["S0"])
    (o0, s0), (o1, s1) = _both(run)
    _same(o1, o0, "o")
    _same(s1, s0, "final state")


@pytest.mark.parametrize("fused", [False, True], ids=["chunk", "fused_prefill"])
def test_grouped_prep_under_a_segment_split(fused):
    """One sequence with few heads split into segments (GDN_SEGMENTS=3; the preparation then runs over the
    segment table): grouped and per-head preparation give the same bits."""
    old = os.environ.get("GDN_SEGMENTS")
    os.environ["GDN_SEGMENTS"] = "3"
    try:
        if fused:
            c = dict(name="segments_fused", T=5000, nk=1, nv=4, bias=True, conv_state=True, s0=True)
            _say("prep grouping under segments", c)
            d = PF._inputs(c, 970)
            (o0, s0, cs0), (o1, s1, cs1) = _both(lambda: PF._fused(d, c["nk"], c["nv"]))
            _same(cs1, cs0, "conv state out")
        else:
            _say("prep grouping under segments, chunk call, T=5000, 1->4 heads")
            wl = W.Workload("t", 971, "chunk", "bf16", nk=1, nv=4, s0_std=0.3)
            x = W.chunk_inputs(wl, lengths=[5000])
            d = {k: (v.to(dev()) if isinstance(v, torch.Tensor) else v) for k, v in x.items()}
            run = lambda: gdn.gdn_chunk_fwd_gated(d["q"], d["k"], d["v"], d["a"], d["b"], d["A_log"], d["dt_bias"],
                                                  initial_state=d["S0"])
            (o0, s0), (o1, s1) = _both(run)
        _same(o1, o0, "o")
        _same(s1, s0, "final state")
    finally:
        if old is None:
            del os.environ["GDN_SEGMENTS"]
        else:
            os.environ["GDN_SEGMENTS"] = old
