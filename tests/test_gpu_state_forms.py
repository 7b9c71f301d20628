"""GPU tests of the two forms of the bf16 chunk state kernel.

The library runs the four-wave form (one workgroup per 16-column slice) while
every slice gets a CU of its own, and the wide form (two slices per
workgroup, one recurrence wave per slice holding all 128 rows of S) when a
launch has more slices than the device has CUs; the environment variable
GDN_STATE_FORM=narrow|wide forces either. The wide form sums K S in the same
two halves as the four-wave form, so both give the same bits. These tests run
each form on the same inputs and require equal o, final state and (for the
fused prefill) conv state, over ragged, short and empty sequences, initial
states, head groupings r = 1, 2 and 4, bf16 output and the conv inside the
chunk kernels, and on the full prefill and varlen workloads. One case is also
checked against the fp64 oracle directly. Each test prints its case before
touching the GPU.
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


def _say(*a):
    print("[case]", *a, flush=True)


@contextlib.contextmanager
def _form(name):
    old = os.environ.get("GDN_STATE_FORM")
    os.environ["GDN_STATE_FORM"] = name
    try:
        yield
    finally:
        if old is None:
            del os.environ["GDN_STATE_FORM"]
        else:
            os.environ["GDN_STATE_FORM"] = old


def _chunk_inputs(lengths, nk, nv, seed, s0_std):
    wl = W.Workload("t", seed, "chunk", "bf16", nk=nk, nv=nv, s0_std=s0_std)
    x = W.chunk_inputs(wl, lengths=lengths)
    return x, {k: (v.to(dev()) if isinstance(v, torch.Tensor) else v) for k, v in x.items()}


def _gated(d, with_s0, o_dtype):
    # one sequence runs without cu_seqlens (the bench's call), several with them
    cu = d["cu_seqlens"] if len(d["lengths"]) > 1 else None
    return gdn.gdn_chunk_fwd_gated(d["q"], d["k"], d["v"], d["a"], d["b"], d["A_log"], d["dt_bias"],
                                   cu_seqlens=cu, initial_state=d["S0"] if with_s0 else None, o_dtype=o_dtype)


def _same(a, b, what):
    diff = (a.double() - b.double()).abs().max().item() if a.numel() else 0.0
    print(f"[exact] {what}: max |wide - narrow| = {diff:.3e}", flush=True)
    assert torch.equal(a, b), f"{what}: the wide form differs from the four-wave form"


def _both_forms(fn):
    with _form("narrow"):
        r_n = fn()
    with _form("wide"):
        r_w = fn()
    torch.cuda.synchronize()
    return r_n, r_w


CASES = [
    dict(name="one_sequence_ragged_r2", lengths=[200], nk=2, nv=4, s0=True),
    dict(name="varlen_short_and_empty_r2", lengths=[1, 63, 64, 65, 130, 0, 7], nk=1, nv=2, s0=True),
    dict(name="r4_bf16_output", lengths=[300], nk=1, nv=4, s0=True, o_dtype="bf16"),
    dict(name="r1_zero_state", lengths=[256, 17], nk=2, nv=2, s0=False),
    dict(name="one_head", lengths=[129], nk=1, nv=1, s0=True),
]


@pytest.mark.parametrize("ci", range(len(CASES)), ids=[c["name"] for c in CASES])
def test_wide_form_equals_four_wave_form(ci):
    c = CASES[ci]
    _say("state forms", c)
    _, d = _chunk_inputs(c["lengths"], c["nk"], c["nv"], 40 + ci, 0.3)
    o_dtype = torch.bfloat16 if c.get("o_dtype") == "bf16" else torch.float32
    (o_n, s_n), (o_w, s_w) = _both_forms(lambda: _gated(d, c["s0"], o_dtype))
    _same(o_w, o_n, "o")
    _same(s_w, s_n, "final state")


@pytest.mark.parametrize("seed", range(8))
def test_wide_form_random_shapes(seed):
    """Seeded random shapes (1-6 sequences of 0-199 tokens, 1-3 key heads with 1, 2 or 4 value heads each,
    with or without an initial state), each form against the other."""
    rng = np.random.RandomState(3000 + seed)
    nk = int(rng.choice([1, 2, 3]))
    nv = nk * int(rng.choice([1, 2, 4]))
    lengths = [int(v) for v in rng.randint(0, 200, size=int(rng.randint(1, 7)))]
    with_s0 = bool(rng.randint(0, 2))
    _say("state forms random", seed, lengths, nk, nv, "S0" if with_s0 else "zero S0")
    _, d = _chunk_inputs(lengths, nk, nv, 600 + seed, 0.3)
    (o_n, s_n), (o_w, s_w) = _both_forms(lambda: _gated(d, with_s0, torch.float32))
    _same(o_w, o_n, "o")
    _same(s_w, s_n, "final state")


def test_wide_form_against_oracle():
    """The wide form on its own against the fp64 oracle (varlen with initial states)."""
    lengths, nk, nv = [5, 130, 64, 0, 77], 1, 2
    _say("wide form vs oracle", lengths, nk, nv)
    x, d = _chunk_inputs(lengths, nk, nv, 77, 0.3)
    with _form("wide"):
        o, st = _gated(d, True, torch.float32)
    torch.cuda.synchronize()
    g_ref, b_ref = oracle.gating(f64(x["a"]), f64(x["b"]), f64(x["A_log"]), f64(x["dt_bias"]))
    o_ref, S_ref = oracle.delta_rule(f64(x["q"]), f64(x["k"]), f64(x["v"]), g_ref, b_ref,
                                     cu_seqlens=x["cu_seqlens"].numpy(), initial_state=f64(x["S0"]))
    assert_close(o, o_ref, TOL["bf16"], "wide o")
    assert_close(st, S_ref, TOL["bf16"], "wide final state")


@pytest.mark.parametrize("ci", range(len(PF.CASES)), ids=[c["name"] for c in PF.CASES])
def test_wide_form_fused_prefill(ci):
    """The conv inside the chunk kernels: gdn_prefill_fused in each form, o, final state and conv state."""
    c = PF.CASES[ci]
    _say("state forms, fused prefill", c)
    d = PF._inputs(c, 170 + ci)
    (o_n, s_n, cs_n), (o_w, s_w, cs_w) = _both_forms(lambda: PF._fused(d, c["nk"], c["nv"]))
    _same(o_w, o_n, "o")
    _same(s_w, s_n, "final state")
    _same(cs_w, cs_n, "conv state out")


@pytest.mark.parametrize("name", ["prefill_chunk_t8k", "varlen_prefill_8seq"])
def test_wide_form_full_workloads(name):
    """Both forms on the full prefill workload (which the library runs in the four-wave form) and on the
    full varlen workload (which it runs in the wide form), bit for bit."""
    wl = W.WORKLOADS[name]
    _say("state forms, full workload", name)
    x = W.chunk_inputs(wl, device=dev())
    with_s0 = x.get("S0") is not None
    (o_n, s_n), (o_w, s_w) = _both_forms(lambda: _gated(x, with_s0, torch.float32))
    _same(o_w, o_n, "o")
    _same(s_w, s_n, "final state")
