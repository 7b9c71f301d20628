"""GPU parity of gdn_prefill_fused_norm: the fused prefill followed by the
layer's gated RMSNorm of its output in one call.

Reference: gdn_prefill_fused (held bit for bit to the separate conv, gating
and chunk launches, and through them to the fp64 oracle) followed by
gdn_gated_rmsnorm (held to the oracle's gated_rmsnorm by the kernel tests).
The final state and the conv state out must equal the reference's bit for
bit. y must equal it bit for bit where the norm runs as a second launch (the
four-wave state form); where it runs inside the wide state kernel, y differs
only by the order in which a row's 128 squares are summed, so the bound is
relative per element: two fp32 sums of 128 non-negative terms in different
orders differ by at most 2 * 127 u of the sum (u = 2^-24), which moves
rms^-1 by half of that, plus a few roundings of the final products; 2e-5 of
|y| covers both with room. The wide form is forced with GDN_STATE_FORM=wide
on the small cases (it is chosen by itself once the slices outnumber the
CUs). Each test prints its case before touching the GPU.
"""
import os

import pytest
import torch

import gated_deltanet_gdn_amd as gdn
import workloads as W
from gpu_common import dev

import test_gpu_prefill_fused as PF

pytestmark = pytest.mark.gpu
DK = 128
EPS = 1e-6
RTOL = 2e-5

CASES = [
    dict(name="one_sequence_ragged", T=200, nk=2, nv=4),
    dict(name="varlen_short_and_empty", lengths=[1, 2, 0, 70, 130, 64, 5, 129], nk=1, nv=2, bias=True,
         conv_state=True, s0=True),
    dict(name="r4_strided_x_f32_gating", T=300, nk=1, nv=4, bias=True, conv_state=True, s0=True, ab="f32", pad=64),
    dict(name="eight_heads_many_chunks", T=1000, nk=2, nv=8, s0=True),
    dict(name="no_tokens", lengths=[0, 0], nk=1, nv=2, conv_state=True, s0=True),
]


def _say(*a):
    print("[case]", *a, flush=True)


class _Form:
    """Sets GDN_STATE_FORM for the calls inside the block (the library reads it per call)."""

    def __init__(self, form):
        self.form, self.old = form, None

    def __enter__(self):
        self.old = os.environ.get("GDN_STATE_FORM")
        os.environ["GDN_STATE_FORM"] = self.form

    def __exit__(self, *exc):
        if self.old is None:
            del os.environ["GDN_STATE_FORM"]
        else:
            os.environ["GDN_STATE_FORM"] = self.old


def _norm_inputs(c, seed):
    d = PF._inputs(dict(c, o_dtype="f32"), seed)
    T = d["x"].shape[0]
    d["z"] = W.randn((T, c["nv"], DK), seed, W.IDX["z"], "bf16", device=dev())
    d["norm_w"] = W.randn((DK,), seed, W.IDX["norm_w"], "f32", std=0.1, device=dev())
    return d


def _reference(d, nk, nv):
    o, st, cs = PF._fused(d, nk, nv)
    y = gdn.gdn_gated_rmsnorm(o, d["z"], d["norm_w"], eps=EPS)
    return y, st, cs


def _fused_norm(d, nk, nv):
    return gdn.gdn_prefill_fused_norm(d["x"], d["conv_w"], d["a"], d["b"], d["A_log"], d["dt_bias"], nk, nv,
                                      d["z"], d["norm_w"], eps=EPS, conv_bias=d["bias"], cu_seqlens=d["cu"],
                                      conv_state_in=d["conv_state"], state_len=d["state_len"],
                                      initial_state=d["s0"])


def _close(y, y_ref, what):
    if not y.numel():
        return
    assert torch.isfinite(y).all(), f"{what}: non-finite output"
    err = (y.double() - y_ref.double()).abs()
    ratio = (err / y_ref.double().abs().clamp_min(1e-30)).max().item()
    print(f"[tol] {what}: max |y - ref| / |ref| = {ratio:.3e} (bound {RTOL:.0e})", flush=True)
    assert (err <= RTOL * y_ref.double().abs()).all(), f"{what}: beyond {RTOL} of |ref|"


@pytest.mark.parametrize("ci", range(len(CASES)), ids=[c["name"] for c in CASES])
def test_fused_norm_in_the_wide_kernel(ci):
    c = CASES[ci]
    _say("prefill_fused_norm wide", c)
    d = _norm_inputs(c, 500 + ci)
    with _Form("wide"):
        y_r, st_r, cs_r = _reference(d, c["nk"], c["nv"])
        y, st, cs = _fused_norm(d, c["nk"], c["nv"])
    torch.cuda.synchronize()
    PF._same(st, st_r, "final state")
    if cs_r is not None:
        PF._same(cs, cs_r, "conv state out")
    _close(y, y_r, "y")
    if y.numel():
        # the in-kernel route sums squares in another order than the norm kernel, so some bits differ;
        # equal bits everywhere would mean the call fell back to the second launch
        assert not torch.equal(y, y_r), "the norm did not run inside the state kernel"


@pytest.mark.parametrize("ci", [0, 1, 3], ids=[CASES[i]["name"] for i in (0, 1, 3)])
def test_fused_norm_second_launch_is_bit_exact(ci):
    """With the four-wave state form the norm runs as a second launch over y: the same bits as the
    separate calls."""
    c = CASES[ci]
    _say("prefill_fused_norm narrow", c)
    d = _norm_inputs(c, 600 + ci)
    with _Form("narrow"):
        y_r, st_r, cs_r = _reference(d, c["nk"], c["nv"])
        y, st, cs = _fused_norm(d, c["nk"], c["nv"])
    torch.cuda.synchronize()
    PF._same(y, y_r, "y")
    PF._same(st, st_r, "final state")


def test_fused_norm_segment_parallel_falls_back():
    """One sequence with few heads runs segment-parallel; the norm then follows as a second launch."""
    c = dict(name="segments", T=4096, nk=1, nv=2, s0=True)
    _say("prefill_fused_norm segment-parallel", c)
    d = _norm_inputs(c, 650)
    y_r, st_r, _ = _reference(d, 1, 2)
    y, st, _ = _fused_norm(d, 1, 2)
    torch.cuda.synchronize()
    PF._same(y, y_r, "y")
    PF._same(st, st_r, "final state")


def test_fused_norm_twice_with_a_shared_workspace():
    """The tag ring in the workspace is cleared per call: a second, smaller call on the same workspace
    (stale tags of the first in it) gives the same result as on a fresh one."""
    big = dict(name="big", lengths=[700, 300, 129], nk=1, nv=4)
    small = dict(name="small", lengths=[200, 64], nk=1, nv=4, s0=True)
    _say("prefill_fused_norm twice", big["name"], small["name"])
    db, ds = _norm_inputs(big, 660), _norm_inputs(small, 661)
    need = gdn.gdn_chunk_fwd_workspace_size(1129, 3, 1, 4, DK, DK, gdn.BF16)
    ws = torch.empty(need, device=dev(), dtype=torch.uint8)
    with _Form("wide"):
        a = gdn.gdn_prefill_fused_norm(db["x"], db["conv_w"], db["a"], db["b"], db["A_log"], db["dt_bias"], 1, 4,
                                       db["z"], db["norm_w"], eps=EPS, cu_seqlens=db["cu"], workspace=ws)
        y1, st1, _ = gdn.gdn_prefill_fused_norm(ds["x"], ds["conv_w"], ds["a"], ds["b"], ds["A_log"],
                                                ds["dt_bias"], 1, 4, ds["z"], ds["norm_w"], eps=EPS,
                                                cu_seqlens=ds["cu"], initial_state=ds["s0"], workspace=ws)
        y2, st2, _ = _fused_norm(ds, 1, 4)
    torch.cuda.synchronize()
    del a
    PF._same(y1, y2, "y")
    PF._same(st1, st2, "final state")


def test_fused_norm_rejects_bad_arguments():
    c = CASES[0]
    _say("prefill_fused_norm argument checks")
    d = _norm_inputs(c, 670)
    with pytest.raises(gdn.GdnError):
        gdn.gdn_prefill_fused_norm(d["x"], d["conv_w"], d["a"], d["b"], d["A_log"], d["dt_bias"], 2, 4,
                                   d["z"].float(), d["norm_w"], eps=EPS)
    with pytest.raises(gdn.GdnError):
        gdn.gdn_prefill_fused_norm(d["x"], d["conv_w"], d["a"], d["b"], d["A_log"], d["dt_bias"], 2, 4,
                                   d["z"], d["norm_w"], eps=-1.0)


@pytest.mark.parametrize("seed", range(6))
def test_fused_norm_random_shapes(seed):
    """Seeded random shapes (sequence count and lengths, head grouping, conv history and bias, initial state,
    gating dtype, x stride, state form): the final state and conv state bit for bit, y within the bound."""
    import numpy as np
    rng = np.random.RandomState(4000 + seed)
    nk = int(rng.choice([1, 2]))
    c = dict(name=f"random_{seed}", lengths=[int(v) for v in rng.randint(0, 260, size=int(rng.randint(1, 5)))],
             nk=nk, nv=nk * int(rng.choice([1, 2, 4])), bias=bool(rng.randint(0, 2)),
             conv_state=bool(rng.randint(0, 2)), s0=bool(rng.randint(0, 2)), ab=["bf16", "f32"][int(rng.randint(0, 2))],
             pad=int(rng.choice([0, 8, 64])), state_len=int(rng.choice([3, 4])))
    form = ["wide", "narrow"][seed % 2]
    _say("prefill_fused_norm random", form, c)
    d = _norm_inputs(c, 700 + seed)
    with _Form(form):
        y_r, st_r, cs_r = _reference(d, c["nk"], c["nv"])
        y, st, cs = _fused_norm(d, c["nk"], c["nv"])
    torch.cuda.synchronize()
    PF._same(st, st_r, "final state")
    if cs_r is not None:
        PF._same(cs, cs_r, "conv state out")
    if form == "narrow":
        PF._same(y, y_r, "y")
    else:
        _close(y, y_r, "y")
