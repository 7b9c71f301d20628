"""GPU parity of the fused prefill (causal conv1d + SiLU, gating and the
chunked rule in one call, the conv applied inside the chunk kernels).

The fused call must equal the separate launches (gdn_causal_conv1d,
gdn_gating, gdn_chunk_fwd on the views of the conv output) bit for bit: o,
the final state and the conv state out. Those launches are held to the fp64
oracle by the other GPU tests. Cases cover one ragged sequence, packed
sequences of 0, 1 and 2 tokens (shorter than the conv window), sequences that
end on and off a chunk boundary, a conv history longer than the window,
conv bias, initial states, fp32 and bf16 gating inputs and outputs, a
token-strided x view, and a batch with no tokens. Each test prints its case
before touching the GPU.
"""
import numpy as np
import pytest
import torch

import gated_deltanet_gdn_amd as gdn
import workloads as W
from gpu_common import dev

pytestmark = pytest.mark.gpu
DK = 128

CASES = [
    dict(name="one_sequence_ragged", T=200, nk=2, nv=4),
    dict(name="varlen_short_and_empty", lengths=[1, 2, 0, 70, 130, 64, 5, 129], nk=1, nv=2, bias=True,
         conv_state=True, s0=True, o_dtype="bf16"),
    dict(name="r4_strided_x_f32_gating", T=300, nk=1, nv=4, bias=True, conv_state=True, s0=True, ab="f32", pad=64),
    dict(name="r1_two_sequences", lengths=[100, 37], nk=2, nv=2, conv_state=True),
    dict(name="history_longer_than_window", lengths=[3, 66, 1], nk=1, nv=2, conv_state=True, state_len=5, s0=True),
    dict(name="no_tokens", lengths=[0, 0], nk=1, nv=2, conv_state=True, s0=True),
]


def _say(*a):
    print("[case]", *a, flush=True)


def _inputs(c, seed):
    nk, nv = c["nk"], c["nv"]
    C = (2 * nk + nv) * DK
    lengths = c.get("lengths")
    T = sum(lengths) if lengths is not None else c["T"]
    n = len(lengths) if lengths is not None else 1
    sl = c.get("state_len", 3)
    pad = c.get("pad", 0)
    ab = c.get("ab", "bf16")
    D = dev()
    xw = W.randn((T, C + pad), seed, W.IDX["x"], "bf16", device=D)
    d = dict(
        x=xw[:, :C],
        conv_w=W.uniform((C, 4), seed, W.IDX["conv_w"], -0.5, 0.5, D),
        bias=W.randn((C,), seed, W.IDX["conv_w"] + 100, "f32", std=0.1, device=D) if c.get("bias") else None,
        conv_state=W.randn((n, C, sl), seed, W.IDX["conv_state"], "bf16", device=D) if c.get("conv_state") else None,
        a=W.randn((T, nv), seed, W.IDX["a"], ab, device=D),
        b=W.randn((T, nv), seed, W.IDX["b"], ab, device=D),
        A_log=W.a_log(nv, seed, D),
        dt_bias=W.randn((nv,), seed, W.IDX["dt_bias"], "f32", std=0.1, device=D),
        s0=W.randn((n, nv, DK, DK), seed, W.IDX["S0"], "f32", std=0.02, device=D) if c.get("s0") else None,
        cu=torch.from_numpy(W.cu_from_lengths(lengths)).to(D, torch.int32) if lengths is not None else None,
        state_len=sl,
        o_dtype=torch.bfloat16 if c.get("o_dtype") == "bf16" else torch.float32,
    )
    return d


def _separate(d, nk, nv):
    y, cs = gdn.gdn_causal_conv1d(d["x"], d["conv_w"], bias=d["bias"], cu_seqlens=d["cu"],
                                  conv_state_in=d["conv_state"], state_len=d["state_len"])
    T = y.shape[0]
    kd = nk * DK
    q = y[:, :kd].view(T, nk, DK)
    k = y[:, kd:2 * kd].view(T, nk, DK)
    v = y[:, 2 * kd:].view(T, nv, DK)
    g, beta = gdn.gdn_gating(d["a"], d["b"], d["A_log"], d["dt_bias"])
    o, st = gdn.gdn_chunk_fwd(q, k, v, g, beta, cu_seqlens=d["cu"], initial_state=d["s0"], o_dtype=d["o_dtype"])
    return o, st, cs


def _fused(d, nk, nv):
    return gdn.gdn_prefill_fused(d["x"], d["conv_w"], d["a"], d["b"], d["A_log"], d["dt_bias"], nk, nv,
                                 conv_bias=d["bias"], cu_seqlens=d["cu"], conv_state_in=d["conv_state"],
                                 state_len=d["state_len"], initial_state=d["s0"], o_dtype=d["o_dtype"])


def _same(a, b, what):
    diff = (a.double() - b.double()).abs().max().item() if a.numel() else 0.0
    print(f"[exact] {what}: max |fused - separate| = {diff:.3e}", flush=True)
    assert torch.equal(a, b), f"{what}: the fused prefill differs from the separate launches"


@pytest.mark.parametrize("ci", range(len(CASES)), ids=[c["name"] for c in CASES])
def test_prefill_fused_equals_separate_launches(ci):
    c = CASES[ci]
    _say("prefill_fused", c)
    d = _inputs(c, 70 + ci)
    o_s, st_s, cs_s = _separate(d, c["nk"], c["nv"])
    o_f, st_f, cs_f = _fused(d, c["nk"], c["nv"])
    torch.cuda.synchronize()
    _same(o_f, o_s, "o")
    _same(st_f, st_s, "final state")
    _same(cs_f, cs_s, "conv state out")


@pytest.mark.parametrize("seed", range(8))
def test_prefill_fused_random_shapes(seed):
    """Seeded random shapes (sequence count and lengths, head grouping, conv history and bias, initial state,
    gating and output dtypes, x stride), each against the separate launches."""
    rng = np.random.RandomState(2000 + seed)
    nk = int(rng.choice([1, 2, 3]))
    c = dict(name=f"random_{seed}", lengths=[int(v) for v in rng.randint(0, 180, size=int(rng.randint(1, 6)))],
             nk=nk, nv=nk * int(rng.choice([1, 2, 4])), bias=bool(rng.randint(0, 2)),
             conv_state=bool(rng.randint(0, 2)), s0=bool(rng.randint(0, 2)), ab=["bf16", "f32"][int(rng.randint(0, 2))],
             o_dtype=["f32", "bf16"][int(rng.randint(0, 2))], pad=int(rng.choice([0, 8, 64])),
             state_len=int(rng.choice([3, 4])))
    _say("prefill_fused random", c)
    d = _inputs(c, 300 + seed)
    o_s, st_s, cs_s = _separate(d, c["nk"], c["nv"])
    o_f, st_f, cs_f = _fused(d, c["nk"], c["nv"])
    torch.cuda.synchronize()
    _same(o_f, o_s, "o")
    _same(st_f, st_s, "final state")
    _same(cs_f, cs_s, "conv state out")


def test_prefill_fused_called_twice_gives_the_same_bits():
    """The workspace's stale contents from a larger call do not leak into a smaller one."""
    c = CASES[1]
    _say("prefill_fused twice", c["name"])
    big = _inputs(dict(c, lengths=[300, 200, 129]), 90)
    small = _inputs(c, 71)
    need = max(gdn.gdn_chunk_fwd_workspace_size(629, 3, 1, 2, DK, DK, gdn.BF16),
               gdn.gdn_chunk_fwd_workspace_size(401, 8, 1, 2, DK, DK, gdn.BF16))
    ws = torch.empty(need, device=dev(), dtype=torch.uint8)
    gdn.gdn_prefill_fused(big["x"], big["conv_w"], big["a"], big["b"], big["A_log"], big["dt_bias"], 1, 2,
                          conv_bias=big["bias"], cu_seqlens=big["cu"], conv_state_in=big["conv_state"],
                          initial_state=big["s0"], o_dtype=big["o_dtype"], workspace=ws)
    r1 = gdn.gdn_prefill_fused(small["x"], small["conv_w"], small["a"], small["b"], small["A_log"],
                               small["dt_bias"], 1, 2, conv_bias=small["bias"], cu_seqlens=small["cu"],
                               conv_state_in=small["conv_state"], initial_state=small["s0"],
                               o_dtype=small["o_dtype"], workspace=ws)
    o_s, st_s, cs_s = _separate(small, 1, 2)
    torch.cuda.synchronize()
    _same(r1[0], o_s, "o")
    _same(r1[1], st_s, "final state")
    _same(r1[2], cs_s, "conv state out")
