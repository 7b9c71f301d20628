"""GPU parity of every libgdn entry point against the fp64 CPU oracle (small inputs).

Sizes span several 64-token chunks with ragged tails, several sequences
(including empty and one-token ones), both input dtypes and grouped heads.
Each test prints the case it runs before touching the GPU.
"""
import math

import numpy as np
import pytest
import torch

import gated_deltanet_gdn_amd as gdn
import oracle
import workloads as W
from gpu_common import TOL, assert_close, assert_conv_close, bf16_ulp_diff, conv_abs_sum, dev, f64

pytestmark = pytest.mark.gpu


def _say(*a):
    print("[case]", *a, flush=True)


def _inputs(dtype, lengths, nk, nv, s0_std=0.0, seed=7):
    wl = W.Workload("t", seed, "chunk", dtype, nk=nk, nv=nv, s0_std=s0_std)
    return W.chunk_inputs(wl, lengths=lengths)


def _to(d, device):
    return {k: (v.to(device) if isinstance(v, torch.Tensor) else v) for k, v in d.items()}


# ------------------------------------------------------------------ gating

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("nk,nv", [(2, 6), (1, 4), (3, 12), (4, 32)])   # one, four or eight heads per thread
def test_gating(dtype, nk, nv):
    _say("gating", dtype, nk, nv)
    x = _inputs(dtype, [300], nk, nv)
    d = _to(x, dev())
    g, beta = gdn.gdn_gating(d["a"], d["b"], d["A_log"], d["dt_bias"])
    torch.cuda.synchronize()
    g_ref, b_ref = oracle.gating(f64(x["a"]), f64(x["b"]), f64(x["A_log"]), f64(x["dt_bias"]))
    # fp32 evaluation of exp / log1p / sigmoid: a few ulps of the result
    np.testing.assert_allclose(f64(g), g_ref, rtol=4e-6, atol=0)
    np.testing.assert_allclose(f64(beta), b_ref, rtol=4e-6, atol=0)


def test_gating_unaligned_views():
    _say("gating on views that start one token in (not 16-byte aligned)")
    x = _inputs("bf16", [101], 1, 8)
    d = _to(x, dev())
    a, b = d["a"][1:], d["b"][1:]                        # 16 bytes in for bf16 x 8 heads: aligned
    a2 = torch.empty((a.shape[0] * 8 + 1,), device=a.device, dtype=a.dtype)[1:].view(a.shape)
    a2.copy_(a)                                           # 2 bytes off a 16-byte boundary
    g2 = torch.empty((a.shape[0] * 8 + 1,), device=a.device)[1:].view(a.shape)
    g, beta = gdn.gdn_gating(a2, b, d["A_log"], d["dt_bias"], g=g2)
    g_ref, b_ref = oracle.gating(f64(x["a"][1:]), f64(x["b"][1:]), f64(x["A_log"]), f64(x["dt_bias"]))
    np.testing.assert_allclose(f64(g), g_ref, rtol=4e-6)
    np.testing.assert_allclose(f64(beta), b_ref, rtol=4e-6)


def test_gating_odd_head_count():
    _say("gating nv=3")
    x = _inputs("bf16", [77], 1, 3)
    d = _to(x, dev())
    g, beta = gdn.gdn_gating(d["a"], d["b"], d["A_log"], d["dt_bias"])
    g_ref, b_ref = oracle.gating(f64(x["a"]), f64(x["b"]), f64(x["A_log"]), f64(x["dt_bias"]))
    np.testing.assert_allclose(f64(g), g_ref, rtol=4e-6)
    np.testing.assert_allclose(f64(beta), b_ref, rtol=4e-6)


# ------------------------------------------------------------------ gated RMSNorm

@pytest.mark.parametrize("xd,zd,yd", [("f32", "f32", "f32"), ("f32", "bf16", "f32"), ("bf16", "bf16", "bf16")])
def test_gated_rmsnorm(xd, zd, yd):
    _say("rmsnorm", xd, zd, yd)
    rows, D = 777, 128
    x = W.randn((rows, D), 3, 1, xd)
    z = W.randn((rows, D), 3, 2, zd)
    w = W.randn((D,), 3, 3, "f32", std=0.1)
    y = gdn.gdn_gated_rmsnorm(x.to(dev()), z.to(dev()), w.to(dev()), eps=1e-6, y_dtype=W.TORCH_DTYPE[yd])
    ref = oracle.gated_rmsnorm(f64(x), f64(z), f64(w), eps=1e-6)
    if yd == "f32":
        assert_close(y, ref, TOL["f32"], "rmsnorm")
    else:
        assert int(bf16_ulp_diff(y, ref).max()) <= 1


def test_gated_rmsnorm_wide_rows():
    _say("rmsnorm D=512")
    x = W.randn((33, 512), 4, 1); z = W.randn((33, 512), 4, 2); w = W.randn((512,), 4, 3, std=0.1)
    y = gdn.gdn_gated_rmsnorm(x.to(dev()), z.to(dev()), w.to(dev()))
    assert_close(y, oracle.gated_rmsnorm(f64(x), f64(z), f64(w)), TOL["f32"], "rmsnorm D=512")


# ------------------------------------------------------------------ causal conv

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("with_state", [False, True])
def test_causal_conv1d_varlen(dtype, with_state):
    _say("conv", dtype, with_state)
    lengths = [70, 0, 1, 130, 2, 200]
    C, K, SL = 96, 4, 3
    cu = W.cu_from_lengths(lengths)
    T = int(cu[-1])
    x = W.randn((T, C), 5, 1, dtype)
    w = W.uniform((C, K), 5, 2, -0.5, 0.5)
    b = W.randn((C,), 5, 3, "f32")
    st = W.randn((len(lengths), C, SL), 5, 4, dtype) if with_state else None
    d = dev()
    y, so = gdn.gdn_causal_conv1d(x.to(d), w.to(d), b.to(d), cu_seqlens=torch.tensor(cu, dtype=torch.int32, device=d),
                                  conv_state_in=None if st is None else st.to(d), state_len=SL)
    y_ref, so_ref = oracle.causal_conv1d(f64(x), f64(w), f64(b), cu_seqlens=cu,
                                         conv_state=None if st is None else f64(st), state_len=SL)
    if dtype == "bf16":
        s_abs = np.concatenate([conv_abs_sum(np.concatenate([(f64(st)[n].T[-3:] if st is not None else np.zeros((3, C))),
                                                             f64(x)[cu[n]:cu[n + 1]]]), f64(w))
                                for n in range(len(lengths))]) + np.abs(f64(b))[None]
        assert_conv_close(y, y_ref, s_abs, "conv varlen")
    else:
        assert_close(y, y_ref, TOL["f32"], "conv f32")
    np.testing.assert_array_equal(f64(so), so_ref)   # the state is a copy of inputs: exact


def test_causal_conv1d_strided_view_and_long_state():
    _say("conv strided view, state_len 4")
    T, Cfull, C, SL = 150, 160, 64, 4
    xfull = W.randn((T, Cfull), 6, 1, "bf16")
    x = xfull[:, 32:32 + C]                     # token stride 160
    w = W.uniform((C, 4), 6, 2, -0.5, 0.5)
    st = W.randn((1, C, SL), 6, 3, "bf16")
    d = dev()
    y, so = gdn.gdn_causal_conv1d(xfull.to(d)[:, 32:32 + C], w.to(d), conv_state_in=st.to(d))
    y_ref, so_ref = oracle.causal_conv1d(f64(x), f64(w), conv_state=f64(st))
    assert_conv_close(y, y_ref, conv_abs_sum(np.concatenate([f64(st)[0].T[-3:], f64(x)]), f64(w)), "conv strided")
    np.testing.assert_array_equal(f64(so), so_ref)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("state_len,C", [(3, 200), (4, 200), (3, 36)])   # 8-channel vector path when C % 8 == 0
def test_causal_conv1d_update(dtype, state_len, C):
    _say("conv update", dtype, state_len, C)
    n = 37
    x = W.randn((n, C), 8, 1, dtype)
    st = W.randn((n, C, state_len), 8, 2, dtype)
    w = W.uniform((C, 4), 8, 3, -0.5, 0.5)
    b = W.randn((C,), 8, 4)
    d = dev()
    st_d = st.to(d)
    y = gdn.gdn_causal_conv1d_update(x.to(d), st_d, w.to(d), b.to(d))
    y_ref, st_ref = oracle.causal_conv1d_update(f64(x), f64(st), f64(w), f64(b))
    if dtype == "bf16":
        win = np.concatenate([f64(st)[:, :, -3:], f64(x)[:, :, None]], axis=2)
        s_abs = np.sum(np.abs(win) * np.abs(f64(w))[None], axis=2) + np.abs(f64(b))[None]
        assert_conv_close(y, y_ref, s_abs, "conv update")
    else:
        assert_close(y, y_ref, TOL["f32"], "conv update")
    np.testing.assert_array_equal(f64(st_d), st_ref)


# ------------------------------------------------------------------ recurrent (decode)

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_recurrent_one_token_per_sequence(dtype):
    _say("recurrent 1 token", dtype)
    n, nk, nv = 40, 2, 4
    x = _inputs(dtype, [1] * n, nk, nv, s0_std=0.5)
    d = _to(x, dev())
    g, beta = gdn.gdn_gating(d["a"], d["b"], d["A_log"], d["dt_bias"])
    state = d["S0"].clone()
    o = gdn.gdn_recurrent_fwd(d["q"], d["k"], d["v"], g, beta, state)
    g_ref, b_ref = oracle.gating(f64(x["a"]), f64(x["b"]), f64(x["A_log"]), f64(x["dt_bias"]))
    o_ref, S_ref = oracle.delta_rule(f64(x["q"]), f64(x["k"]), f64(x["v"]), g_ref, b_ref,
                                     cu_seqlens=np.arange(n + 1), initial_state=f64(x["S0"]))
    assert_close(o, o_ref, TOL[dtype], "recurrent o")
    assert_close(state, S_ref, TOL[dtype], "recurrent state")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_recurrent_multi_token_varlen(dtype):
    _say("recurrent varlen", dtype)
    lengths = [4, 0, 1, 9, 3]
    x = _inputs(dtype, lengths, 1, 2, s0_std=0.5)
    d = _to(x, dev())
    cu = x["cu_seqlens"]
    g, beta = gdn.gdn_gating(d["a"], d["b"], d["A_log"], d["dt_bias"])
    state = d["S0"].clone()
    o = gdn.gdn_recurrent_fwd(d["q"], d["k"], d["v"], g, beta, state, cu_seqlens=d["cu_seqlens"])
    g_ref, b_ref = oracle.gating(f64(x["a"]), f64(x["b"]), f64(x["A_log"]), f64(x["dt_bias"]))
    o_ref, S_ref = oracle.delta_rule(f64(x["q"]), f64(x["k"]), f64(x["v"]), g_ref, b_ref,
                                     cu_seqlens=cu.numpy(), initial_state=f64(x["S0"]))
    assert_close(o, o_ref, TOL[dtype], "recurrent varlen o")
    assert_close(state, S_ref, TOL[dtype], "recurrent varlen state")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_recurrent_strong_decay_rescale(dtype):
    """The decode kernels carry the state as E times a rescaled state, E the product of the decays since the
    last rescale, and fold E in once it would fall below 2^-64. Decays of e^-30 per token cross that floor
    on the third token of a sequence, e^-120 underflows to zero in fp32 (the state is then replaced by the
    update alone), and mixed runs alternate; each against the oracle, with g and beta given directly."""
    _say("recurrent strong decay", dtype)
    lengths = [6, 5, 4, 1]
    x = _inputs(dtype, lengths, 1, 2, s0_std=0.5)
    T = sum(lengths)
    gvals = np.concatenate([np.full(6, -30.0), np.full(5, -120.0), np.array([-0.1, -45.0, -0.2, -60.0]),
                            np.array([-200.0])])
    g = np.stack([gvals, gvals * 0.5], 1).astype(np.float32)              # [T, nv]
    beta = np.full((T, 2), 0.7, dtype=np.float32)
    d = _to(x, dev())
    state = d["S0"].clone()
    o = gdn.gdn_recurrent_fwd(d["q"], d["k"], d["v"], torch.from_numpy(g).to(dev()),
                              torch.from_numpy(beta).to(dev()), state, cu_seqlens=d["cu_seqlens"])
    o_ref, S_ref = oracle.delta_rule(f64(x["q"]), f64(x["k"]), f64(x["v"]), g.astype(np.float64),
                                     beta.astype(np.float64), cu_seqlens=x["cu_seqlens"].numpy(),
                                     initial_state=f64(x["S0"]))
    assert_close(o, o_ref, TOL[dtype], "recurrent strong decay o")
    assert_close(state, S_ref, TOL[dtype], "recurrent strong decay state")


# ------------------------------------------------------------------ chunk with the gating folded in

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("lengths,nk,nv", [([200], 2, 4), ([1, 63, 64, 65, 130, 0, 7], 1, 2), ([300], 1, 4)])
def test_chunk_fwd_gated_equals_gating_then_chunk(dtype, lengths, nk, nv):
    _say("chunk with gating folded in", dtype, lengths, nk, nv)
    x = _inputs(dtype, lengths, nk, nv, s0_std=0.5)
    d = _to(x, dev())
    g, beta = gdn.gdn_gating(d["a"], d["b"], d["A_log"], d["dt_bias"])
    o1, s1 = gdn.gdn_chunk_fwd(d["q"], d["k"], d["v"], g, beta, cu_seqlens=d["cu_seqlens"], initial_state=d["S0"])
    o2, s2 = gdn.gdn_chunk_fwd_gated(d["q"], d["k"], d["v"], d["a"], d["b"], d["A_log"], d["dt_bias"],
                                     cu_seqlens=d["cu_seqlens"], initial_state=d["S0"])
    torch.cuda.synchronize()
    assert torch.equal(o1, o2), f"o differs by {(o1 - o2).abs().max().item():.3e}"
    assert torch.equal(s1, s2), f"state differs by {(s1 - s2).abs().max().item():.3e}"


# ------------------------------------------------------------------ chunk (prefill)

def _run_chunk(x, dtype, with_s0=True, alias=False, o_dtype=torch.float32):
    d = _to(x, dev())
    g, beta = gdn.gdn_gating(d["a"], d["b"], d["A_log"], d["dt_bias"])
    s0 = d["S0"] if with_s0 else None
    if alias:
        st = s0.clone()
        o, fs = gdn.gdn_chunk_fwd(d["q"], d["k"], d["v"], g, beta, cu_seqlens=d["cu_seqlens"], initial_state=st,
                                  final_state=st, o_dtype=o_dtype)
    else:
        o, fs = gdn.gdn_chunk_fwd(d["q"], d["k"], d["v"], g, beta, cu_seqlens=d["cu_seqlens"], initial_state=s0,
                                  o_dtype=o_dtype)
    torch.cuda.synchronize()
    g_ref, b_ref = oracle.gating(f64(x["a"]), f64(x["b"]), f64(x["A_log"]), f64(x["dt_bias"]))
    o_ref, S_ref = oracle.delta_rule(f64(x["q"]), f64(x["k"]), f64(x["v"]), g_ref, b_ref,
                                     cu_seqlens=x["cu_seqlens"].numpy(),
                                     initial_state=None if s0 is None else f64(x["S0"]))
    return o, fs, o_ref, S_ref


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("lengths,nk,nv", [
    ([256], 1, 2),                       # whole chunks, grouped heads
    ([200], 2, 4),                       # ragged tail
    ([1, 63, 64, 65, 130, 0, 7], 1, 2),  # varlen incl. empty and one-token sequences
    ([300], 1, 4),                       # 4 value heads per key head
])
def test_chunk_small(dtype, lengths, nk, nv):
    _say("chunk", dtype, lengths, nk, nv)
    x = _inputs(dtype, lengths, nk, nv, s0_std=0.3)
    o, fs, o_ref, S_ref = _run_chunk(x, dtype)
    assert_close(o, o_ref, TOL[dtype], "chunk o")
    assert_close(fs, S_ref, TOL[dtype], "chunk final state")


@pytest.mark.parametrize("seed", range(12))
def test_chunk_random_shapes(seed):
    """Seeded random shapes: 1-6 sequences of 0-199 tokens, 1-3 key heads with 1, 2 or 4 value heads each
    (so the state kernel's work order takes each of its mappings), either dtype, with or without an
    initial state; each against the oracle."""
    rng = np.random.RandomState(1000 + seed)
    dtype = ["f32", "bf16"][seed % 2]
    nk = int(rng.choice([1, 2, 3]))
    nv = nk * int(rng.choice([1, 2, 4]))
    lengths = [int(v) for v in rng.randint(0, 200, size=int(rng.randint(1, 7)))]
    if sum(lengths) == 0:
        lengths[0] = 1
    with_s0 = bool(rng.randint(0, 2))
    _say("chunk random", seed, dtype, lengths, nk, nv, "S0" if with_s0 else "zero S0")
    x = _inputs(dtype, lengths, nk, nv, s0_std=0.3, seed=500 + seed)
    o, fs, o_ref, S_ref = _run_chunk(x, dtype, with_s0=with_s0)
    assert_close(o, o_ref, TOL[dtype], "chunk o")
    assert_close(fs, S_ref, TOL[dtype], "chunk final state")


def test_chunk_zero_initial_state_and_alias():
    _say("chunk zero S0 / aliased state")
    x = _inputs("bf16", [190, 70], 1, 2, s0_std=0.3)
    o, fs, o_ref, S_ref = _run_chunk(x, "bf16", with_s0=False)
    assert_close(o, o_ref, TOL["bf16"], "chunk o (S0 = 0)")
    assert_close(fs, S_ref, TOL["bf16"], "chunk state (S0 = 0)")
    o2, fs2, o_ref2, S_ref2 = _run_chunk(x, "bf16", alias=True)
    assert_close(o2, o_ref2, TOL["bf16"], "chunk o (aliased)")
    assert_close(fs2, S_ref2, TOL["bf16"], "chunk state (aliased)")


def test_chunk_slow_decay_stress():
    """A_log = 0 and a ~ N(-4, 1): g ~ -0.02, the carried state dominates the output."""
    _say("chunk slow decay")
    x = _inputs("bf16", [640], 1, 2, s0_std=0.3)
    x["A_log"] = torch.zeros_like(x["A_log"])
    x["a"] = (x["a"].float() - 4.0).to(torch.bfloat16)
    o, fs, o_ref, S_ref = _run_chunk(x, "bf16")
    assert_close(o, o_ref, TOL["bf16"], "slow decay o")
    assert_close(fs, S_ref, TOL["bf16"], "slow decay state")


def test_chunk_matches_recurrent_path():
    """Chunked and recurrent forms of the same sequence agree (both against the oracle and each other)."""
    _say("chunk vs recurrent")
    x = _inputs("bf16", [150], 1, 2, s0_std=0.3)
    d = _to(x, dev())
    g, beta = gdn.gdn_gating(d["a"], d["b"], d["A_log"], d["dt_bias"])
    o_c, s_c = gdn.gdn_chunk_fwd(d["q"], d["k"], d["v"], g, beta, initial_state=d["S0"])
    st = d["S0"].clone()
    o_r = gdn.gdn_recurrent_fwd(d["q"], d["k"], d["v"], g, beta, st, cu_seqlens=d["cu_seqlens"])
    assert_close(o_c, f64(o_r), 2 * TOL["bf16"], "chunk vs recurrent o")
    assert_close(s_c, f64(st), 2 * TOL["bf16"], "chunk vs recurrent state")


def test_chunk_bf16_output():
    _say("chunk bf16 output")
    x = _inputs("bf16", [200], 1, 2, s0_std=0.3)
    o, fs, o_ref, S_ref = _run_chunk(x, "bf16", o_dtype=torch.bfloat16)
    # one rounding of the output on top of the fp32 bar: 2e-3 RMS + half a bf16 ulp of |ref|
    err = np.abs(f64(o) - o_ref)
    rms = np.sqrt(np.mean(o_ref ** 2))
    assert np.all(err <= 2e-3 * rms + np.abs(o_ref) * 2.0 ** -8 + 1e-30)


# ------------------------------------------------------------------ closed forms through the GPU

def test_chunk_beta_zero_is_pure_decay():
    _say("chunk beta = 0")
    x = _inputs("bf16", [130], 1, 1, s0_std=0.5)
    d = _to(x, dev())
    g, _ = gdn.gdn_gating(d["a"], d["b"], d["A_log"], d["dt_bias"])
    g = g * 0.01                       # slow decay so the state stays visible
    beta = torch.zeros_like(g)
    o, fs = gdn.gdn_chunk_fwd(d["q"], d["k"], d["v"], g, beta, initial_state=d["S0"])
    G = np.cumsum(f64(g)[:, 0])
    q = f64(x["q"])[:, 0]
    qh = q / np.sqrt((q * q).sum(1, keepdims=True) + 1e-6) / math.sqrt(128)
    S0 = f64(x["S0"])[0, 0]
    o_ref = np.exp(G)[:, None] * (qh @ S0)
    assert_close(o[:, 0], o_ref, TOL["bf16"], "beta=0 o")
    assert_close(fs[0, 0], np.exp(G[-1]) * S0, TOL["bf16"], "beta=0 state")


def test_chunk_reset_and_orthonormal_keys():
    _say("chunk orthonormal keys, beta = 1, g = 0, no l2norm")
    T = 100
    rng = np.random.default_rng(3)
    Qm, _ = np.linalg.qr(rng.standard_normal((128, 128)))
    keys = torch.from_numpy(Qm[:T]).float()[:, None, :]     # fp32 inputs: exact keys
    v = torch.randn(T, 1, 128, generator=torch.Generator().manual_seed(5))
    S0 = torch.randn(1, 1, 128, 128, generator=torch.Generator().manual_seed(6))
    d = dev()
    g = torch.zeros(T, 1, device=d); beta = torch.ones(T, 1, device=d)
    o, fs = gdn.gdn_chunk_fwd(keys.to(d), keys.to(d), v.to(d), g, beta, initial_state=S0.to(d), scale=1.0,
                              qk_l2norm=False)
    assert_close(o[:, 0], f64(v)[:, 0], TOL["f32"], "orthonormal read-back")
    assert_close(keys[:, 0].double().numpy() @ f64(fs)[0, 0], f64(v)[:, 0], TOL["f32"], "values retrievable")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_chunk_and_recurrent_without_l2norm_custom_scale(dtype):
    """qk_l2norm = 0 and an explicit scale, on keys and queries of about unit norm (q, k drawn N(0, 1/128)),
    for the chunked rule and the recurrent rule against the oracle."""
    _say("no l2norm, scale 0.3", dtype)
    lengths, nk, nv = [150, 1, 77], 1, 2
    x = _inputs(dtype, lengths, nk, nv, s0_std=0.3, seed=41)
    TD = W.TORCH_DTYPE[dtype]
    for key in ("q", "k"):   # rescale in fp32, then back to the workload dtype (the oracle reads the same values)
        x[key] = (x[key].float() * (128 ** -0.5)).to(TD)
    d = _to(x, dev())
    g, beta = gdn.gdn_gating(d["a"], d["b"], d["A_log"], d["dt_bias"])
    o, fs = gdn.gdn_chunk_fwd(d["q"], d["k"], d["v"], g, beta, cu_seqlens=d["cu_seqlens"], initial_state=d["S0"],
                              scale=0.3, qk_l2norm=False)
    st = d["S0"].clone()
    o_r = gdn.gdn_recurrent_fwd(d["q"], d["k"], d["v"], g, beta, st, cu_seqlens=d["cu_seqlens"], scale=0.3,
                                qk_l2norm=False)
    torch.cuda.synchronize()
    g_ref, b_ref = oracle.gating(f64(x["a"]), f64(x["b"]), f64(x["A_log"]), f64(x["dt_bias"]))
    o_ref, S_ref = oracle.delta_rule(f64(x["q"]), f64(x["k"]), f64(x["v"]), g_ref, b_ref,
                                     cu_seqlens=x["cu_seqlens"].numpy(), initial_state=f64(x["S0"]), scale=0.3,
                                     l2norm=False)
    assert_close(o, o_ref, TOL[dtype], "chunk o (no l2norm)")
    assert_close(fs, S_ref, TOL[dtype], "chunk state (no l2norm)")
    assert_close(o_r, o_ref, TOL[dtype], "recurrent o (no l2norm)")
    assert_close(st, S_ref, TOL[dtype], "recurrent state (no l2norm)")


# ------------------------------------------------------------------ device graphs of the small kernels

def test_gating_and_conv_update_in_a_device_graph():
    """The bench times these two short kernels as captured graph replays: every replay (with eager work and
    syncs in between) must equal the eager calls on the same buffers."""
    _say("gating + conv update captured in a graph")
    d = dev()
    x = _to(_inputs("bf16", [96], 2, 8), d)
    n, C = 16, 256
    xc = W.randn((n, C), 9, 1, "bf16").to(d)
    w = W.uniform((C, 4), 9, 2, -0.5, 0.5).to(d)
    cs_g = W.randn((n, C, 3), 9, 3, "bf16").to(d)
    cs_e = cs_g.clone()
    g_g, b_g = torch.empty((96, 8), device=d), torch.empty((96, 8), device=d)
    y_g = torch.empty_like(xc)

    def calls(cs, g, b, y, stream=None):
        gdn.gdn_gating(x["a"], x["b"], x["A_log"], x["dt_bias"], g=g, beta=b, stream=stream)
        gdn.gdn_causal_conv1d_update(xc, cs, w, y=y, stream=stream)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side), torch.cuda.graph(graph, stream=side):
        calls(cs_g, g_g, b_g, y_g, stream=side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for rep in range(3):
        g_e, b_e, y_e = torch.empty_like(g_g), torch.empty_like(b_g), torch.empty_like(y_g)
        calls(cs_e, g_e, b_e, y_e)
        filler = torch.randn(1 << 20, device=d).sum()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.isfinite(filler)
        for a, b, nm in ((g_g, g_e, "g"), (b_g, b_e, "beta"), (y_g, y_e, "conv y"), (cs_g, cs_e, "conv state")):
            assert torch.equal(a, b), f"replay {rep}: {nm} differs from the eager call"


# ------------------------------------------------------------------ degenerate batches

def test_batches_without_tokens():
    """Sequences with no tokens at all (T_tot = 0): every entry point leaves the states as they were."""
    _say("batches of empty sequences")
    d = dev()
    nk, nv, n = 2, 4, 3
    cu = torch.zeros(n + 1, dtype=torch.int32, device=d)
    S0 = W.randn((n, nv, 128, 128), 21, 1, "f32", std=0.5).to(d)
    q = torch.empty((0, nk, 128), device=d, dtype=torch.bfloat16)
    v = torch.empty((0, nv, 128), device=d, dtype=torch.bfloat16)
    ab = torch.empty((0, nv), device=d, dtype=torch.bfloat16)
    gb = torch.empty((0, nv), device=d)
    A_log, dt_bias = torch.zeros(nv, device=d), torch.zeros(nv, device=d)
    o, st = gdn.gdn_chunk_fwd(q, q, v, gb, gb, cu_seqlens=cu, initial_state=S0)
    o2, st2 = gdn.gdn_chunk_fwd_gated(q, q, v, ab, ab, A_log, dt_bias, cu_seqlens=cu, initial_state=S0)
    rs = S0.clone()
    gdn.gdn_recurrent_fwd(q, q, v, gb, gb, rs, cu_seqlens=cu)
    C = (2 * nk + nv) * 128
    cs0 = W.randn((n, C, 3), 21, 2, "bf16").to(d)
    cs, fs = cs0.clone(), S0.clone()
    gdn.gdn_decode_step_fused(torch.empty((0, C), device=d, dtype=torch.bfloat16), cs,
                              W.uniform((C, 4), 21, 3, -0.5, 0.5).to(d), ab, ab, A_log, dt_bias, fs, nk, cu_seqlens=cu)
    torch.cuda.synchronize()
    assert o.shape[0] == 0 and o2.shape[0] == 0
    for t, nm in ((st, "chunk final state"), (st2, "gated chunk final state"), (rs, "recurrent state"),
                  (fs, "fused decode state")):
        assert torch.equal(t, S0), f"{nm} changed without tokens"
    assert torch.equal(cs, cs0), "conv state changed without tokens"


def test_chunk_more_than_65536_chunks():
    """A call of more than 65536 chunks (one sequence of 4.19 M tokens, 1 -> 2 heads): its last tokens and
    final state equal, bit for bit, a second call over those tokens started from the state a first call
    leaves at a chunk boundary (no part of the long call is dropped or repeated)."""
    T0 = 65536 * 64 - 64
    T = T0 + 164
    _say("chunk call over", T, "tokens,", (T + 63) // 64, "chunks")
    D = dev()
    q = W.randn((T, 1, 128), 77, 1, "bf16", device=D)
    k = W.randn((T, 1, 128), 77, 2, "bf16", device=D)
    v = W.randn((T, 2, 128), 77, 3, "bf16", device=D)
    a = W.randn((T, 2), 77, 4, "bf16", device=D)
    b = W.randn((T, 2), 77, 5, "bf16", device=D)
    A_log = W.a_log(2, 77, D)
    dt_bias = W.randn((2,), 77, 7, "f32", std=0.1, device=D)
    o_all, s_all = gdn.gdn_chunk_fwd_gated(q, k, v, a, b, A_log, dt_bias)
    _, s_mid = gdn.gdn_chunk_fwd_gated(q[:T0], k[:T0], v[:T0], a[:T0], b[:T0], A_log, dt_bias)
    o_tail, s_tail = gdn.gdn_chunk_fwd_gated(q[T0:], k[T0:], v[T0:], a[T0:].contiguous(), b[T0:].contiguous(),
                                             A_log, dt_bias, initial_state=s_mid)
    torch.cuda.synchronize()
    assert torch.equal(o_tail, o_all[T0:]), "last tokens of the long call"
    assert torch.equal(s_tail, s_all), "final state of the long call"
    assert torch.isfinite(o_all[::4096]).all()
