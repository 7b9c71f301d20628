"""Full-size parity of the five workloads against the fp64 CPU oracle.

Each workload runs on the GPU exactly as the benchmark launches it (the
binding's defaults). Checks:
  * tiny chunk fp32 (T=256, 1->2 heads) and prefill T=8192 (16->32 heads):
    every output and final state against the oracle, and the benchmark's
    gated chunk call equal to gating + chunk bit for bit;
  * varlen packed prefill (8 sequences, nonzero initial states): every head
    of every sequence;
  * decode step (256 sequences, 512 MiB state in place): stage-wise --
    conv update (fp32-accumulation + one bf16 rounding bound, state exact),
    then gating + recurrent update
    from the GPU's own bf16 conv output, every unit;
  * long fused prefill (T=262144, 16->64 heads): stage-wise on samples the
    oracle can compute -- conv on three token windows of all channels, gating
    on every 61st token, the core on 16 value heads (one per key head, each
    of the four positions inside a key head four times) over the full
    sequence, for both the separate launches and the fused prefill (outputs
    and final state), gated RMSNorm on every 257th token and on a contiguous
    block of 4096 tokens (all heads).
Parity bar: max-abs <= 2e-3 * RMS for bf16 inputs, 1e-5 * RMS for fp32.
"""
import os

import numpy as np
import pytest
import torch

import gated_deltanet_gdn_amd as gdn
import oracle
import workloads as W
from gpu_common import TOL, assert_close, assert_conv_close, conv_abs_sum, dev, f64

pytestmark = pytest.mark.gpu
THREADS = min(16, os.cpu_count() or 1)


def _say(*a):
    print("[case]", *a, flush=True)


def _chunk_config(name):
    wl = W.WORKLOADS[name]
    _say(name, "generate")
    x = W.chunk_inputs(wl)
    d = {k: (v.to(dev()) if isinstance(v, torch.Tensor) else v) for k, v in x.items()}
    _say(name, "gpu", "T =", int(x["cu_seqlens"][-1]))
    cu = d["cu_seqlens"] if wl.len_range else None
    g, beta = gdn.gdn_gating(d["a"], d["b"], d["A_log"], d["dt_bias"])
    o, st = gdn.gdn_chunk_fwd(d["q"], d["k"], d["v"], g, beta, cu_seqlens=cu, initial_state=d["S0"])
    # the benchmark's entry point (gating folded into the chunk call) gives the same bits
    o2, st2 = gdn.gdn_chunk_fwd_gated(d["q"], d["k"], d["v"], d["a"], d["b"], d["A_log"], d["dt_bias"],
                                      cu_seqlens=cu, initial_state=d["S0"])
    torch.cuda.synchronize()
    assert torch.equal(o2, o) and torch.equal(st2, st), f"{name}: gated call differs from gating + chunk"
    _say(name, "oracle")
    g_ref, b_ref = oracle.gating(f64(x["a"]), f64(x["b"]), f64(x["A_log"]), f64(x["dt_bias"]))
    o_ref, s_ref = oracle.delta_rule(f64(x["q"]), f64(x["k"]), f64(x["v"]), g_ref, b_ref,
                                     cu_seqlens=x["cu_seqlens"].numpy(),
                                     initial_state=None if x["S0"] is None else f64(x["S0"]), threads=THREADS)
    return wl, o, st, o_ref, s_ref


@pytest.mark.parametrize("name", ["tiny_chunk_f32", "prefill_chunk_t8k", "varlen_prefill_8seq"])
def test_chunk_workload(name):
    wl, o, st, o_ref, s_ref = _chunk_config(name)
    tol = TOL[wl.dtype]
    assert_close(o, o_ref, tol, f"{name} o")
    assert_close(st, s_ref, tol, f"{name} final state")
    # worst head, for the log
    per_head = [np.max(np.abs(f64(o[:, h]) - o_ref[:, h])) / np.sqrt(np.mean(o_ref[:, h] ** 2))
                for h in range(o.shape[1])]
    print(f"[parity] {name} worst head ratio {max(per_head):.3e} (head {int(np.argmax(per_head))})", flush=True)


def test_decode_step_workload():
    wl = W.WORKLOADS["decode_256seq"]
    _say(wl.name, "generate")
    x = W.decode_inputs(wl)
    d = {k: v.to(dev()) for k, v in x.items()}
    n, C = x["x"].shape
    kd = wl.nk * wl.dk
    _say(wl.name, "gpu")
    conv_state = d["conv_state"].clone()
    y = gdn.gdn_causal_conv1d_update(d["x"], conv_state, d["conv_w"])
    q = y[:, :kd].view(n, wl.nk, wl.dk)
    k = y[:, kd:2 * kd].view(n, wl.nk, wl.dk)
    v = y[:, 2 * kd:].view(n, wl.nv, wl.dv)
    g, beta = gdn.gdn_gating(d["a"], d["b"], d["A_log"], d["dt_bias"])
    state = d["state"].clone()
    o = gdn.gdn_recurrent_fwd(q, k, v, g, beta, state)
    torch.cuda.synchronize()

    _say(wl.name, "oracle: conv update")
    y_ref, cs_ref = oracle.causal_conv1d_update(f64(x["x"]), f64(x["conv_state"]), f64(x["conv_w"]))
    win = np.concatenate([f64(x["conv_state"]), f64(x["x"])[:, :, None]], axis=2)     # [n, C, 4]
    s_abs = np.sum(np.abs(win) * np.abs(f64(x["conv_w"]))[None], axis=2)
    assert_conv_close(y, y_ref, s_abs, "decode conv update")
    np.testing.assert_array_equal(f64(conv_state), cs_ref)

    _say(wl.name, "oracle: recurrent on the GPU's conv output")
    yg = f64(y)
    g_ref, b_ref = oracle.gating(f64(x["a"]), f64(x["b"]), f64(x["A_log"]), f64(x["dt_bias"]))
    o_ref, s_ref = oracle.delta_rule(yg[:, :kd].reshape(n, wl.nk, wl.dk), yg[:, kd:2 * kd].reshape(n, wl.nk, wl.dk),
                                     yg[:, 2 * kd:].reshape(n, wl.nv, wl.dv), g_ref, b_ref,
                                     cu_seqlens=np.arange(n + 1), initial_state=f64(x["state"]), threads=THREADS)
    assert_close(o, o_ref, TOL["bf16"], "decode o")
    assert_close(state, s_ref, TOL["bf16"], "decode state")


# ------------------------------------------------------------------ long fused prefill

@pytest.fixture(scope="module")
def long_run():
    wl = W.WORKLOADS["long_fused_t256k"]
    D = dev()
    _say(wl.name, "generate on the GPU")
    x = W.fused_inputs(wl, device=D)
    T, C = x["x"].shape
    kd = wl.nk * wl.dk
    _say(wl.name, "gpu pipeline")
    y, cs = gdn.gdn_causal_conv1d(x["x"], x["conv_w"], state_len=wl.state_len)
    q = y[:, :kd].view(T, wl.nk, wl.dk)
    k = y[:, kd:2 * kd].view(T, wl.nk, wl.dk)
    v = y[:, 2 * kd:].view(T, wl.nv, wl.dv)
    g, beta = gdn.gdn_gating(x["a"], x["b"], x["A_log"], x["dt_bias"])
    o, st = gdn.gdn_chunk_fwd(q, k, v, g, beta)
    out = gdn.gdn_gated_rmsnorm(o, x["z"], x["norm_w"], eps=1e-6)
    _say(wl.name, "gpu fused prefill")
    fo, fst, fcs = gdn.gdn_prefill_fused(x["x"], x["conv_w"], x["a"], x["b"], x["A_log"], x["dt_bias"], wl.nk, wl.nv,
                                         state_len=wl.state_len)
    _say(wl.name, "gpu fused prefill with the norm")
    ny, nst, _ = gdn.gdn_prefill_fused_norm(x["x"], x["conv_w"], x["a"], x["b"], x["A_log"], x["dt_bias"], wl.nk,
                                            wl.nv, x["z"], x["norm_w"], eps=1e-6, state_len=wl.state_len,
                                            output_conv_state=False)
    torch.cuda.synchronize()
    return dict(wl=wl, x=x, y=y, cs=cs, g=g, beta=beta, o=o, st=st, out=out, T=T, C=C, kd=kd, fo=fo, fst=fst,
                fcs=fcs, ny=ny, nst=nst)


def test_long_prefill_fused_equals_pipeline(long_run):
    """The fused prefill (conv applied inside the chunk kernels) reproduces the separate conv, gating and
    chunk launches bit for bit on the full long workload."""
    r = long_run
    wl, x = r["wl"], r["x"]
    _say(wl.name, "fused prefill against the separate launches")
    for a, b, what in ((r["fo"], r["o"], "o"), (r["fst"], r["st"], "final state"), (r["fcs"], r["cs"], "conv state out")):
        diff = (a.double() - b.double()).abs().max().item()
        print(f"[exact] {what}: max |fused - separate| = {diff:.3e}", flush=True)
        assert torch.equal(a, b), what


def test_long_prefill_fused_norm_equals_pipeline(long_run):
    """The fused prefill with the norm inside the state kernel against the fused prefill followed by the
    norm launch on the full long workload: final state bit for bit; y within 2e-5 of |y| per element (the
    two routes sum a row's 128 squares in different orders, at most 2 * 127 u apart, which moves rms^-1 by
    half of that), and not bit-equal everywhere, which shows the in-kernel route ran."""
    r = long_run
    _say(r["wl"].name, "fused prefill with the norm against the two launches")
    assert torch.equal(r["nst"], r["fst"]), "final state"
    ny, out = r["ny"], r["out"]
    worst = 0.0
    for t0 in range(0, r["T"], 16384):   # in slabs, to bound the temporaries
        a, b = ny[t0:t0 + 16384].double(), out[t0:t0 + 16384].double()
        err = (a - b).abs()
        worst = max(worst, (err / b.abs().clamp_min(1e-30)).max().item())
        assert (err <= 2e-5 * b.abs()).all(), f"y beyond 2e-5 of |ref| in tokens {t0}.."
    print(f"[tol] y: max |fused - pipeline| / |pipeline| = {worst:.3e}", flush=True)
    assert not torch.equal(ny, out), "the norm did not run inside the state kernel"


def test_long_conv_windows(long_run):
    r = long_run
    T = r["T"]
    for t0, t1 in ((0, 2048), (T // 2 - 1000, T // 2 + 1048), (T - 2048, T)):
        _say("long conv window", t0, t1)
        lo = max(t0 - 3, 0)
        xs = f64(r["x"]["x"][lo:t1])
        y_ref, _ = oracle.causal_conv1d(xs, f64(r["x"]["conv_w"]))
        xe = np.concatenate([np.zeros((3 - (t0 - lo), xs.shape[1])), xs])
        s_abs = conv_abs_sum(xe, f64(r["x"]["conv_w"]))          # outputs for tokens t0 .. t1-1
        assert_conv_close(r["y"][t0:t1], y_ref[t0 - lo:], s_abs, f"long conv [{t0},{t1})")
    np.testing.assert_array_equal(f64(r["cs"][0]), f64(r["x"]["x"][T - 3:]).T)


def test_long_gating_sampled(long_run):
    r = long_run
    idx = torch.arange(0, r["T"], 61, device=r["g"].device)
    g_ref, b_ref = oracle.gating(f64(r["x"]["a"][idx]), f64(r["x"]["b"][idx]), f64(r["x"]["A_log"]),
                                 f64(r["x"]["dt_bias"]))
    np.testing.assert_allclose(f64(r["g"][idx]), g_ref, rtol=4e-6)
    np.testing.assert_allclose(f64(r["beta"][idx]), b_ref, rtol=4e-6)


@pytest.fixture(scope="module")
def long_core_ref(long_run):
    """The oracle on 16 value heads of the long prefill over all 262,144 tokens, from the GPU's own conv
    output (stage-wise): one value head per key head, and the position inside the key head's group of
    four rotating, so every (key head, position) work-order case of the state kernel appears."""
    r = long_run
    wl = r["wl"]
    rr = wl.nv // wl.nk
    heads = [hk * rr + hk % rr for hk in range(wl.nk)]
    _say("long core heads", heads)
    yg = r["y"]
    kd = r["kd"]
    q = torch.stack([yg[:, hk * 128:(hk + 1) * 128] for hk in range(wl.nk)], 1)
    k = torch.stack([yg[:, kd + hk * 128:kd + (hk + 1) * 128] for hk in range(wl.nk)], 1)
    v = torch.stack([yg[:, 2 * kd + h * 128:2 * kd + (h + 1) * 128] for h in heads], 1)
    hs = torch.tensor(heads, device=yg.device)
    g_ref, b_ref = oracle.gating(f64(r["x"]["a"][:, hs]), f64(r["x"]["b"][:, hs]), f64(r["x"]["A_log"][hs]),
                                 f64(r["x"]["dt_bias"][hs]))
    # q/k of key head hk pair with value head heads[hk]: one key head per value head here
    o_ref, s_ref = oracle.delta_rule(f64(q), f64(k), f64(v), g_ref, b_ref, threads=THREADS)
    return heads, o_ref, s_ref


@pytest.mark.timeout(300)
def test_long_core_sixteen_heads_full_sequence(long_run, long_core_ref):
    r = long_run
    heads, o_ref, s_ref = long_core_ref
    for i, h in enumerate(heads):
        assert_close(r["o"][:, h], o_ref[:, i], TOL["bf16"], f"long o head {h}")
        assert_close(r["st"][0, h], s_ref[0, i], TOL["bf16"], f"long final state head {h}")


@pytest.mark.timeout(300)
def test_long_fused_prefill_sixteen_heads_against_oracle(long_run, long_core_ref):
    """The fused prefill's own outputs against the oracle on the same 16 heads (the oracle reads the
    separate conv's bf16 output, which the fused kernels reproduce bit for bit in registers)."""
    r = long_run
    heads, o_ref, s_ref = long_core_ref
    for i, h in enumerate(heads):
        assert_close(r["fo"][:, h], o_ref[:, i], TOL["bf16"], f"fused prefill o head {h}")
        assert_close(r["fst"][0, h], s_ref[0, i], TOL["bf16"], f"fused prefill final state head {h}")


def test_long_rmsnorm_sampled_rows(long_run):
    r = long_run
    rows = torch.arange(0, r["T"], 257, device=r["o"].device)
    x = r["o"][rows]              # [rows, 64, 128] fp32 from the GPU core (stage-wise)
    z = r["x"]["z"][rows]
    ref = oracle.gated_rmsnorm(f64(x), f64(z), f64(r["x"]["norm_w"]), eps=1e-6)
    assert_close(r["out"][rows], ref, TOL["f32"], "long gated rmsnorm (fp32 x)")


def test_long_rmsnorm_contiguous_block(long_run):
    r = long_run
    t0 = r["T"] // 2 + 123
    x = r["o"][t0:t0 + 4096]      # 4096 tokens x 64 heads of rows, contiguous
    ref = oracle.gated_rmsnorm(f64(x), f64(r["x"]["z"][t0:t0 + 4096]), f64(r["x"]["norm_w"]), eps=1e-6)
    assert_close(r["out"][t0:t0 + 4096], ref, TOL["f32"], "long gated rmsnorm, 4096 contiguous tokens")
