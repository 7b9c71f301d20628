"""Pins of the fp64 CPU oracle against facts fixed by the pages and by mathematics.

Nothing here compares the oracle with a retyped copy of itself: each check is a
hand-derived golden value (tests/golden/, each citing its passage), a closed
form, an invariant, a library routine for a special case, or a different
algorithm (the chunk-parallel form, the explicit product form) that must reach
the same result.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle.chunk_form import chunk_delta_rule

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def _rand_core(rng, T, nk, nv, dk, dv, s0=False, g_scale=1.0):
    q = rng.standard_normal((T, nk, dk))
    k = rng.standard_normal((T, nk, dk))
    v = rng.standard_normal((T, nv, dv))
    g = -g_scale * rng.uniform(0.0, 1.0, (T, nv))
    beta = rng.uniform(0.05, 0.95, (T, nv))
    S0 = rng.standard_normal((1, nv, dk, dv)) * 0.3 if s0 else None
    return q, k, v, g, beta, S0


# ---------------------------------------------------------------- golden values

def test_golden_delta_rule_hand_example():
    d = _gold("delta_rule_dk2_dv3.json")
    q = np.array(d["q"])[:, None, :]
    k = np.array(d["k"])[:, None, :]
    v = np.array(d["v"])[:, None, :]
    g = np.log(np.array(d["exp_g"]))[:, None]
    beta = np.array(d["beta"])[:, None]
    S0 = np.array(d["S0"])[None, None]
    o, ST = oracle.delta_rule(q, k, v, g, beta, initial_state=S0, scale=d["scale"], l2norm=False)
    np.testing.assert_allclose(o[:, 0], np.array(d["o"]), rtol=0, atol=1e-14)
    np.testing.assert_allclose(ST[0, 0], np.array(d["ST"]), rtol=0, atol=1e-14)


def test_golden_l2norm_one_token():
    d = _gold("delta_rule_l2norm_one_token.json")
    q = np.array(d["q"])[:, None, :]
    k = np.array(d["k"])[:, None, :]
    v = np.array(d["v"])[:, None, :]
    o, ST = oracle.delta_rule(q, k, v, np.array(d["g"])[:, None], np.array(d["beta"])[:, None],
                              eps=d["eps"], l2norm=True)
    np.testing.assert_allclose(o[:, 0], np.array(d["o"]), rtol=1e-15, atol=1e-15)
    np.testing.assert_allclose(ST[0, 0], np.array(d["ST"]), rtol=1e-15, atol=1e-15)


def test_golden_gating_points():
    d = _gold("gating_points.json")
    for c in d["cases"]:
        g, beta = oracle.gating([[c["a"]]], [[c["b"]]], [c["A_log"]], [c["dt_bias"]])
        assert g[0, 0] == pytest.approx(c["g"], rel=1e-15, abs=1e-15)
        assert beta[0, 0] == pytest.approx(c["beta"], rel=1e-15)


def test_golden_conv_impulse_and_ones():
    d = _gold("conv_impulse.json")
    w = np.array([d["w"]], dtype=np.float64)
    for xk, yk in (("x_impulse", "y_impulse"), ("x_ones", "y_ones")):
        x = np.array(d[xk], dtype=np.float64)[:, None]
        y, _ = oracle.causal_conv1d(x, w, silu=False)
        np.testing.assert_array_equal(y[:, 0], np.array(d[yk], dtype=np.float64))


def test_golden_gated_rmsnorm_row():
    d = _gold("gated_rmsnorm_row.json")
    y = oracle.gated_rmsnorm(np.array([d["x"]]), np.array([d["z"]]), np.array(d["w"]), eps=d["eps"])
    np.testing.assert_allclose(y[0], np.array(d["y"]), rtol=1e-14)


# ---------------------------------------------------------------- gating

def test_gating_special_cases_and_ranges():
    rng = np.random.default_rng(11)
    T, nv = 257, 5
    a = rng.standard_normal((T, nv)) * 4
    b = rng.standard_normal((T, nv)) * 4
    A_log = np.log(rng.uniform(1, 16, nv))
    dt = rng.standard_normal(nv) * 0.1
    g, beta = oracle.gating(a, b, A_log, dt)
    # beta is the logistic function (library routine)
    from scipy.special import expit
    np.testing.assert_allclose(beta, expit(b), rtol=1e-15)
    # softplus = log(1 + e^s) = logaddexp(0, s) (library routine)
    np.testing.assert_allclose(g, -np.exp(A_log) * np.logaddexp(0.0, a + dt), rtol=1e-14)
    assert np.all(g < 0) and np.all((beta > 0) & (beta < 1))
    # A_log = 0 -> g = -softplus(a + dt_bias)
    g0, _ = oracle.gating(a, b, np.zeros(nv), dt)
    np.testing.assert_allclose(g0, -np.logaddexp(0.0, a + dt), rtol=1e-14)
    # large argument: softplus(s) -> s, so g -> -exp(A_log) * s
    gl, _ = oracle.gating(np.full((1, 1), 60.0), np.zeros((1, 1)), [math.log(3.0)], [0.0])
    assert gl[0, 0] == pytest.approx(-180.0, rel=1e-15)
    # very negative argument: softplus(s) -> e^s
    gs, _ = oracle.gating(np.full((1, 1), -40.0), np.zeros((1, 1)), [0.0], [0.0])
    assert gs[0, 0] == pytest.approx(-math.exp(-40.0), rel=1e-12)


# ---------------------------------------------------------------- core closed forms

@pytest.mark.parametrize("dk,dv", [(4, 3), (8, 8)])
def test_core_single_token_closed_form(dk, dv):
    rng = np.random.default_rng(1)
    q, k, v, g, beta, _ = _rand_core(rng, 1, 1, 1, dk, dv)
    scale = 0.37
    o, ST = oracle.delta_rule(q, k, v, g, beta, scale=scale, eps=0.0)
    kh = k[0, 0] / np.linalg.norm(k[0, 0])
    qh = q[0, 0] / np.linalg.norm(q[0, 0]) * scale
    np.testing.assert_allclose(ST[0, 0], beta[0, 0] * np.outer(kh, v[0, 0]), rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(o[0, 0], beta[0, 0] * (kh @ qh) * v[0, 0], rtol=1e-12, atol=1e-15)


def test_core_beta_zero_is_pure_decay():
    rng = np.random.default_rng(2)
    T, dk, dv = 37, 6, 5
    q, k, v, g, beta, S0 = _rand_core(rng, T, 1, 1, dk, dv, s0=True)
    beta[:] = 0.0
    o, ST = oracle.delta_rule(q, k, v, g, beta, initial_state=S0, eps=0.0)
    G = np.cumsum(g[:, 0])
    qh = q[:, 0] / np.linalg.norm(q[:, 0], axis=1, keepdims=True) * dk ** -0.5
    for t in range(T):
        np.testing.assert_allclose(o[t, 0], math.exp(G[t]) * S0[0, 0].T @ qh[t], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(ST[0, 0], math.exp(G[-1]) * S0[0, 0], rtol=1e-12)


def test_core_reset_forgets_history():
    rng = np.random.default_rng(3)
    T, dk, dv = 20, 5, 7
    q, k, v, g, beta, S0 = _rand_core(rng, T, 1, 1, dk, dv, s0=True)
    g[:] = -1e4  # exp(-1e4) underflows to exactly 0
    o, ST = oracle.delta_rule(q, k, v, g, beta, initial_state=S0, eps=0.0)
    kh = k[:, 0] / np.linalg.norm(k[:, 0], axis=1, keepdims=True)
    qh = q[:, 0] / np.linalg.norm(q[:, 0], axis=1, keepdims=True) * dk ** -0.5
    for t in range(T):
        ref = beta[t, 0] * (kh[t] @ qh[t]) * v[t, 0]
        np.testing.assert_allclose(o[t, 0], ref, rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(ST[0, 0], beta[-1, 0] * np.outer(kh[-1], v[-1, 0]), rtol=1e-13, atol=1e-16)


def test_core_orthonormal_keys_write_values_exactly():
    rng = np.random.default_rng(4)
    dk, dv, T = 16, 9, 12
    Qm, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
    keys = Qm[:T]                      # orthonormal rows
    v = rng.standard_normal((T, 1, dv))
    S0 = rng.standard_normal((1, 1, dk, dv))
    k = keys[:, None, :]
    q = keys[:, None, :].copy()        # read back with the key just written
    g = np.zeros((T, 1)); beta = np.ones((T, 1))
    scale = 0.5
    o, ST = oracle.delta_rule(q, k, v, g, beta, initial_state=S0, scale=scale, l2norm=False)
    np.testing.assert_allclose(o[:, 0], scale * v[:, 0], rtol=0, atol=1e-13)
    # and every value stays retrievable after all later writes
    np.testing.assert_allclose(keys @ ST[0, 0], v[:, 0], rtol=0, atol=1e-13)


def test_core_fixed_point():
    rng = np.random.default_rng(5)
    dk, dv = 6, 4
    S0 = rng.standard_normal((1, 1, dk, dv))
    k = rng.standard_normal((1, 1, dk)); q = rng.standard_normal((1, 1, dk))
    g = np.array([[-0.3]]); beta = np.array([[0.7]])
    kh = k[0, 0] / np.linalg.norm(k[0, 0])
    v = (math.exp(-0.3) * S0[0, 0].T @ kh)[None, None, :]   # v = e^g S^T k
    _, ST = oracle.delta_rule(q, k, v, g, beta, initial_state=S0, eps=0.0)
    np.testing.assert_allclose(ST[0, 0], math.exp(-0.3) * S0[0, 0], rtol=1e-13, atol=1e-15)


def test_core_product_form_brute_force():
    """S_T = A_T ... A_1 S_0 + sum_t A_T..A_{t+1} B_t with A_t = e^g (I - beta k k^T), B_t = beta k v^T."""
    rng = np.random.default_rng(6)
    dk, dv = 5, 3
    for T in range(1, 9):
        q, k, v, g, beta, S0 = _rand_core(rng, T, 1, 1, dk, dv, s0=True)
        o, ST = oracle.delta_rule(q, k, v, g, beta, initial_state=S0, eps=0.0, scale=1.0)
        kh = k[:, 0] / np.linalg.norm(k[:, 0], axis=1, keepdims=True)
        qh = q[:, 0] / np.linalg.norm(q[:, 0], axis=1, keepdims=True)
        S = S0[0, 0].copy()
        for t in range(T):
            A = math.exp(g[t, 0]) * (np.eye(dk) - beta[t, 0] * np.outer(kh[t], kh[t]))
            S = A @ S + beta[t, 0] * np.outer(kh[t], v[t, 0])
            np.testing.assert_allclose(o[t, 0], S.T @ qh[t], rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(ST[0, 0], S, rtol=1e-12, atol=1e-14)


# ---------------------------------------------------------------- core invariants

def test_core_linear_in_values_and_state():
    rng = np.random.default_rng(7)
    T, dk, dv = 30, 6, 4
    q, k, v1, g, beta, S1 = _rand_core(rng, T, 1, 2, dk, dv, s0=True)
    v2 = rng.standard_normal(v1.shape); S2 = rng.standard_normal(S1.shape)
    al = -1.7
    o1, s1 = oracle.delta_rule(q, k, v1, g, beta, initial_state=S1)
    o2, s2 = oracle.delta_rule(q, k, v2, g, beta, initial_state=S2)
    o3, s3 = oracle.delta_rule(q, k, al * v1 + v2, g, beta, initial_state=al * S1 + S2)
    np.testing.assert_allclose(o3, al * o1 + o2, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(s3, al * s1 + s2, rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("split", [1, 63, 64, 100])
def test_core_split_run_equals_single_run(split):
    rng = np.random.default_rng(8)
    T, dk, dv = 150, 8, 5
    q, k, v, g, beta, S0 = _rand_core(rng, T, 1, 2, dk, dv, s0=True)
    o, ST = oracle.delta_rule(q, k, v, g, beta, initial_state=S0)
    oa, Sa = oracle.delta_rule(q[:split], k[:split], v[:split], g[:split], beta[:split], initial_state=S0)
    ob, Sb = oracle.delta_rule(q[split:], k[split:], v[split:], g[split:], beta[split:], initial_state=Sa)
    np.testing.assert_array_equal(np.concatenate([oa, ob]), o)
    np.testing.assert_array_equal(Sb, ST)


def test_core_varlen_equals_separate_runs():
    rng = np.random.default_rng(9)
    lens = [5, 64, 1, 130, 77]
    T = sum(lens)
    dk, dv, nk, nv = 8, 4, 2, 4
    q, k, v, g, beta, _ = _rand_core(rng, T, nk, nv, dk, dv)
    S0 = rng.standard_normal((len(lens), nv, dk, dv))
    cu = np.concatenate([[0], np.cumsum(lens)])
    o, ST = oracle.delta_rule(q, k, v, g, beta, cu_seqlens=cu, initial_state=S0)
    for n in range(len(lens)):
        s = slice(cu[n], cu[n + 1])
        on, Sn = oracle.delta_rule(q[s], k[s], v[s], g[s], beta[s], initial_state=S0[n:n + 1])
        np.testing.assert_array_equal(o[s], on)
        np.testing.assert_array_equal(ST[n], Sn[0])


def test_core_head_repeat_equals_explicit_copy():
    rng = np.random.default_rng(10)
    T, dk, dv, nk, nv = 40, 8, 4, 2, 6
    q, k, v, g, beta, _ = _rand_core(rng, T, nk, nv, dk, dv)
    o, ST = oracle.delta_rule(q, k, v, g, beta)
    r = nv // nk
    qr, kr = np.repeat(q, r, axis=1), np.repeat(k, r, axis=1)   # repeat_interleave
    o2, ST2 = oracle.delta_rule(qr, kr, v, g, beta)
    np.testing.assert_array_equal(o, o2)
    np.testing.assert_array_equal(ST, ST2)
    # value head h must read key head h // r (not h % nk)
    o3, _ = oracle.delta_rule(np.tile(q, (1, r, 1)), np.tile(k, (1, r, 1)), v, g, beta)
    assert not np.allclose(o3, o)


def test_core_head_permutation_permutes_outputs():
    rng = np.random.default_rng(12)
    T, dk, dv, nh = 33, 6, 5, 4
    q, k, v, g, beta, _ = _rand_core(rng, T, nh, nh, dk, dv)
    perm = np.array([2, 0, 3, 1])
    o, ST = oracle.delta_rule(q, k, v, g, beta)
    op, STp = oracle.delta_rule(q[:, perm], k[:, perm], v[:, perm], g[:, perm], beta[:, perm])
    np.testing.assert_array_equal(op, o[:, perm])
    np.testing.assert_array_equal(STp[:, :], ST[:, perm])


def test_core_qk_scale_invariance():
    rng = np.random.default_rng(13)
    T, dk, dv = 25, 8, 4
    q, k, v, g, beta, _ = _rand_core(rng, T, 1, 1, dk, dv)
    o, _ = oracle.delta_rule(q, k, v, g, beta, eps=0.0)
    o2, _ = oracle.delta_rule(3.5 * q, 0.25 * k, v, g, beta, eps=0.0)
    np.testing.assert_allclose(o2, o, rtol=1e-12, atol=1e-14)


def test_core_state_norm_bound():
    # e^g (I - beta k k^T) has spectral norm <= 1, so ||S_t|| <= ||S_0|| + sum beta ||v||
    rng = np.random.default_rng(14)
    T, dk, dv = 60, 8, 8
    q, k, v, g, beta, S0 = _rand_core(rng, T, 1, 1, dk, dv, s0=True, g_scale=0.01)
    bound = np.linalg.norm(S0[0, 0])
    for t in range(1, T + 1):
        _, S = oracle.delta_rule(q[:t], k[:t], v[:t], g[:t], beta[:t], initial_state=S0)
        bound += beta[t - 1, 0] * np.linalg.norm(v[t - 1, 0])
        assert np.linalg.norm(S[0, 0]) <= bound * (1 + 1e-12)


# ---------------------------------------------------------------- chunk form agreement

@pytest.mark.parametrize("case", [
    dict(lens=[256], nk=1, nv=2, dk=16, dv=8, s0=False),
    dict(lens=[200], nk=2, nv=4, dk=8, dv=12, s0=True),
    dict(lens=[1, 63, 64, 65, 130], nk=1, nv=2, dk=8, dv=8, s0=True),
])
def test_chunk_form_equals_recurrence(case):
    rng = np.random.default_rng(15)
    lens = case["lens"]
    T = sum(lens)
    q, k, v, g, beta, _ = _rand_core(rng, T, case["nk"], case["nv"], case["dk"], case["dv"], g_scale=3.0)
    n = len(lens)
    S0 = rng.standard_normal((n, case["nv"], case["dk"], case["dv"])) if case["s0"] else None
    cu = np.concatenate([[0], np.cumsum(lens)])
    o, ST = oracle.delta_rule(q, k, v, g, beta, cu_seqlens=cu, initial_state=S0)
    oc, STc = chunk_delta_rule(q, k, v, g, beta, cu_seqlens=cu, initial_state=S0)
    rms = np.sqrt(np.mean(o ** 2))
    assert np.max(np.abs(oc - o)) <= 1e-11 * rms
    assert np.max(np.abs(STc - ST)) <= 1e-11 * np.sqrt(np.mean(ST ** 2))


def test_chunk_form_with_config_like_decay():
    """Fast decay (|G| ~ 1e2..1e3 inside a chunk) exercised at config-like gating."""
    rng = np.random.default_rng(16)
    T, dk, dv = 192, 16, 8
    q = rng.standard_normal((T, 1, dk)); k = rng.standard_normal((T, 1, dk))
    v = rng.standard_normal((T, 2, dv))
    a = rng.standard_normal((T, 2)); b = rng.standard_normal((T, 2))
    g, beta = oracle.gating(a, b, np.log([1.0, 16.0]), [0.05, -0.1])
    o, ST = oracle.delta_rule(q, k, v, g, beta)
    oc, STc = chunk_delta_rule(q, k, v, g, beta)
    assert np.max(np.abs(oc - o)) <= 1e-11 * np.sqrt(np.mean(o ** 2))


# ---------------------------------------------------------------- conv

def _torch_conv(x, w, bias=None, silu=True):
    # depthwise causal conv via the library routine (cross-correlation, left pad K-1)
    T, C = x.shape
    K = w.shape[1]
    xt = torch.from_numpy(x.T[None].copy())
    wt = torch.from_numpy(w[:, None, :].copy())
    bt = None if bias is None else torch.from_numpy(bias)
    y = torch.nn.functional.conv1d(xt, wt, bt, padding=K - 1, groups=C)[..., :T]
    if silu:
        y = torch.nn.functional.silu(y)
    return y[0].T.numpy()


def test_conv_matches_library_routine():
    rng = np.random.default_rng(17)
    T, C, K = 50, 12, 4
    x = rng.standard_normal((T, C)); w = rng.uniform(-0.5, 0.5, (C, K)); b = rng.standard_normal(C)
    for bias in (None, b):
        for silu in (False, True):
            y, _ = oracle.causal_conv1d(x, w, bias, silu=silu)
            np.testing.assert_allclose(y, _torch_conv(x, w, bias, silu), rtol=1e-13, atol=1e-14)


def test_conv_with_initial_state_equals_conv_of_concatenation():
    rng = np.random.default_rng(18)
    T, C, K, L = 9, 6, 4, 5
    x = rng.standard_normal((T, C)); w = rng.uniform(-0.5, 0.5, (C, K))
    st = rng.standard_normal((1, C, L))
    y, so = oracle.causal_conv1d(x, w, conv_state=st)
    full = np.concatenate([st[0].T, x])          # [L + T, C]
    yref = _torch_conv(full, w)[L:]
    np.testing.assert_allclose(y, yref, rtol=1e-13, atol=1e-14)
    np.testing.assert_array_equal(so[0], full[-L:].T)
    # a sequence shorter than the state keeps part of the old state
    y2, so2 = oracle.causal_conv1d(x[:2], w, conv_state=st)
    np.testing.assert_array_equal(so2[0], np.concatenate([st[0].T, x[:2]])[-L:].T)


def test_conv_varlen_equals_separate():
    rng = np.random.default_rng(19)
    lens = [3, 1, 10, 4]
    T, C, K = sum(lens), 5, 4
    x = rng.standard_normal((T, C)); w = rng.uniform(-0.5, 0.5, (C, K))
    st = rng.standard_normal((len(lens), C, 3))
    cu = np.concatenate([[0], np.cumsum(lens)])
    y, so = oracle.causal_conv1d(x, w, cu_seqlens=cu, conv_state=st)
    for n in range(len(lens)):
        yn, sn = oracle.causal_conv1d(x[cu[n]:cu[n + 1]], w, conv_state=st[n:n + 1])
        np.testing.assert_array_equal(y[cu[n]:cu[n + 1]], yn)
        np.testing.assert_array_equal(so[n], sn[0])


@pytest.mark.parametrize("state_len", [3, 4])
def test_conv_update_steps_equal_prefill(state_len):
    rng = np.random.default_rng(20)
    T, C, K, n = 7, 8, 4, 3
    x = rng.standard_normal((n, T, C)); w = rng.uniform(-0.5, 0.5, (C, K)); b = rng.standard_normal(C)
    st0 = rng.standard_normal((n, C, state_len))
    st = st0.copy()
    ys = []
    for t in range(T):
        y, st_new = oracle.causal_conv1d_update(x[:, t], st, w, b)
        # the state shift is an exact copy
        np.testing.assert_array_equal(st_new[:, :, :-1], st[:, :, 1:])
        np.testing.assert_array_equal(st_new[:, :, -1], x[:, t])
        st = st_new
        ys.append(y)
    ys = np.stack(ys, axis=1)
    cu = np.arange(n + 1) * T
    yp, sp = oracle.causal_conv1d(x.reshape(n * T, C), w, b, cu_seqlens=cu, conv_state=st0)
    np.testing.assert_allclose(ys.reshape(n * T, C), yp, rtol=1e-14, atol=1e-15)
    np.testing.assert_array_equal(st, sp)


# ---------------------------------------------------------------- gated RMSNorm

def test_gated_rmsnorm_matches_library_rms_norm():
    rng = np.random.default_rng(21)
    rows, D = 40, 128
    x = rng.standard_normal((rows, D)); z = rng.standard_normal((rows, D)); w = rng.normal(0, 0.1, D)
    for ww in (np.zeros(D), w):
        y = oracle.gated_rmsnorm(x, z, ww, eps=1e-6)
        ref = torch.nn.functional.rms_norm(torch.from_numpy(x), (D,), eps=1e-6).numpy()
        ref = ref * (1.0 + ww) * torch.nn.functional.silu(torch.from_numpy(z)).numpy()
        np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-14)


def test_gated_rmsnorm_constant_row():
    D, eps = 16, 1e-6
    for c in (2.0, -0.5, 1e-3):
        x = np.full((1, D), c); z = np.full((1, D), 50.0)   # silu(50) = 50 (to 1e-21)
        y = oracle.gated_rmsnorm(x, z, np.zeros(D), eps=eps)
        np.testing.assert_allclose(y[0], np.sign(c) / math.sqrt(1 + eps / c ** 2) * 50.0, rtol=1e-13)


def test_oracle_rejects_invalid_arguments():
    q = np.zeros((4, 2, 8)); v = np.zeros((4, 3, 8)); g = np.zeros((4, 3))
    with pytest.raises(ValueError):   # nv % nk != 0
        oracle.delta_rule(q, q, v, g, g)
    with pytest.raises(ValueError):   # cu_seqlens does not end at T
        oracle.delta_rule(q[:, :1], q[:, :1], v, g, g, cu_seqlens=[0, 2, 3])
    with pytest.raises(ValueError):   # state_len < K - 1
        oracle.causal_conv1d(np.zeros((4, 2)), np.zeros((2, 4)), state_len=2)
