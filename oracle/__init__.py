"""fp64 CPU oracle for the Gated DeltaNet core -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package. The GPU library never imports, links or calls it, and
the two share no code: this package loads its own ``liboracle_gdn.so``
(compiled from ``gdn_oracle.cpp`` by ``oracle/build.py``) through ctypes.

All functions take and return numpy float64 arrays (inputs are converted with
``np.asarray(..., dtype=np.float64)``, which is exact for bf16/fp32 values).
The definitions follow the published pages (titles as printed):
  * "Qwen3.5 Dense Model Architecture" -- section "Linear Attention":
    gating formulas, repeat_interleave head map, decay + delta update state
    recurrence, cache shapes.
  * "Qwen3.5 Simulation Support Design Document" -- 1.1 (gated RMSNorm with
    1 + weight), 2.2 (decomposed op flow), 2.4 (conv body vs state update).
Readings where the pages are silent (scale 1/sqrt(Dk), eps = 1e-6 for the
L2 norm and RMSNorm, decay applied before the delta read, read-out after the
update) are listed at each function.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle_gdn.so")
_lib = None

_dp = ctypes.POINTER(ctypes.c_double)
_i64p = ctypes.POINTER(ctypes.c_int64)


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _b  # build on first use (CPU-only g++ step)
        _b.build()
    lib = ctypes.CDLL(_LIB_PATH)
    i64, i32, dbl = ctypes.c_int64, ctypes.c_int, ctypes.c_double
    lib.oracle_gating.argtypes = [i64, i32, _dp, _dp, _dp, _dp, _dp, _dp]
    lib.oracle_delta_rule.argtypes = [i64, i32, _i64p, i32, i32, i32, i32,
                                      _dp, _dp, _dp, _dp, _dp, dbl, i32, dbl,
                                      _dp, _dp, _dp, i32]
    lib.oracle_causal_conv1d.argtypes = [i64, i32, _i64p, i32, i32, i32,
                                         _dp, _dp, _dp, _dp, _dp, i32, _dp]
    lib.oracle_causal_conv1d_update.argtypes = [i32, i32, i32, i32,
                                                _dp, _dp, _dp, _dp, i32, _dp]
    lib.oracle_gated_rmsnorm.argtypes = [i64, i32, _dp, _dp, _dp, dbl, _dp]
    for f in ("oracle_gating", "oracle_delta_rule", "oracle_causal_conv1d",
              "oracle_causal_conv1d_update", "oracle_gated_rmsnorm"):
        getattr(lib, f).restype = ctypes.c_int
    _lib = lib
    return lib


def _f64(x):
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a):
    return None if a is None else a.ctypes.data_as(_dp)


def _cu(cu_seqlens, T_tot):
    if cu_seqlens is None:
        return None, 1
    cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int64))
    return cu, len(cu) - 1


def _check(rc, name):
    if rc != 0:
        raise ValueError(f"{name}: invalid argument (oracle returned {rc})")


def gating(a, b, A_log, dt_bias):
    """beta = sigmoid(b); g = -exp(A_log[h]) * softplus(a + dt_bias[h]).

    Follows the beta/g lines of the minimal forward example ("Qwen3.5 Dense
    Model Architecture", Linear Attention). a, b: [T, nv]; A_log, dt_bias:
    [nv]. Returns (g, beta) as [T, nv] float64.
    """
    a, b = _f64(a), _f64(b)
    A_log, dt_bias = _f64(A_log), _f64(dt_bias)
    T, nv = a.shape
    g = np.empty((T, nv)); beta = np.empty((T, nv))
    _check(_load().oracle_gating(T, nv, _ptr(a), _ptr(b), _ptr(A_log), _ptr(dt_bias),
                                 _ptr(g), _ptr(beta)), "gating")
    return g, beta


def delta_rule(q, k, v, g, beta, cu_seqlens=None, initial_state=None, scale=None,
               l2norm=True, eps=1e-6, output_final_state=True, threads=0):
    """Token-by-token gated delta rule (the definition the chunked form must match).

    q, k: [T, nk, dk]; v: [T, nv, dv]; g, beta: [T, nv]; cu_seqlens: [n+1] or
    None; initial_state: [n, nv, dk, dv] or None. scale defaults to dk**-0.5
    (reading: the pages print y = S q with no scale; the 1/sqrt(Dk) factor is
    the stated method's read-out scale). Returns (o [T, nv, dv], S_T or None).
    """
    q, k, v, g, beta = map(_f64, (q, k, v, g, beta))
    T, nk, dk = q.shape
    nv, dv = v.shape[1], v.shape[2]
    cu, n = _cu(cu_seqlens, T)
    if scale is None:
        scale = dk ** -0.5
    S0 = None if initial_state is None else _f64(initial_state)
    ST = np.empty((n, nv, dk, dv)) if output_final_state else None
    o = np.empty((T, nv, dv))
    rc = _load().oracle_delta_rule(T, n, None if cu is None else cu.ctypes.data_as(_i64p),
                                   nk, nv, dk, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                   float(scale), int(bool(l2norm)), float(eps),
                                   _ptr(S0), _ptr(ST), _ptr(o), int(threads))
    _check(rc, "delta_rule")
    return o, ST


def causal_conv1d(x, weight, bias=None, cu_seqlens=None, conv_state=None, state_len=None,
                  silu=True):
    """Causal depthwise conv1d (+SiLU) over packed sequences.

    x: [T, C]; weight: [C, K]; conv_state: [n, C, state_len] or None.
    Returns (y [T, C], conv_state_out [n, C, state_len]).
    """
    x, weight = _f64(x), _f64(weight)
    T, C = x.shape
    K = weight.shape[1]
    cu, n = _cu(cu_seqlens, T)
    if state_len is None:
        state_len = conv_state.shape[2] if conv_state is not None else K - 1
    b = None if bias is None else _f64(bias)
    si = None if conv_state is None else _f64(conv_state)
    so = np.empty((n, C, state_len))
    y = np.empty((T, C))
    rc = _load().oracle_causal_conv1d(T, n, None if cu is None else cu.ctypes.data_as(_i64p),
                                      C, K, state_len, _ptr(x), _ptr(weight), _ptr(b),
                                      _ptr(si), _ptr(so), int(bool(silu)), _ptr(y))
    _check(rc, "causal_conv1d")
    return y, so


def causal_conv1d_update(x, conv_state, weight, bias=None, silu=True):
    """One decode step: returns (y [n, C], new conv_state [n, C, state_len])."""
    x, weight = _f64(x), _f64(weight)
    st = _f64(conv_state).copy()
    n, C, state_len = st.shape
    K = weight.shape[1]
    b = None if bias is None else _f64(bias)
    y = np.empty((n, C))
    rc = _load().oracle_causal_conv1d_update(n, C, K, state_len, _ptr(x), _ptr(st),
                                             _ptr(weight), _ptr(b), int(bool(silu)), _ptr(y))
    _check(rc, "causal_conv1d_update")
    return y, st


def gated_rmsnorm(x, z, weight, eps=1e-6):
    """y = x * rsqrt(mean(x^2) + eps) * (1 + w) * silu(z), row-wise over the last dim."""
    x, z, weight = _f64(x), _f64(z), _f64(weight)
    shape = x.shape
    D = shape[-1]
    x2, z2 = x.reshape(-1, D), z.reshape(-1, D)
    y = np.empty_like(x2)
    _check(_load().oracle_gated_rmsnorm(x2.shape[0], D, _ptr(x2), _ptr(z2), _ptr(weight),
                                        float(eps), _ptr(y)), "gated_rmsnorm")
    return y.reshape(shape)
