"""fp64 numpy evaluation of the chunked gated delta rule -- TEST INFRASTRUCTURE ONLY.

This is the chunk-parallel rewriting of the token recurrence (intra-chunk
attention + inter-chunk recurrence with chunk_size = 64, as the "Qwen3.5
Simulation Support Design Document" glossary describes the chunk gated delta
rule). The pages name the method but print none of its algebra; the steps
below are derived from the recurrence itself (per chunk of C tokens, state
S at the chunk start, G = chunk-local cumulative sum of g):

  A_ij   = beta_i * exp(G_i - G_j) * (k_i . k_j)         for j < i, else 0
  T      = (I + A)^-1                                      (unit lower triangular)
  U      = T diag(beta) V,   W = T diag(beta * exp(G)) K
  U_new  = U - W S
  O      = diag(exp(G)) Q S + (Q K^T o M) U_new,   M_ij = exp(G_i - G_j), j <= i
  S'     = exp(G_C) S + (diag(exp(G_C - G)) K)^T U_new

It is used only to cross-check the token-by-token oracle in ``oracle/`` (two
different algorithms that must agree to ~1e-11 in fp64), which in turn pins
the algebra the GPU chunk kernels implement. It shares no code with either.
"""
from __future__ import annotations

import numpy as np


def _l2(x, eps):
    return x / np.sqrt((x * x).sum(-1, keepdims=True) + eps)


def chunk_delta_rule(q, k, v, g, beta, cu_seqlens=None, initial_state=None, scale=None,
                     l2norm=True, eps=1e-6, chunk=64):
    q, k, v, g, beta = (np.asarray(t, dtype=np.float64) for t in (q, k, v, g, beta))
    T, nk, dk = q.shape
    nv, dv = v.shape[1:]
    r = nv // nk
    if scale is None:
        scale = dk ** -0.5
    cu = [0, T] if cu_seqlens is None else [int(c) for c in cu_seqlens]
    n = len(cu) - 1
    o = np.zeros((T, nv, dv))
    ST = np.zeros((n, nv, dk, dv))
    for s in range(n):
        t0, t1 = cu[s], cu[s + 1]
        for h in range(nv):
            hk = h // r
            S = (np.zeros((dk, dv)) if initial_state is None
                 else np.array(initial_state[s, h], dtype=np.float64))
            for c0 in range(t0, t1, chunk):
                c1 = min(c0 + chunk, t1)
                K = k[c0:c1, hk]
                Q = q[c0:c1, hk]
                if l2norm:
                    K, Q = _l2(K, eps), _l2(Q, eps)
                Q = Q * scale
                V = v[c0:c1, h]
                b = beta[c0:c1, h]
                G = np.cumsum(g[c0:c1, h])
                L = c1 - c0
                D = G[:, None] - G[None, :]                     # G_i - G_j
                lower = np.tril(np.ones((L, L), dtype=bool), -1)
                incl = np.tril(np.ones((L, L), dtype=bool), 0)
                Mstrict = np.where(lower, np.exp(np.where(lower, D, 0.0)), 0.0)
                Mincl = np.where(incl, np.exp(np.where(incl, D, 0.0)), 0.0)
                A = b[:, None] * Mstrict * (K @ K.T)
                Tm = np.linalg.inv(np.eye(L) + A)
                U = Tm @ (b[:, None] * V)
                W = Tm @ ((b * np.exp(G))[:, None] * K)
                Unew = U - W @ S
                o[c0:c1, h] = (np.exp(G)[:, None] * (Q @ S)) + ((Q @ K.T) * Mincl) @ Unew
                S = np.exp(G[-1]) * S + (np.exp(G[-1] - G)[:, None] * K).T @ Unew
            ST[s, h] = S
    return o, ST
