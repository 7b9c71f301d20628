/*
 * gdn_oracle.h -- plain fp64 CPU oracle for the Gated DeltaNet core.
 *
 * TEST INFRASTRUCTURE ONLY. Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library. It shares no code,
 * header or constant with the GPU library and must never be linked into it.
 *
 * Every routine is the plain definition of what it computes, written in
 * double precision, one token at a time, with no blocking or reordering
 * beyond what the definition states. Sources (page titles as published):
 *   [DMA]  "Qwen3.5 Dense Model Architecture" (blog), section "Linear
 *          Attention": mechanism list, minimal forward example, cache table.
 *   [SIM]  "Qwen3.5 Simulation Support Design Document" (msmodeling RFC),
 *          sections 1.1, 2.2 (decomposed op flow), 2.4 (CausalConv1d split),
 *          Appendix B glossary.
 * Where the pages leave a step open the reading is stated at the routine.
 *
 * Conventions: all arrays are dense, row-major, double precision, host memory.
 *   tokens are packed: sequence n occupies tokens [cu[n], cu[n+1]).
 *   q, k : [T_tot, nk, dk]    v : [T_tot, nv, dv]    g, beta : [T_tot, nv]
 *   state: [n_seqs, nv, dk, dv]   (S is dk x dv; the read-out is S^T q)
 * Return value: 0 on success, -1 on an invalid argument (nothing written).
 */
#ifndef GDN_ORACLE_H
#define GDN_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Gating ([DMA] minimal example, the beta/g lines):
 *   beta = sigmoid(b),  g = -exp(A_log[h]) * softplus(a + dt_bias[h]).
 * a, b : [T, nv]; A_log, dt_bias : [nv]; g, beta : [T, nv]. */
int oracle_gating(int64_t T, int nv, const double* a, const double* b,
                  const double* A_log, const double* dt_bias,
                  double* g, double* beta);

/* Gated delta rule, token by token ([DMA] mechanism list and the schematic
 * state update; exact order: decay, delta update on the decayed state,
 * read-out after the update).  Per sequence n and value head h, with key
 * head hk = h / (nv/nk) (repeat_interleave):
 *   S <- S0[n,h] (or 0)
 *   for t in sequence:  qh = q[t,hk] * rsqrt(|q|^2+eps) * scale
 *                       kh = k[t,hk] * rsqrt(|k|^2+eps)      (if l2norm)
 *                       S  <- exp(g[t,h]) * S
 *                       u  <- v[t,h] - S^T kh
 *                       S  <- S + beta[t,h] * kh u^T
 *                       o[t,h] <- S^T qh
 *   ST[n,h] <- S
 * cu_seqlens: [n_seqs+1] or NULL (one sequence of T_tot tokens).
 * S0 may be NULL (zero state); ST may be NULL (not written).
 * threads <= 0 uses the OpenMP default. */
int oracle_delta_rule(int64_t T_tot, int n_seqs, const int64_t* cu_seqlens,
                      int nk, int nv, int dk, int dv,
                      const double* q, const double* k, const double* v,
                      const double* g, const double* beta,
                      double scale, int l2norm, double eps,
                      const double* S0, double* ST, double* o, int threads);

/* Causal depthwise conv1d (+ optional SiLU) over packed sequences
 * ([DMA] minimal example, prefill branch; [SIM] 2.4 conv body).
 * Cross-correlation with left context: for token t of a sequence,
 *   y[t,c] = act(bias[c] + sum_{j<K} w[c,j] * xe[t + j])
 * where xe = concat(state_in[n,c,:], x[seq tokens, c]) restricted to its
 * last (K-1) history entries before the first token.  state_in may be NULL
 * (zero history).  state_out[n,c,:] = last state_len entries of
 * concat(state_in[n,c,:] or zeros, x[seq tokens, c]); may be NULL.
 * x, y: [T_tot, conv_dim]; w: [conv_dim, K]; bias: [conv_dim] or NULL;
 * state_*: [n_seqs, conv_dim, state_len] with state_len >= K-1. */
int oracle_causal_conv1d(int64_t T_tot, int n_seqs, const int64_t* cu_seqlens,
                         int conv_dim, int K, int state_len,
                         const double* x, const double* w, const double* bias,
                         const double* state_in, double* state_out,
                         int silu, double* y);

/* One decode step of the causal conv ([DMA] decode branch; [SIM] 2.4 state
 * update): window = [state[n,c, state_len-(K-1):], x[n,c]],
 *   y[n,c] = act(bias[c] + sum_j w[c,j] * window[j]),
 * then state[n,c,:] <- [state[n,c,1:], x[n,c]] (shift left, append). */
int oracle_causal_conv1d_update(int n_seqs, int conv_dim, int K, int state_len,
                                const double* x, double* state,
                                const double* w, const double* bias,
                                int silu, double* y);

/* Gated RMSNorm ([SIM] 1.1 and glossary: output * (1 + weight); [DMA]
 * minimal example: norm(core_output, z) over rows of Dv):
 *   y = x * (mean(x^2) + eps)^(-1/2) * (1 + w) * z * sigmoid(z).
 * x, z, y: [rows, D]; w: [D]. */
int oracle_gated_rmsnorm(int64_t rows, int D, const double* x, const double* z,
                         const double* w, double eps, double* y);

#ifdef __cplusplus
}
#endif

#endif /* GDN_ORACLE_H */
