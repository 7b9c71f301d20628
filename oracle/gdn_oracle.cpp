// gdn_oracle.cpp -- plain fp64 CPU oracle for the Gated DeltaNet core.
//
// TEST INFRASTRUCTURE ONLY (see gdn_oracle.h). Slow and obviously correct:
// every loop below is the definition of the quantity, in double precision.
// OpenMP only distributes independent (sequence, value head) or
// (sequence, channel) units; the arithmetic inside a unit is sequential.

#include "gdn_oracle.h"

#include <cmath>
#include <cstdint>
#include <vector>

#ifdef _OPENMP
#include <omp.h>
#endif

namespace {

double sigmoid(double x) { return 1.0 / (1.0 + std::exp(-x)); }

// softplus(s) = log(1 + e^s), written so that e^{|s|} never overflows:
// log(1 + e^s) = max(s, 0) + log1p(e^{-|s|}).
double softplus(double s) { return (s > 0 ? s : 0.0) + std::log1p(std::exp(-std::fabs(s))); }

double silu(double x) { return x * sigmoid(x); }

bool valid_cu(const int64_t* cu, int n_seqs, int64_t T_tot) {
  if (!cu) return true;
  if (cu[0] != 0 || cu[n_seqs] != T_tot) return false;
  for (int n = 0; n < n_seqs; ++n)
    if (cu[n + 1] < cu[n]) return false;
  return true;
}

int64_t seq_begin(const int64_t* cu, int n, int64_t T_tot) { return cu ? cu[n] : (n == 0 ? 0 : T_tot); }
int64_t seq_end(const int64_t* cu, int n, int64_t T_tot) { return cu ? cu[n + 1] : T_tot; }

}  // namespace

extern "C" int oracle_gating(int64_t T, int nv, const double* a, const double* b,
                             const double* A_log, const double* dt_bias,
                             double* g, double* beta) {
  if (T < 0 || nv <= 0 || !a || !b || !A_log || !dt_bias || !g || !beta) return -1;
  for (int64_t t = 0; t < T; ++t) {
    for (int h = 0; h < nv; ++h) {
      const int64_t i = t * nv + h;
      beta[i] = sigmoid(b[i]);
      g[i] = -std::exp(A_log[h]) * softplus(a[i] + dt_bias[h]);
    }
  }
  return 0;
}

extern "C" int oracle_delta_rule(int64_t T_tot, int n_seqs, const int64_t* cu_seqlens,
                                 int nk, int nv, int dk, int dv,
                                 const double* q, const double* k, const double* v,
                                 const double* g, const double* beta,
                                 double scale, int l2norm, double eps,
                                 const double* S0, double* ST, double* o, int threads) {
  if (T_tot < 0 || n_seqs <= 0 || nk <= 0 || nv <= 0 || dk <= 0 || dv <= 0) return -1;
  if (nv % nk != 0) return -1;
  if (!cu_seqlens && n_seqs != 1) return -1;
  if (!valid_cu(cu_seqlens, n_seqs, T_tot)) return -1;
  if (T_tot > 0 && (!q || !k || !v || !g || !beta || !o)) return -1;
  const int r = nv / nk;
  const int64_t units = static_cast<int64_t>(n_seqs) * nv;
#ifdef _OPENMP
  if (threads > 0) omp_set_num_threads(threads);
#else
  (void)threads;
#endif

#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t unit = 0; unit < units; ++unit) {
    const int n = static_cast<int>(unit / nv);
    const int h = static_cast<int>(unit % nv);
    const int hk = h / r;  // repeat_interleave: value head h reads key head h / r
    std::vector<double> S(static_cast<size_t>(dk) * dv, 0.0);  // S[i*dv + j], i over dk
    if (S0) {
      const double* src = S0 + unit * dk * dv;
      for (int64_t e = 0; e < static_cast<int64_t>(dk) * dv; ++e) S[e] = src[e];
    }
    std::vector<double> qh(dk), kh(dk), u(dv), acc(dv);
    const int64_t t0 = seq_begin(cu_seqlens, n, T_tot), t1 = seq_end(cu_seqlens, n, T_tot);
    for (int64_t t = t0; t < t1; ++t) {
      const double* qt = q + (t * nk + hk) * dk;
      const double* kt = k + (t * nk + hk) * dk;
      const double* vt = v + (t * nv + h) * dv;
      double rq = 1.0, rk = 1.0;
      if (l2norm) {
        double sq = 0.0, sk = 0.0;
        for (int i = 0; i < dk; ++i) { sq += qt[i] * qt[i]; sk += kt[i] * kt[i]; }
        rq = 1.0 / std::sqrt(sq + eps);
        rk = 1.0 / std::sqrt(sk + eps);
      }
      for (int i = 0; i < dk; ++i) { qh[i] = qt[i] * rq * scale; kh[i] = kt[i] * rk; }
      // decay
      const double decay = std::exp(g[t * nv + h]);
      for (auto& s : S) s *= decay;
      // delta update on the decayed state: u = v - S^T kh ; S += beta kh u^T.
      // (S^T kh)_j = sum_i S_ij kh_i, summed over i in increasing order for
      // every j; the i-outer loop only interleaves the independent j sums.
      for (int j = 0; j < dv; ++j) acc[j] = 0.0;
      for (int i = 0; i < dk; ++i)
        for (int j = 0; j < dv; ++j) acc[j] += S[static_cast<size_t>(i) * dv + j] * kh[i];
      for (int j = 0; j < dv; ++j) u[j] = vt[j] - acc[j];
      const double bt = beta[t * nv + h];
      for (int i = 0; i < dk; ++i)
        for (int j = 0; j < dv; ++j) S[static_cast<size_t>(i) * dv + j] += bt * kh[i] * u[j];
      // read-out after the update: o = S^T qh (same summation order)
      double* ot = o + (t * nv + h) * dv;
      for (int j = 0; j < dv; ++j) acc[j] = 0.0;
      for (int i = 0; i < dk; ++i)
        for (int j = 0; j < dv; ++j) acc[j] += S[static_cast<size_t>(i) * dv + j] * qh[i];
      for (int j = 0; j < dv; ++j) ot[j] = acc[j];
    }
    if (ST) {
      double* dst = ST + unit * dk * dv;
      for (int64_t e = 0; e < static_cast<int64_t>(dk) * dv; ++e) dst[e] = S[e];
    }
  }
  return 0;
}

extern "C" int oracle_causal_conv1d(int64_t T_tot, int n_seqs, const int64_t* cu_seqlens,
                                    int conv_dim, int K, int state_len,
                                    const double* x, const double* w, const double* bias,
                                    const double* state_in, double* state_out,
                                    int silu_on, double* y) {
  if (T_tot < 0 || n_seqs <= 0 || conv_dim <= 0 || K <= 0 || state_len < K - 1) return -1;
  if (!cu_seqlens && n_seqs != 1) return -1;
  if (!valid_cu(cu_seqlens, n_seqs, T_tot)) return -1;
  if (!w || (T_tot > 0 && (!x || !y))) return -1;
  const int64_t units = static_cast<int64_t>(n_seqs) * conv_dim;
#pragma omp parallel for schedule(static)
  for (int64_t unit = 0; unit < units; ++unit) {
    const int n = static_cast<int>(unit / conv_dim);
    const int c = static_cast<int>(unit % conv_dim);
    const int64_t t0 = seq_begin(cu_seqlens, n, T_tot), t1 = seq_end(cu_seqlens, n, T_tot);
    const int64_t L = t1 - t0;
    // ext = concat(history of state_len entries, sequence inputs)
    std::vector<double> ext(static_cast<size_t>(state_len + L), 0.0);
    if (state_in)
      for (int s = 0; s < state_len; ++s) ext[s] = state_in[unit * state_len + s];
    for (int64_t t = 0; t < L; ++t) ext[state_len + t] = x[(t0 + t) * conv_dim + c];
    for (int64_t t = 0; t < L; ++t) {
      // input t sits at ext[state_len + t]; tap j multiplies input t-(K-1)+j
      double acc = bias ? bias[c] : 0.0;
      for (int j = 0; j < K; ++j) acc += w[static_cast<int64_t>(c) * K + j] * ext[state_len + t - (K - 1) + j];
      y[(t0 + t) * conv_dim + c] = silu_on ? silu(acc) : acc;
    }
    if (state_out)
      for (int s = 0; s < state_len; ++s) state_out[unit * state_len + s] = ext[L + s];
  }
  return 0;
}

extern "C" int oracle_causal_conv1d_update(int n_seqs, int conv_dim, int K, int state_len,
                                           const double* x, double* state,
                                           const double* w, const double* bias,
                                           int silu_on, double* y) {
  if (n_seqs <= 0 || conv_dim <= 0 || K <= 0 || state_len < K - 1) return -1;
  if (!x || !state || !w || !y) return -1;
  const int64_t units = static_cast<int64_t>(n_seqs) * conv_dim;
  std::vector<double> win(K);
  for (int64_t unit = 0; unit < units; ++unit) {
    const int c = static_cast<int>(unit % conv_dim);
    double* st = state + unit * state_len;
    for (int j = 0; j < K - 1; ++j) win[j] = st[state_len - (K - 1) + j];
    win[K - 1] = x[unit];
    double acc = bias ? bias[c] : 0.0;
    for (int j = 0; j < K; ++j) acc += w[static_cast<int64_t>(c) * K + j] * win[j];
    y[unit] = silu_on ? silu(acc) : acc;
    for (int s = 0; s + 1 < state_len; ++s) st[s] = st[s + 1];
    if (state_len > 0) st[state_len - 1] = x[unit];
  }
  return 0;
}

extern "C" int oracle_gated_rmsnorm(int64_t rows, int D, const double* x, const double* z,
                                    const double* w, double eps, double* y) {
  if (rows < 0 || D <= 0 || !w || (rows > 0 && (!x || !z || !y))) return -1;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    const double* xr = x + r * D;
    const double* zr = z + r * D;
    double ss = 0.0;
    for (int i = 0; i < D; ++i) ss += xr[i] * xr[i];
    const double inv = 1.0 / std::sqrt(ss / D + eps);
    for (int i = 0; i < D; ++i) y[r * D + i] = xr[i] * inv * (1.0 + w[i]) * silu(zr[i]);
  }
  return 0;
}
