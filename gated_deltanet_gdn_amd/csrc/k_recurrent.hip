// k_recurrent.hip -- recurrent gated delta rule (decode path), dk = dv = 128.
//
// Token-by-token update of "Qwen3.5 Dense Model Architecture", Linear
// Attention (decay, delta update, read-out; state updated in place during
// decode per its cache table); "Qwen3.5 Simulation Support Design Document"
// 2.3 routes single-token and multi-token (MTP) decode batches here.
//
// One workgroup of 256 threads per (sequence, value head, NCOL columns of the
// state): the Dk-reductions run down columns, so column blocks are
// independent. Thread t owns columns 4*(t % CGN) .. +3 of the block (CGN =
// NCOL / 4) in rows (t / CGN) + RGN*i, so each fp32 state block is read once
// into registers with contiguous float4 loads and written back once at the
// end. Per token both Dk-reductions (S^T kh and S^T qh) share one pass over
// the registers:
//   a = S^T kh, b = S^T qh (qh carries the scale)
//   delta = beta (v - e a),  e = exp(g)
//   o = e b + (kh . qh) delta          (= S'^T qh)
//   S' = e S + kh delta^T
#include "gdn_device.hpp"
#include "gdn_internal.hpp"

namespace gdn {
namespace {

constexpr int D = 128;

template <typename TIn, typename TO, int NCOL>
__global__ void __launch_bounds__(256) recurrent_kernel(const TIn* __restrict__ q, const TIn* __restrict__ k,
                                                        const TIn* __restrict__ v, int64_t qs, int64_t ks,
                                                        int64_t vs, const float* __restrict__ g,
                                                        const float* __restrict__ beta,
                                                        const int32_t* __restrict__ cu, int64_t T, int nk, int nv,
                                                        float scale, int l2, float* __restrict__ state,
                                                        TO* __restrict__ o) {
  constexpr int CGN = NCOL / 4;         // column groups
  constexpr int RGN = 256 / CGN;        // row groups
  constexpr int RPT = D / RGN;          // rows per thread
  __shared__ float kq_s[2][2][D];       // [parity][k|q][D]
  __shared__ float red[2][4][2][NCOL];  // [parity][wave][a|b][column]

  constexpr int NB = D / NCOL;
  const int unit = blockIdx.x / NB;     // n * nv + h
  const int col0 = (blockIdx.x % NB) * NCOL;
  const int n = unit / nv;
  const int h = unit % nv;
  const int hk = h / (nv / nk);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int cg = tid % CGN;
  const int rg = tid / CGN;
  const int col = col0 + 4 * cg;        // first of this thread's 4 columns

  int64_t t0, t1;
  if (cu) seq_bounds(cu, n, T, t0, t1);
  else { t0 = n; t1 = n + 1; }   // one token per sequence (T == n_seqs)

  // a token's inputs for this thread, as loaded (converted at use: any
  // arithmetic at load time would wait for the load right there): one
  // element of k (threads < 128) or of q, 4 of v, g and beta
  TIn kq_n{}, vv_n[4] = {};
  float gt_n = 0.f, bt_n = 0.f;
  auto load_token = [&](int64_t t) {
    kq_n = tid < D ? k[t * ks + static_cast<int64_t>(hk) * D + tid] : q[t * qs + static_cast<int64_t>(hk) * D + (tid - D)];
#pragma unroll
    for (int c = 0; c < 4; ++c) vv_n[c] = v[t * vs + static_cast<int64_t>(h) * D + col + c];
    gt_n = g[t * nv + h];
    bt_n = beta[t * nv + h];
  };
  // the first token's inputs go out before the state stream: completions are
  // counted in order, so the norms below then wait only for these
  if (t0 < t1) load_token(t0);

  // The state streams through once each way. It is read with ordinary loads
  // and written back non-temporally (each state is touched once per call);
  // of the four load/store hint combinations this one streams fastest.
  float* Sp = state + static_cast<int64_t>(unit) * D * D;
  float S[RPT][4];
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const f32x4 s4 = *reinterpret_cast<const f32x4*>(Sp + (rg + RGN * i) * D + col);
    S[i][0] = s4[0]; S[i][1] = s4[1]; S[i][2] = s4[2]; S[i][3] = s4[3];
  }

  int par = 0;
  for (int64_t t = t0; t < t1; ++t, par ^= 1) {
    const float kqv = Elem<TIn>::cvt(kq_n), gt = gt_n, bt = bt_n;
    float vv[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) vv[c] = Elem<TIn>::cvt(vv_n[c]);
    if (t + 1 < t1) load_token(t + 1);   // the next token's inputs
    // stage k and q of this token's key head in LDS (fp32)
    kq_s[par][tid < D ? 0 : 1][tid & (D - 1)] = kqv;
    __syncthreads();

    // norms and k.q, redundantly per wave (no extra barrier)
    const float k0 = kq_s[par][0][2 * lane], k1 = kq_s[par][0][2 * lane + 1];
    const float q0 = kq_s[par][1][2 * lane], q1 = kq_s[par][1][2 * lane + 1];
    const float skk = wave_sum(k0 * k0 + k1 * k1);
    const float sqq = wave_sum(q0 * q0 + q1 * q1);
    const float sqk = wave_sum(q0 * k0 + q1 * k1);
    const float rk = l2 ? 1.0f / sqrtf(skk + 1e-6f) : 1.0f;
    const float rq = (l2 ? 1.0f / sqrtf(sqq + 1e-6f) : 1.0f) * scale;
    const float kq = sqk * rk * rq;
    const float e = expf(gt);

    float pa[4] = {0.f, 0.f, 0.f, 0.f}, pb[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const float kh = kq_s[par][0][rg + RGN * i] * rk;
      const float qh = kq_s[par][1][rg + RGN * i] * rq;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        pa[c] = fmaf(S[i][c], kh, pa[c]);
        pb[c] = fmaf(S[i][c], qh, pb[c]);
      }
    }
    // the 64 / CGN row groups of a wave sit in lanes l, l ^ CGN, ... of that wave
#pragma unroll
    for (int x = CGN; x < 64; x <<= 1) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        pa[c] += __shfl_xor(pa[c], x, 64);
        pb[c] += __shfl_xor(pb[c], x, 64);
      }
    }
    if (lane < CGN) {
      *reinterpret_cast<float4*>(&red[par][wave][0][4 * cg]) = make_float4(pa[0], pa[1], pa[2], pa[3]);
      *reinterpret_cast<float4*>(&red[par][wave][1][4 * cg]) = make_float4(pb[0], pb[1], pb[2], pb[3]);
    }
    __syncthreads();
    float a4[4] = {0.f, 0.f, 0.f, 0.f}, b4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float4 ra = *reinterpret_cast<const float4*>(&red[par][w][0][4 * cg]);
      const float4 rb = *reinterpret_cast<const float4*>(&red[par][w][1][4 * cg]);
      a4[0] += ra.x; a4[1] += ra.y; a4[2] += ra.z; a4[3] += ra.w;
      b4[0] += rb.x; b4[1] += rb.y; b4[2] += rb.z; b4[3] += rb.w;
    }
    float dl[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) dl[c] = bt * (vv[c] - e * a4[c]);
    if (rg == 0) {
      const int64_t ob = t * static_cast<int64_t>(nv) * D + static_cast<int64_t>(h) * D + col;
#pragma unroll
      for (int c = 0; c < 4; ++c) Elem<TO>::store(o, ob + c, fmaf(e, b4[c], kq * dl[c]));
    }
    // (k re-read from LDS rather than held across the barrier: fewer VGPRs,
    // one more workgroup per CU)
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const float kh = kq_s[par][0][rg + RGN * i] * rk;
#pragma unroll
      for (int c = 0; c < 4; ++c) S[i][c] = fmaf(e, S[i][c], kh * dl[c]);
    }
  }

#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    f32x4 s4;
    s4[0] = S[i][0]; s4[1] = S[i][1]; s4[2] = S[i][2]; s4[3] = S[i][3];
    __builtin_nontemporal_store(s4, reinterpret_cast<f32x4*>(Sp + (rg + RGN * i) * D + col));
  }
}

template <typename TIn>
hipError_t rec_dispatch(const void* q, const void* k, const void* v, int64_t qs, int64_t ks, int64_t vs,
                        const float* g, const float* beta, const int32_t* cu, int n_seqs, int64_t T, int nk,
                        int nv, float scale, int l2, float* state, void* o, int o_bf16, hipStream_t s) {
  constexpr int NCOL = 128;   // one workgroup per state: each wave load covers 1 KB of contiguous rows
  const dim3 grid(static_cast<unsigned>(n_seqs) * static_cast<unsigned>(nv) * (D / NCOL));
  if (o_bf16)
    recurrent_kernel<TIn, uint16_t, NCOL><<<grid, 256, 0, s>>>(
        static_cast<const TIn*>(q), static_cast<const TIn*>(k), static_cast<const TIn*>(v), qs, ks, vs, g, beta,
        cu, T, nk, nv, scale, l2, state, static_cast<uint16_t*>(o));
  else
    recurrent_kernel<TIn, float, NCOL><<<grid, 256, 0, s>>>(
        static_cast<const TIn*>(q), static_cast<const TIn*>(k), static_cast<const TIn*>(v), qs, ks, vs, g, beta,
        cu, T, nk, nv, scale, l2, state, static_cast<float*>(o));
  return hipGetLastError();
}

}  // namespace

hipError_t launch_recurrent(const void* q, const void* k, const void* v, int bf16, int64_t qs, int64_t ks,
                            int64_t vs, const float* g, const float* beta, const int32_t* cu, int n_seqs,
                            int64_t T, int nk, int nv, float scale, int l2, float* state, void* o, int o_bf16,
                            hipStream_t s) {
  if (bf16)
    return rec_dispatch<uint16_t>(q, k, v, qs, ks, vs, g, beta, cu, n_seqs, T, nk, nv, scale, l2, state, o, o_bf16,
                                  s);
  return rec_dispatch<float>(q, k, v, qs, ks, vs, g, beta, cu, n_seqs, T, nk, nv, scale, l2, state, o, o_bf16, s);
}

}  // namespace gdn
