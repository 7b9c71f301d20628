// k_recurrent.hip -- recurrent gated delta rule (decode path), dk = dv = 128,
// and the fused decode step built on it.
//
// Token-by-token update of "Qwen3.5 Dense Model Architecture", Linear
// Attention (decay, delta update, read-out; state updated in place during
// decode per its cache table); "Qwen3.5 Simulation Support Design Document"
// 2.3 routes single-token and multi-token (MTP) decode batches here.
//
// 256 threads per (sequence, value head) state, two states of one sequence
// per workgroup: thread t owns columns 4 (t % 32) .. +3 in rows t / 32 + 8 i,
// so the 64 KB fp32 state is read once into registers with contiguous float4
// loads (each wave load covers 1 KB of rows) and written back once at the end. Per token both
// Dk-reductions (S^T kh and S^T qh) share one pass over the registers:
//   a = S^T kh, b = S^T qh (qh carries the scale)
//   delta = beta (v - e a),  e = exp(g)
//   o = e b + (kh . qh) delta          (= S'^T qh)
//   S' = e S + kh delta^T
//
// The fused decode step runs the layer's whole decode prologue in the same
// launch ("Qwen3.5 Dense Model Architecture", Linear Attention, decode branch
// of the minimal example: conv update with SiLU over the packed q|k|v
// channels, gating, then the recurrent rule; "Qwen3.5 / Qwen3.6 Inference
// Path on vLLM Ascend", stage 4 of its per-step flow, captures decode steps
// in device graphs, where fewer launches per layer count). One workgroup per
// (sequence, key head) with 256 threads per value head of that key head, so
// every conv channel it reads (q and k of the key head, v of its value heads)
// is owned by exactly one workgroup and the conv state can be updated in
// place. The conv output is rounded to the activation dtype before use, as it
// is when stored between separate launches, and the per-token arithmetic is
// the same code as the separate kernels': the fused step reproduces conv
// update + gating + recurrent launches bit for bit.
#include "gdn_device.hpp"
#include "gdn_internal.hpp"

namespace gdn {
namespace {

constexpr int D = 128;
constexpr int CGN = 32;           // column groups of 4 in a 128-column state
constexpr int RGN = 256 / CGN;    // row groups
constexpr int RPT = D / RGN;      // rows per thread

// fp32 -> activation dtype -> fp32 (the value a separate launch would store and re-read)
__device__ __forceinline__ float act_round(float v, float) { return v; }
__device__ __forceinline__ float act_round(float v, uint16_t) { return bf16_to_f32(f32_to_bf16(v)); }

// k and q of a token sit in LDS grouped by row group: row r at slot
// (r % RGN) * RPT + r / RGN, so a thread's 16 rows (r = rg + RGN i) are the
// 16 consecutive floats at rg * RPT (four 16-byte reads).
__device__ __forceinline__ int kq_slot(int r) { return (r % RGN) * RPT + r / RGN; }

// In a launch with several tokens per sequence (cu_seqlens given), within a
// sequence's tokens the state is carried as S = E St with a scalar E
// per state (the product of the decays since the last fold, the same in every
// thread), so a token's update is one fma per element, St += k (rk delta /
// E')^T with E' = e E, instead of a decay multiply and an fma. A token at
// which E' would fall below kStateScaleMin folds E' into St instead
// (St' = E' St + k (rk delta)^T, E = 1). S = E St is formed where the state
// leaves the thread (the final store, a snapshot), the same way after every
// token, so the state after token t does not depend on whether more tokens
// follow (a snapshot after token t equals the final state of the same step
// run on the tokens up to t). A launch of one token per sequence (no
// cu_seqlens) updates S directly, S' = e S + k (rk delta)^T, and skips the
// final multiply (DEFER = false).
constexpr float kStateScaleMin = 0x1p-64f;

// a value that is the same in every lane (a butterfly wave sum, per-state
// gating), moved to a scalar register
__device__ __forceinline__ float uni(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, v)));
}

// One token of the recurrence for a state held by 256 threads (thread t256:
// columns 4 (t256 % 32) .. +3, rows t256 / 32 + 8 i), in two halves around a
// barrier of the whole workgroup. ks and qs are this token's raw k and q of
// the key head (fp32 in LDS in kq_slot order, written before a barrier that
// precedes the first half); red is LDS scratch [4 waves][a | b][128 columns].
// The first half forms the norms and this thread's partial sums of St^T k and
// St^T q (raw k and q: the norms, the scale and E multiply the sums after the
// reduction) and writes them to red; the second half (after the barrier)
// adds them up, stores o (row element offset ob, the thread's first column;
// rows of group rg == 0 store) and updates St and E. ks must still hold the
// token's k then.
struct RecNorms { float rk, rq, kq; };
__device__ __forceinline__ RecNorms rec_pass(const float (&S)[RPT][4], const float* ks, const float* qs, float* red,
                                             int t256, float scale, int l2) {
  const int lane = t256 & 63, wave = t256 >> 6, cg = t256 % CGN, rg = t256 / CGN;
  // norms and k.q, redundantly per wave (no extra barrier)
  const float k0 = ks[2 * lane], k1 = ks[2 * lane + 1];
  const float q0 = qs[2 * lane], q1 = qs[2 * lane + 1];
  const float skk = wave_sum(k0 * k0 + k1 * k1);
  const float sqq = wave_sum(q0 * q0 + q1 * q1);
  const float sqk = wave_sum(q0 * k0 + q1 * k1);
  // (hardware reciprocal square root, about 1 ulp: a correctly rounded
  // 1 / sqrt costs some twenty VALU operations per token and wave)
  const float rk = uni(l2 ? __builtin_amdgcn_rsqf(skk + 1e-6f) : 1.0f);
  const float rq = uni((l2 ? __builtin_amdgcn_rsqf(sqq + 1e-6f) : 1.0f) * scale);
  const float kq = uni(sqk * rk * rq);

  float pa[4] = {0.f, 0.f, 0.f, 0.f}, pb[4] = {0.f, 0.f, 0.f, 0.f};
  const float4* k4 = reinterpret_cast<const float4*>(ks + rg * RPT);
  const float4* q4 = reinterpret_cast<const float4*>(qs + rg * RPT);
#pragma unroll
  for (int i4 = 0; i4 < RPT / 4; ++i4) {
    const float4 kk = k4[i4], qq = q4[i4];
    const float kr[4] = {kk.x, kk.y, kk.z, kk.w}, qr[4] = {qq.x, qq.y, qq.z, qq.w};
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        pa[c] = fmaf(S[4 * i4 + u][c], kr[u], pa[c]);
        pb[c] = fmaf(S[4 * i4 + u][c], qr[u], pb[c]);
      }
  }
  // the two row groups of a wave sit in lanes l and l ^ 32
#pragma unroll
  for (int x = CGN; x < 64; x <<= 1) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      pa[c] += __shfl_xor(pa[c], x, 64);
      pb[c] += __shfl_xor(pb[c], x, 64);
    }
  }
  if (lane < CGN) {
    *reinterpret_cast<float4*>(red + (wave * 2 + 0) * D + 4 * cg) = make_float4(pa[0], pa[1], pa[2], pa[3]);
    *reinterpret_cast<float4*>(red + (wave * 2 + 1) * D + 4 * cg) = make_float4(pb[0], pb[1], pb[2], pb[3]);
  }
  return {rk, rq, kq};
}
template <typename TO, bool DEFER>
__device__ __forceinline__ void rec_finish(float (&S)[RPT][4], float& E, const float* ks, const float (&vv)[4],
                                           float gt, float bt, const float* red, int t256, RecNorms nr,
                                           TO* __restrict__ o, int64_t ob) {
  const int cg = t256 % CGN, rg = t256 / CGN;
  const float e = uni(expf(gt));
  float a4[4] = {0.f, 0.f, 0.f, 0.f}, b4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const float4 ra = *reinterpret_cast<const float4*>(red + (w * 2 + 0) * D + 4 * cg);
    const float4 rb = *reinterpret_cast<const float4*>(red + (w * 2 + 1) * D + 4 * cg);
    a4[0] += ra.x; a4[1] += ra.y; a4[2] += ra.z; a4[3] += ra.w;
    b4[0] += rb.x; b4[1] += rb.y; b4[2] += rb.z; b4[3] += rb.w;
  }
  // a = S^T k_hat = E rk St^T k, b = S^T q_hat = E rq St^T q
  const float sa = E * nr.rk, sb = E * nr.rq;
  float dl[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) dl[c] = bt * (vv[c] - e * (a4[c] * sa));
  if (rg == 0) {
#pragma unroll
    for (int c = 0; c < 4; ++c) Elem<TO>::store(o, ob + c, fmaf(e, b4[c] * sb, nr.kq * dl[c]));
  }
  // S' = e S + k_hat delta^T: St' = St + k (rk delta / E')^T with E' = e E,
  // or, below the floor, St' = E' St + k (rk delta)^T and E = 1 (k re-read
  // from LDS rather than held across the barrier: fewer VGPRs)
  const float4* k4 = reinterpret_cast<const float4*>(ks + rg * RPT);
  if constexpr (!DEFER) {
    float d2[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) d2[c] = dl[c] * nr.rk;
#pragma unroll
    for (int i4 = 0; i4 < RPT / 4; ++i4) {
      const float4 kk = k4[i4];
      const float kr[4] = {kk.x, kk.y, kk.z, kk.w};
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int c = 0; c < 4; ++c) S[4 * i4 + u][c] = fmaf(e, S[4 * i4 + u][c], kr[u] * d2[c]);
    }
    return;
  }
  const float En = uni(e * E);
  const bool keep = En >= kStateScaleMin;
  const float f = uni(keep ? nr.rk * __builtin_amdgcn_rcpf(En) : nr.rk);   // En >= 2^-64: a normal number
  float d2[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) d2[c] = dl[c] * f;
  if (!keep) {   // fold E' into St (a uniform branch)
#pragma unroll
    for (int i = 0; i < RPT; ++i)
#pragma unroll
      for (int c = 0; c < 4; ++c) S[i][c] *= En;
  }
#pragma unroll
  for (int i4 = 0; i4 < RPT / 4; ++i4) {
    const float4 kk = k4[i4];
    const float kr[4] = {kk.x, kk.y, kk.z, kk.w};
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int c = 0; c < 4; ++c) S[4 * i4 + u][c] = fmaf(kr[u], d2[c], S[4 * i4 + u][c]);
  }
  E = uni(keep ? En : 1.0f);
}
// The direct forms, for launches of one token per sequence (no cu_seqlens):
// k and q in LDS in natural row order, scaled by the norms row by row, and
// S' = e S + k_hat delta^T in place (one multiply and one fma per element;
// with a single token the scaled state saves nothing, and these measured
// faster there).
__device__ __forceinline__ RecNorms rec_pass_direct(const float (&S)[RPT][4], const float* ks, const float* qs, float* red,
                                             int t256, float scale, int l2) {
  const int lane = t256 & 63, wave = t256 >> 6, cg = t256 % CGN, rg = t256 / CGN;
  // norms and k.q, redundantly per wave (no extra barrier)
  const float k0 = ks[2 * lane], k1 = ks[2 * lane + 1];
  const float q0 = qs[2 * lane], q1 = qs[2 * lane + 1];
  const float skk = wave_sum(k0 * k0 + k1 * k1);
  const float sqq = wave_sum(q0 * q0 + q1 * q1);
  const float sqk = wave_sum(q0 * k0 + q1 * k1);
  const float rk = l2 ? 1.0f / sqrtf(skk + 1e-6f) : 1.0f;
  const float rq = (l2 ? 1.0f / sqrtf(sqq + 1e-6f) : 1.0f) * scale;
  const float kq = sqk * rk * rq;

  float pa[4] = {0.f, 0.f, 0.f, 0.f}, pb[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const float kh = ks[rg + RGN * i] * rk;
    const float qh = qs[rg + RGN * i] * rq;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      pa[c] = fmaf(S[i][c], kh, pa[c]);
      pb[c] = fmaf(S[i][c], qh, pb[c]);
    }
  }
  // the two row groups of a wave sit in lanes l and l ^ 32
#pragma unroll
  for (int x = CGN; x < 64; x <<= 1) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      pa[c] += __shfl_xor(pa[c], x, 64);
      pb[c] += __shfl_xor(pb[c], x, 64);
    }
  }
  if (lane < CGN) {
    *reinterpret_cast<float4*>(red + (wave * 2 + 0) * D + 4 * cg) = make_float4(pa[0], pa[1], pa[2], pa[3]);
    *reinterpret_cast<float4*>(red + (wave * 2 + 1) * D + 4 * cg) = make_float4(pb[0], pb[1], pb[2], pb[3]);
  }
  return {rk, rq, kq};
}
template <typename TO>
__device__ __forceinline__ void rec_finish_direct(float (&S)[RPT][4], const float* ks, const float (&vv)[4], float gt,
                                           float bt, const float* red, int t256, RecNorms nr, TO* __restrict__ o,
                                           int64_t ob) {
  const int cg = t256 % CGN, rg = t256 / CGN;
  const float rk = nr.rk, kq = nr.kq;
  const float e = expf(gt);
  float a4[4] = {0.f, 0.f, 0.f, 0.f}, b4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const float4 ra = *reinterpret_cast<const float4*>(red + (w * 2 + 0) * D + 4 * cg);
    const float4 rb = *reinterpret_cast<const float4*>(red + (w * 2 + 1) * D + 4 * cg);
    a4[0] += ra.x; a4[1] += ra.y; a4[2] += ra.z; a4[3] += ra.w;
    b4[0] += rb.x; b4[1] += rb.y; b4[2] += rb.z; b4[3] += rb.w;
  }
  float dl[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) dl[c] = bt * (vv[c] - e * a4[c]);
  if (rg == 0) {
#pragma unroll
    for (int c = 0; c < 4; ++c) Elem<TO>::store(o, ob + c, fmaf(e, b4[c], kq * dl[c]));
  }
  // (k re-read from LDS rather than held across the barrier: fewer VGPRs,
  // one more workgroup per CU)
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const float kh = ks[rg + RGN * i] * rk;
#pragma unroll
    for (int c = 0; c < 4; ++c) S[i][c] = fmaf(e, S[i][c], kh * dl[c]);
  }
}
template <typename TO, bool DEFER>
__device__ __forceinline__ void rec_token(float (&S)[RPT][4], float& E, const float* ks, const float* qs,
                                          const float (&vv)[4], float gt, float bt, float* red, int t256, float scale,
                                          int l2, TO* __restrict__ o, int64_t ob) {
  if constexpr (DEFER) {
    const RecNorms nr = rec_pass(S, ks, qs, red, t256, scale, l2);
    __syncthreads();
    rec_finish<TO, DEFER>(S, E, ks, vv, gt, bt, red, t256, nr, o, ob);
  } else {
    const RecNorms nr = rec_pass_direct(S, ks, qs, red, t256, scale, l2);
    __syncthreads();
    rec_finish_direct<TO>(S, ks, vv, gt, bt, red, t256, nr, o, ob);
  }
}

// G consecutive (sequence, value head) states per workgroup, 256 threads
// each; G divides nv, so all G belong to one sequence and run the same
// token loop (its barriers are the whole workgroup's).
template <typename TIn, typename TO, int G, bool DEFER>
__global__ void __launch_bounds__(256 * G) __attribute__((amdgpu_waves_per_eu(4)))
recurrent_kernel(const TIn* __restrict__ q, const TIn* __restrict__ k, const TIn* __restrict__ v, int64_t qs,
                 int64_t ks, int64_t vs, const float* __restrict__ g, const float* __restrict__ beta,
                 const int32_t* __restrict__ cu, int64_t T, int nk, int nv, float scale, int l2,
                 float* __restrict__ state, TO* __restrict__ o) {
  __shared__ __attribute__((aligned(16))) float kq_s[2][G][2][D];    // [parity][state][k|q][kq_slot]
  __shared__ float red[2][G][4][2][D];  // [parity][state][wave][a|b][column]

  const int tid = threadIdx.x, t256 = tid & 255;
  const int rho = __builtin_amdgcn_readfirstlane(tid >> 8);
  const int unit = blockIdx.x * G + rho;   // n * nv + h
  const int n = unit / nv;
  const int h = unit % nv;
  const int hk = h / (nv / nk);
  const int col = 4 * (t256 % CGN);     // first of this thread's 4 columns

  int64_t t0, t1;
  if (cu) seq_bounds(cu, n, T, t0, t1);
  else { t0 = n; t1 = n + 1; }   // one token per sequence (T == n_seqs)

  // a token's inputs for this thread, as loaded (converted at use: any
  // arithmetic at load time would wait for the load right there): one
  // element of k (threads < 128 of the state's group) or of q, 4 of v, g and beta
  TIn kq_n{}, vv_n[4] = {};
  float gt_n = 0.f, bt_n = 0.f;
  auto load_token = [&](int64_t t) {
    kq_n = t256 < D ? k[t * ks + static_cast<int64_t>(hk) * D + t256]
                    : q[t * qs + static_cast<int64_t>(hk) * D + (t256 - D)];
#pragma unroll
    for (int c = 0; c < 4; ++c) vv_n[c] = v[t * vs + static_cast<int64_t>(h) * D + col + c];
    gt_n = g[t * nv + h];
    bt_n = beta[t * nv + h];
  };
  // the first token's inputs go out before the state stream: completions are
  // counted in order, so the norms below then wait only for these
  if (t0 < t1) load_token(t0);

  float* Sp = state + static_cast<int64_t>(unit) * D * D;
  // The state streams through once each way. It is read with ordinary loads
  // and written back non-temporally (each state is touched once per call);
  // of the four load/store hint combinations this one streams fastest.
  // (Written out in each kernel: as a shared helper the compiler kept all
  // sixteen row addresses live across the token loop, 40 more VGPRs.)
  float S[RPT][4];
  {
    const int rg = t256 / CGN;
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const f32x4 s4 = *reinterpret_cast<const f32x4*>(Sp + (rg + RGN * i) * D + col);
      S[i][0] = s4[0]; S[i][1] = s4[1]; S[i][2] = s4[2]; S[i][3] = s4[3];
    }
  }

  float E = 1.0f;   // S = E St (see kStateScaleMin)
  int par = 0;
  for (int64_t t = t0; t < t1; ++t, par ^= 1) {
    const float kqv = Elem<TIn>::cvt(kq_n), gt = DEFER ? uni(gt_n) : gt_n, bt = DEFER ? uni(bt_n) : bt_n;
    float vv[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) vv[c] = Elem<TIn>::cvt(vv_n[c]);
    if (t + 1 < t1) load_token(t + 1);   // the next token's inputs
    // stage k and q of this token's key head in LDS (fp32)
    kq_s[par][rho][t256 < D ? 0 : 1][DEFER ? kq_slot(t256 & (D - 1)) : t256 & (D - 1)] = kqv;
    __syncthreads();
    rec_token<TO, DEFER>(S, E, kq_s[par][rho][0], kq_s[par][rho][1], vv, gt, bt, &red[par][rho][0][0][0], t256, scale, l2,
                  o, t * static_cast<int64_t>(nv) * D + static_cast<int64_t>(h) * D + col);
  }
  if constexpr (DEFER) {
#pragma unroll
    for (int i = 0; i < RPT; ++i)   // S = E St
#pragma unroll
      for (int c = 0; c < 4; ++c) S[i][c] *= E;
  }
  {
    const int rg = t256 / CGN;
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      f32x4 s4;
      s4[0] = S[i][0]; s4[1] = S[i][1]; s4[2] = S[i][2]; s4[3] = S[i][3];
      __builtin_nontemporal_store(s4, reinterpret_cast<f32x4*>(Sp + (rg + RGN * i) * D + col));
    }
  }
}

// Fused decode step, R value heads per key head. Local channel j of the
// workgroup: q of key head hk (j < 128), its k (j < 256), then v of value
// heads R hk .. R hk + R - 1; one or two channels per thread. The gating
// inputs are wave-uniform (one value head per wave), so every thread computes
// g and beta itself from scalar loads.
template <typename T, typename TO, int R, bool SNAP, bool DEFER>
__global__ void __launch_bounds__(256 * R) __attribute__((amdgpu_waves_per_eu(R == 1 ? 3 : 4)))
decode_fused_kernel(const T* __restrict__ x, int64_t xs, T* __restrict__ cst, int state_len,
                    const float* __restrict__ cw, const float* __restrict__ cb, const T* __restrict__ a,
                    const T* __restrict__ b, const float* __restrict__ A_log, const float* __restrict__ dt_bias,
                    const int32_t* __restrict__ cu, int64_t T_tot, int nk, int nv, float scale, int l2,
                    float* __restrict__ state, const int32_t* __restrict__ slots, int n_slots,
                    float* __restrict__ snap, TO* __restrict__ o) {
  constexpr int NCH = (2 + R) * D;
  constexpr int NT = 256 * R;
  constexpr int CPT = (NCH + NT - 1) / NT;
  constexpr int KW = 4;
  __shared__ __attribute__((aligned(16))) float kqv_s[3][NCH];   // [token % 3][q | k (kq_slot) | v]: conv outputs
  __shared__ float red[2][R][4][2][D];  // [parity][value head][wave][a|b][column]

  const int n = blockIdx.x / nk, hk = blockIdx.x % nk;
  // the sequence's slot in the state pools; a negative slot (padding) or one
  // past the pool leaves the sequence untouched (the whole workgroup returns)
  const int slot = slots ? slots[n] : n;
  if (slot < 0 || slot >= n_slots) return;
  const int tid = threadIdx.x, t256 = tid & 255;
  const int rho = __builtin_amdgcn_readfirstlane(tid >> 8);
  const int h = hk * R + rho;
  const int col = 4 * (t256 % CGN);
  const int conv_dim = (2 * nk + nv) * D;
  // global channel of local channel j
  auto chan = [&](int j) {
    return j < D ? hk * D + j : (j < 2 * D ? nk * D + hk * D + (j - D) : 2 * nk * D + hk * R * D + (j - 2 * D));
  };

  int64_t t0, t1;
  if (cu) seq_bounds(cu, n, T_tot, t0, t1);
  else { t0 = n; t1 = n + 1; }

  // this thread's conv windows (the last K-1 inputs) and first inputs, loaded
  // ahead of the state stream (completions are counted in order)
  float hist[CPT][KW - 1];
  T x_n[CPT];
#pragma unroll
  for (int u = 0; u < CPT; ++u) {
    const int j = tid + u * NT;
    if (j < NCH) {
      const T* sp = cst + (static_cast<int64_t>(slot) * conv_dim + chan(j)) * state_len + (state_len - (KW - 1));
#pragma unroll
      for (int i = 0; i < KW - 1; ++i) hist[u][i] = Elem<T>::load(sp, i);
      if (t0 < t1) x_n[u] = x[t0 * xs + chan(j)];
    }
  }
  const float alog = A_log[h], dtb = dt_bias[h];
  T a_n{}, b_n{};
  if (t0 < t1) { a_n = a[t0 * nv + h]; b_n = b[t0 * nv + h]; }

  float* Sp = state + (static_cast<int64_t>(slot) * nv + h) * D * D;
  // the state stream, as in the recurrent kernel
  float S[RPT][4];
  {
    const int rg = t256 / CGN;
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const f32x4 s4 = *reinterpret_cast<const f32x4*>(Sp + (rg + RGN * i) * D + col);
      S[i][0] = s4[0]; S[i][1] = s4[1]; S[i][2] = s4[2]; S[i][3] = s4[3];
    }
  }

  // conv update + SiLU of token t into kqv_s[buf], in the order of the
  // separate kernel; prefetches the next token's inputs
  auto conv_token = [&](int64_t t, int buf) {
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      const int j = tid + u * NT;
      if (j < NCH) {
        const int c = chan(j);
        const float xv = Elem<T>::cvt(x_n[u]);
        if (t + 1 < t1) x_n[u] = x[(t + 1) * xs + c];
        float acc = cb ? cb[c] : 0.0f;
#pragma unroll
        for (int i = 0; i < KW - 1; ++i) acc = fmaf(cw[c * KW + i], hist[u][i], acc);
        acc = fmaf(cw[c * KW + KW - 1], xv, acc);
        kqv_s[buf][DEFER && j < 2 * D ? (j & ~(D - 1)) + kq_slot(j & (D - 1)) : j] = act_round(siluf_(acc), T{});
#pragma unroll
        for (int i = 0; i + 1 < KW - 1; ++i) hist[u][i] = hist[u][i + 1];
        hist[u][KW - 2] = xv;
      }
    }
  };
  // One barrier per token: the conv of token t + 1 is formed before the
  // barrier that completes token t's reductions. kqv_s rotates over three
  // buffers and red over two, so no buffer is rewritten while a thread that
  // is one phase behind may still read it.
  if (t0 < t1) conv_token(t0, 0);
  __syncthreads();
  float E = 1.0f;   // S = E St (see kStateScaleMin)
  int buf = 0, par = 0;
  for (int64_t t = t0; t < t1; ++t) {
    // gating, as the separate gating kernel computes it
    const float av = Elem<T>::cvt(a_n), bv = Elem<T>::cvt(b_n);
    if (t + 1 < t1) { a_n = a[(t + 1) * nv + h]; b_n = b[(t + 1) * nv + h]; }
    float gt = -exp_(alog) * softplusf_(av + dtb);
    float bt = sigmoidf_(bv);
    if constexpr (DEFER) {   // wave-uniform: scalar registers
      gt = uni(gt);
      bt = uni(bt);
    }
    float* rd = &red[par][rho][0][0][0];
    RecNorms nr;
    if constexpr (DEFER)
      nr = rec_pass(S, &kqv_s[buf][D], &kqv_s[buf][0], rd, t256, scale, l2);
    else
      nr = rec_pass_direct(S, &kqv_s[buf][D], &kqv_s[buf][0], rd, t256, scale, l2);
    const int nbuf = buf == 2 ? 0 : buf + 1;
    if (t + 1 < t1) conv_token(t + 1, nbuf);
    __syncthreads();
    const float4 v4 = *reinterpret_cast<const float4*>(&kqv_s[buf][2 * D + rho * D + col]);
    const float vv[4] = {v4.x, v4.y, v4.z, v4.w};
    if constexpr (DEFER)
      rec_finish<TO, DEFER>(S, E, &kqv_s[buf][D], vv, gt, bt, rd, t256, nr, o,
                            t * static_cast<int64_t>(nv) * D + static_cast<int64_t>(h) * D + col);
    else
      rec_finish_direct<TO>(S, &kqv_s[buf][D], vv, gt, bt, rd, t256, nr, o,
                            t * static_cast<int64_t>(nv) * D + static_cast<int64_t>(h) * D + col);
    if constexpr (SNAP) {   // the state after this token, for rolling back rejected draft tokens
      // (buffer stores off one per-lane offset: the row addresses are not kept live)
      const rsrc_t rs = make_rsrc(snap + (t * nv + h) * static_cast<int64_t>(D) * D, D * D * 4);
      const uint32_t vo = static_cast<uint32_t>(((t256 / CGN) * D + col) * 4);
#pragma unroll
      for (int i = 0; i < RPT; ++i)
        bstore16_nt(rs, vo + static_cast<uint32_t>(RGN * D * 4 * i),
                    make_uint4(__float_as_uint(S[i][0] * E), __float_as_uint(S[i][1] * E),
                               __float_as_uint(S[i][2] * E), __float_as_uint(S[i][3] * E)));
    }
    buf = nbuf;
    par ^= 1;
  }
  if constexpr (DEFER) {
#pragma unroll
    for (int i = 0; i < RPT; ++i)   // S = E St
#pragma unroll
      for (int c = 0; c < 4; ++c) S[i][c] *= E;
  }
  {
    const int rg = t256 / CGN;
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      f32x4 s4;
      s4[0] = S[i][0]; s4[1] = S[i][1]; s4[2] = S[i][2]; s4[3] = S[i][3];
      __builtin_nontemporal_store(s4, reinterpret_cast<f32x4*>(Sp + (rg + RGN * i) * D + col));
    }
  }

  // conv state <- last state_len entries of [old state, this sequence's x]:
  // entry s reads old entry L + s (not yet overwritten, L >= 1) or an input
  const int64_t L = t1 - t0;
  if (L > 0) {
#pragma unroll
    for (int u = 0; u < CPT; ++u) {
      const int j = tid + u * NT;
      if (j < NCH) {
        const int c = chan(j);
        T* sp = cst + (static_cast<int64_t>(slot) * conv_dim + c) * state_len;
        for (int s = 0; s < state_len; ++s) {
          const int64_t idx = L + s;
          sp[s] = idx < state_len ? sp[idx] : x[(t0 + idx - state_len) * xs + c];
        }
      }
    }
  }
}

template <typename TIn, typename TO, int G>
hipError_t rec_launch(const void* q, const void* k, const void* v, int64_t qs, int64_t ks, int64_t vs,
                      const float* g, const float* beta, const int32_t* cu, int n_seqs, int64_t T, int nk, int nv,
                      float scale, int l2, float* state, void* o, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(n_seqs) * static_cast<unsigned>(nv / G));
  auto kern = cu ? recurrent_kernel<TIn, TO, G, true> : recurrent_kernel<TIn, TO, G, false>;
  kern<<<grid, 256 * G, 0, s>>>(static_cast<const TIn*>(q), static_cast<const TIn*>(k), static_cast<const TIn*>(v), qs,
                                ks, vs, g, beta, cu, T, nk, nv, scale, l2, state, static_cast<TO*>(o));
  return hipGetLastError();
}

template <typename TIn>
hipError_t rec_dispatch(const void* q, const void* k, const void* v, int64_t qs, int64_t ks, int64_t vs,
                        const float* g, const float* beta, const int32_t* cu, int n_seqs, int64_t T, int nk,
                        int nv, float scale, int l2, float* state, void* o, int o_bf16, hipStream_t s) {
  // Two states per workgroup when nv is even: measured in the decode step at
  // 256 x 32 states, 6.1 TB/s against 5.5 TB/s with one state per workgroup
  // and 5.9 TB/s with four (each workgroup then writes 128 KB of contiguous
  // state at its end, and half as many workgroups are scheduled).
  constexpr int G = 2;
  if (nv % G == 0)
    return o_bf16 ? rec_launch<TIn, uint16_t, G>(q, k, v, qs, ks, vs, g, beta, cu, n_seqs, T, nk, nv, scale, l2, state, o, s)
                  : rec_launch<TIn, float, G>(q, k, v, qs, ks, vs, g, beta, cu, n_seqs, T, nk, nv, scale, l2, state, o, s);
  return o_bf16 ? rec_launch<TIn, uint16_t, 1>(q, k, v, qs, ks, vs, g, beta, cu, n_seqs, T, nk, nv, scale, l2, state, o, s)
                : rec_launch<TIn, float, 1>(q, k, v, qs, ks, vs, g, beta, cu, n_seqs, T, nk, nv, scale, l2, state, o, s);
}

template <typename T, typename TO, int R>
hipError_t fused_launch(const void* x, int64_t xs, void* cst, int state_len, const float* cw, const float* cb,
                        const void* a, const void* b, const float* A_log, const float* dt_bias, const int32_t* cu,
                        int n_seqs, int64_t T_tot, int nk, int nv, float scale, int l2, float* state,
                        const int32_t* slots, int n_slots, float* snap, void* o, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(n_seqs) * static_cast<unsigned>(nk));
  // snapshots are a separate instantiation: their stores inside the token
  // loop would otherwise cost the plain step about 30 spilled VGPRs
  auto kern = snap ? (cu ? decode_fused_kernel<T, TO, R, true, true> : decode_fused_kernel<T, TO, R, true, false>)
                   : (cu ? decode_fused_kernel<T, TO, R, false, true> : decode_fused_kernel<T, TO, R, false, false>);
  kern<<<grid, 256 * R, 0, s>>>(static_cast<const T*>(x), xs, static_cast<T*>(cst), state_len, cw, cb,
                                static_cast<const T*>(a), static_cast<const T*>(b), A_log, dt_bias, cu, T_tot, nk, nv,
                                scale, l2, state, slots, n_slots, snap, static_cast<TO*>(o));
  return hipGetLastError();
}

template <typename T, typename TO>
hipError_t fused_dispatch_r(int r, const void* x, int64_t xs, void* cst, int state_len, const float* cw,
                            const float* cb, const void* a, const void* b, const float* A_log, const float* dt_bias,
                            const int32_t* cu, int n_seqs, int64_t T_tot, int nk, int nv, float scale, int l2,
                            float* state, const int32_t* slots, int n_slots, float* snap, void* o, hipStream_t s) {
  switch (r) {
    case 1: return fused_launch<T, TO, 1>(x, xs, cst, state_len, cw, cb, a, b, A_log, dt_bias, cu, n_seqs, T_tot,
                                          nk, nv, scale, l2, state, slots, n_slots, snap, o, s);
    case 2: return fused_launch<T, TO, 2>(x, xs, cst, state_len, cw, cb, a, b, A_log, dt_bias, cu, n_seqs, T_tot,
                                          nk, nv, scale, l2, state, slots, n_slots, snap, o, s);
    case 4: return fused_launch<T, TO, 4>(x, xs, cst, state_len, cw, cb, a, b, A_log, dt_bias, cu, n_seqs, T_tot,
                                          nk, nv, scale, l2, state, slots, n_slots, snap, o, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_decode_fused(const void* x, int bf16, int64_t x_stride, void* conv_state, int state_len,
                               const float* conv_w, const float* conv_b, const void* a, const void* b,
                               const float* A_log, const float* dt_bias, const int32_t* cu, int n_seqs, int64_t T_tot,
                               int nk, int nv, float scale, int l2, float* state, const int32_t* slots, int n_slots,
                               float* snap, void* o, int o_bf16, hipStream_t s) {
  const int r = nv / nk;
  if (bf16)
    return o_bf16 ? fused_dispatch_r<uint16_t, uint16_t>(r, x, x_stride, conv_state, state_len, conv_w, conv_b, a, b,
                                                         A_log, dt_bias, cu, n_seqs, T_tot, nk, nv, scale, l2, state,
                                                         slots, n_slots, snap, o, s)
                  : fused_dispatch_r<uint16_t, float>(r, x, x_stride, conv_state, state_len, conv_w, conv_b, a, b,
                                                      A_log, dt_bias, cu, n_seqs, T_tot, nk, nv, scale, l2, state,
                                                      slots, n_slots, snap, o, s);
  return o_bf16 ? fused_dispatch_r<float, uint16_t>(r, x, x_stride, conv_state, state_len, conv_w, conv_b, a, b,
                                                    A_log, dt_bias, cu, n_seqs, T_tot, nk, nv, scale, l2, state, slots,
                                                    n_slots, snap, o, s)
                : fused_dispatch_r<float, float>(r, x, x_stride, conv_state, state_len, conv_w, conv_b, a, b, A_log,
                                                 dt_bias, cu, n_seqs, T_tot, nk, nv, scale, l2, state, slots, n_slots,
                                                 snap, o, s);
}

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
