// k_chunk.hip -- chunked gated delta rule (prefill path), chunk = 64, dk = dv = 128.
//
// "Qwen3.5 Simulation Support Design Document" (2.2 op 4, Appendix B) splits
// the sequence into chunks of 64 tokens: attention inside a chunk plus a
// recurrence between chunks. The pages give no algebra; the form used here is
// derived from the token recurrence of "Qwen3.5 Dense Model Architecture",
// Linear Attention (decay, then delta update on the decayed state, then the
// read-out). Per chunk of C tokens with state S at its start, G the
// chunk-local cumulative sum of g, kh = rk * k, qh = rq * scale * q:
//
//   A_ij  = beta_i rk_i rk_j exp(G_i - G_j) (k_i . k_j)     j < i
//   T     = (I + A)^-1                                       (unit lower)
//   R_i   = beta_i v_i - beta_i rk_i exp(G_i) (K S)_i
//   U     = T R                                              (new values)
//   O_i   = scale rq_i exp(G_i) (Q S)_i + sum_{j<=i} P_ij U_j,
//           P_ij = scale rq_i rk_j exp(G_i - G_j) (q_i . k_j)
//   S'    = exp(G_C) S + K^T diag(rk_j exp(G_C - G_j)) U
//
// Only exponents <= 0 are ever formed (masked before exp), and G is summed in
// fp64 so that G_i - G_j keeps full fp32 precision when |G| reaches 1e3.
//
// Kernels:
//   chunk_offsets : exclusive prefix of ceil(len/64) over sequences (varlen
//                   chunk table on the device; no host synchronisation).
//   chunk_prep    : one wave per (chunk, value head), fully parallel. Grams
//                   K K^T and Q K^T on MFMA from the raw inputs (exact
//                   operands, kept in registers), fp64 cumsum of g, A, the
//                   blocked inverse T (16x16 diagonal blocks by substitution,
//                   off-diagonal blocks on MFMA), P and per-token scalars.
//                   Output per (chunk, value head): one packed 64x64 fp32
//                   tile X with X[i][j] = T[i][j] for j < i and
//                   X[63-i][63-j] = P[i][j] for j <= i (P turned by 180
//                   degrees into the upper triangle), so rows of both T and
//                   P are contiguous; plus 64 float4 scalars and exp(G_C).
//   chunk_state   : sequential over a sequence's chunks. bf16 inputs: four
//                   waves per (sequence, value head, 16 value columns); wave
//                   w holds rows 32w..32w+31 of S (128 x 16, fp32) in MFMA
//                   accumulators and computes token rows 16w..16w+15 of the
//                   chunk; S is exchanged through LDS once per chunk. Q, T,
//                   P and V operands are loaded straight into registers in
//                   MFMA fragment layout one chunk ahead; K is staged in LDS
//                   (double-buffered) because the state update reads it
//                   transposed. fp32 inputs use a simple one-wave variant.
//                   Products with an fp32 operand split it into bf16 hi + lo.
#include "gdn_device.hpp"
#include "gdn_internal.hpp"

namespace gdn {
namespace {

constexpr int CH = 64;     // chunk length
constexpr int D = 128;     // dk = dv
constexpr int AP = 68;     // LDS pitch (floats) of 64 x 64 fp32 tiles (16-byte rows)
constexpr float kEps = 1e-6f;

struct WsLayout {
  size_t off_chunk_off, off_tp, off_sc, off_egc, total;
};
inline WsLayout ws_layout(int64_t T, int n_seqs, int nv) {
  const int64_t nch = T / CH + n_seqs;   // >= sum_n ceil(len_n / 64)
  WsLayout w{};
  size_t o = 0;
  w.off_chunk_off = o; o += (static_cast<size_t>(n_seqs) + 1) * sizeof(int32_t); o = (o + 255) & ~size_t(255);
  w.off_tp = o;        o += static_cast<size_t>(nch) * nv * CH * CH * sizeof(float);
  w.off_sc = o;        o += static_cast<size_t>(nch) * nv * CH * sizeof(float4);
  w.off_egc = o;       o += static_cast<size_t>(nch) * nv * sizeof(float); o = (o + 255) & ~size_t(255);
  w.total = o;
  return w;
}

// ------------------------------------------------------------------ chunk table
// Capped at nch (the workspace's chunk capacity) so a malformed cu_seqlens can
// never index past the workspace.
__global__ void __launch_bounds__(256) chunk_offsets_kernel(const int32_t* __restrict__ cu, int n_seqs,
                                                            int64_t T, int32_t nch, int32_t* __restrict__ off) {
  __shared__ int32_t part[256];
  const int tid = threadIdx.x;
  int32_t carry = 0;
  for (int base = 0; base < n_seqs; base += 256) {
    const int n = base + tid;
    int32_t c = 0;
    if (n < n_seqs) {
      int64_t b, e;
      seq_bounds(cu, n, T, b, e);
      c = static_cast<int32_t>((e - b + CH - 1) / CH);
    }
    part[tid] = c;
    __syncthreads();
    for (int d = 1; d < 256; d <<= 1) {   // inclusive Hillis-Steele scan
      const int32_t add = tid >= d ? part[tid - d] : 0;
      __syncthreads();
      part[tid] += add;
      __syncthreads();
    }
    if (n < n_seqs) off[n] = min(carry + part[tid] - c, nch);
    carry = min(carry + part[255], nch);
    __syncthreads();
  }
  if (tid == 0) off[n_seqs] = min(carry, nch);
}

__device__ __forceinline__ int find_le(const int32_t* a, int n, int64_t x) {
  // largest i in [0, n-1] with a[i] <= x
  int lo = 0, hi = n - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (a[mid] <= x) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Raw copies of 8 input elements (16 bytes of bf16 or 32 bytes of fp32).
__device__ __forceinline__ void copy8(const uint16_t* src, uint16_t* dst) {
  *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(src);
}
__device__ __forceinline__ void copy8(const float* src, float* dst) {
  *reinterpret_cast<float4*>(dst) = *reinterpret_cast<const float4*>(src);
  *reinterpret_cast<float4*>(dst + 4) = *reinterpret_cast<const float4*>(src + 4);
}
__device__ __forceinline__ uint4 zero_if(bool z, uint4 u) {
  return z ? make_uint4(0, 0, 0, 0) : u;
}
__device__ __forceinline__ float4 zero_if(bool z, float4 u) {
  return z ? make_float4(0.f, 0.f, 0.f, 0.f) : u;
}
__device__ __forceinline__ void copy8_or_zero(const uint16_t* src, uint16_t* dst, bool z) {
  *reinterpret_cast<uint4*>(dst) = zero_if(z, *reinterpret_cast<const uint4*>(src));
}
__device__ __forceinline__ void copy8_or_zero(const float* src, float* dst, bool z) {
  *reinterpret_cast<float4*>(dst) = zero_if(z, *reinterpret_cast<const float4*>(src));
  *reinterpret_cast<float4*>(dst + 4) = zero_if(z, *reinterpret_cast<const float4*>(src + 4));
}
__device__ __forceinline__ float tof(uint16_t x) { return bf16_to_f32(x); }
__device__ __forceinline__ float tof(float x) { return x; }

// x = hi + lo with hi = bf16(x), lo = bf16(x - hi); four values packed into
// two dwords per plane (element 0 in the low half of the first dword).
typedef float f32x2v __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void split2(f32x2v x, uint32_t& hi, uint32_t& lo) {
  const bf16x2v h = __builtin_convertvector(x, bf16x2v);
  const f32x2v hf = __builtin_convertvector(h, f32x2v);
  const f32x2v r = {x.x - hf.x, x.y - hf.y};
  hi = __builtin_bit_cast(uint32_t, h);
  lo = __builtin_bit_cast(uint32_t, __builtin_convertvector(r, bf16x2v));
}
__device__ __forceinline__ void split4_packed(float4 x, uint2& hi, uint2& lo) {
  split2(f32x2v{x.x, x.y}, hi.x, lo.x);
  split2(f32x2v{x.z, x.w}, hi.y, lo.y);
}

// lower 16x16 tiles of a 64x64 matrix, p = 0..9 -> (mi, mj), mi >= mj
__device__ __forceinline__ int tile_mi(int p) { return p >= 6 ? 3 : p >= 3 ? 2 : p >= 1 ? 1 : 0; }
__device__ __forceinline__ int tile_mj(int p) { const int mi = tile_mi(p); return p - mi * (mi + 1) / 2; }

// acc += A(16x16) * B(16x16), both fp32 in LDS (row pitches lda, ldb).
template <bool BF>
__device__ __forceinline__ void mm16(f32x4& acc, const float* A, int lda, const float* B, int ldb, int lr, int lg) {
  using M = Mma16<BF, false, false>;
#pragma unroll
  for (int s = 0; s < 16 / M::KS; ++s) {
    float a[M::KPL], b[M::KPL];
#pragma unroll
    for (int j = 0; j < M::KPL; ++j) {
      const int kk = s * M::KS + M::KPL * lg + j;
      a[j] = A[lr * lda + kk];
      b[j] = B[kk * ldb + lr];
    }
    M::run(acc, a, b);
  }
}

// ------------------------------------------------------------------ prep
template <typename TIn>
constexpr int prep_pitch() { return sizeof(TIn) == 2 ? 136 : 132; }   // 16-byte rows
template <typename TIn>
constexpr size_t prep_lds_bytes() {
  constexpr size_t tiles = 2 * CH * prep_pitch<TIn>() * sizeof(TIn);
  constexpr size_t at = 2 * CH * AP * sizeof(float);
  return (tiles > at ? tiles : at) + CH * sizeof(double) + 4 * CH * sizeof(float) + 16 * 20 * sizeof(float);
}

template <typename TIn>
__global__ void __launch_bounds__(64) chunk_prep_kernel(
    const TIn* __restrict__ q, const TIn* __restrict__ k, int64_t qs, int64_t ks,
    const float* __restrict__ g, const float* __restrict__ beta, const int32_t* __restrict__ cu,
    int n_seqs, int64_t T, int nk, int nv, float scale, int l2, const int32_t* __restrict__ chunk_off,
    float* __restrict__ tp, float4* __restrict__ sc, float* __restrict__ egc) {
  constexpr bool BF = sizeof(TIn) == 2;
  constexpr int EP = prep_pitch<TIn>();
  using MG = Mma<BF, true, true>;
  constexpr int KS = MG::KS, KPL = MG::KPL;
  constexpr size_t tiles = 2 * CH * EP * sizeof(TIn);
  constexpr size_t at = 2 * CH * AP * sizeof(float);
  constexpr size_t head = tiles > at ? tiles : at;

  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  TIn* Ks = reinterpret_cast<TIn*>(smem);          // [64][EP]   (input tiles)
  TIn* Qs = Ks + CH * EP;                          // [64][EP]
  float* Aw = reinterpret_cast<float*>(smem);      // [64][AP]   (after the Grams)
  float* Tw = Aw + CH * AP;                        // [64][AP]
  double* Gs = reinterpret_cast<double*>(smem + head);
  float* rk_s = reinterpret_cast<float*>(Gs + CH);
  float* rq_s = rk_s + CH;
  float* b_s = rq_s + CH;
  float* scr = b_s + 2 * CH;                       // [16][20] scratch

  const int c = blockIdx.x;
  const int h = blockIdx.y;
  const int hk = h / (nv / nk);
  const int total = chunk_off[n_seqs];
  if (c >= total) return;
  const int n = find_le(chunk_off, n_seqs, c);
  int64_t s_begin, s_end;
  seq_bounds(cu, n, T, s_begin, s_end);
  const int64_t t0 = s_begin + static_cast<int64_t>(c - chunk_off[n]) * CH;
  const int L = static_cast<int>(min<int64_t>(CH, s_end - t0));
  const int lane = threadIdx.x, lr = lane & 15, lg = lane >> 4;

  // 1. K and Q tiles into LDS (rows >= L zero); 4 rows per instruction
  {
    const TIn* kb = k + t0 * ks + static_cast<int64_t>(hk) * D;
    const TIn* qb = q + t0 * qs + static_cast<int64_t>(hk) * D;
#pragma unroll
    for (int it = 0; it < 16; ++it) {
      const int idx = it * 64 + lane, row = idx >> 4, seg = idx & 15;
      // rows past the sequence end re-read the last valid row: their norms
      // are forced to 0 below, so they contribute nothing to A, P or scalars
      const int rr = min(row, L - 1);
      copy8(kb + rr * ks + seg * 8, Ks + row * EP + seg * 8);
      copy8(qb + rr * qs + seg * 8, Qs + row * EP + seg * 8);
    }
  }
  __syncthreads();

  // 2. |q_i|^2 (lane = row)
  float sqq = 0.f;
#pragma unroll 8
  for (int e = 0; e < D; ++e) {
    const float x = tof(Qs[lane * EP + e]);
    sqq = fmaf(x, x, sqq);
  }
  // 3. Grams on the lower 16x16 tiles, kept in registers
  f32x4 gkk[10], gqk[10];
#pragma unroll
  for (int p = 0; p < 10; ++p) {
    const int mi = tile_mi(p), mj = tile_mj(p);
    gkk[p] = f32x4{0.f, 0.f, 0.f, 0.f};
    gqk[p] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < D / KS; ++s) {
      if constexpr (BF) {   // raw bf16 fragments, one 16-byte LDS read each
        const int kk = s * KS + KPL * lg;
        const bf16x8 ak = *reinterpret_cast<const bf16x8*>(Ks + (16 * mi + lr) * EP + kk);
        const bf16x8 aq = *reinterpret_cast<const bf16x8*>(Qs + (16 * mi + lr) * EP + kk);
        const bf16x8 bk = *reinterpret_cast<const bf16x8*>(Ks + (16 * mj + lr) * EP + kk);
        gkk[p] = mfma_bf16(ak, bk, gkk[p]);
        gqk[p] = mfma_bf16(aq, bk, gqk[p]);
      } else {
        float ak[KPL], aq[KPL], bk[KPL];
#pragma unroll
        for (int j = 0; j < KPL; ++j) {
          const int kk = s * KS + KPL * lg + j;
          ak[j] = tof(Ks[(16 * mi + lr) * EP + kk]);
          aq[j] = tof(Qs[(16 * mi + lr) * EP + kk]);
          bk[j] = tof(Ks[(16 * mj + lr) * EP + kk]);
        }
        MG::run(gkk[p], ak, bk);
        MG::run(gqk[p], aq, bk);
      }
    }
  }
  // 4. norms: |k_i|^2 from the Gram diagonal (diagonal tiles p = 0, 2, 5, 9)
  if (lr >= 4 * lg && lr < 4 * lg + 4) {
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int p = m * (m + 1) / 2 + m;
      const int row = 16 * m + lr;
      const float skk = gkk[p][lr - 4 * lg];
      rk_s[row] = row < L ? (l2 ? 1.0f / sqrtf(skk + kEps) : 1.0f) : 0.0f;
    }
  }
  rq_s[lane] = lane < L ? (l2 ? 1.0f / sqrtf(sqq + kEps) : 1.0f) : 0.0f;
  // 5. chunk-local cumulative decay in fp64
  const bool valid = lane < L;
  const float g_ld = g[(t0 + min(lane, L - 1)) * nv + h];
  const float b_ld = beta[(t0 + min(lane, L - 1)) * nv + h];
  const float gi = valid ? g_ld : 0.0f;
  const float bi = valid ? b_ld : 0.0f;
  double G = gi;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const double y = __shfl_up(G, off, 64);
    if (lane >= off) G += y;
  }
  const double GC = __shfl(G, 63, 64);
  Gs[lane] = G;
  b_s[lane] = bi;
  __syncthreads();   // norms, G, beta visible; K/Q tiles no longer read

  // 6. A (into LDS) and P (kept in registers, in place of the QK^T Gram)
  {
    double Gc[4];
    float rkc[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) { Gc[m] = Gs[16 * m + lr]; rkc[m] = rk_s[16 * m + lr]; }
#pragma unroll
    for (int p = 0; p < 10; ++p) {
      const int mi = tile_mi(p), mj = tile_mj(p);
      const int j = 16 * mj + lr;
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int i = 16 * mi + 4 * lg + ii;
        const double Gi = Gs[i];
        const float dec = (j <= i) ? expf(static_cast<float>(Gi - Gc[mj])) : 0.0f;
        const float rki = rk_s[i];
        Aw[i * AP + j] = (j < i) ? b_s[i] * rki * rkc[mj] * dec * gkk[p][ii] : 0.0f;
        gqk[p][ii] = (j <= i) ? scale * rq_s[i] * rkc[mj] * dec * gqk[p][ii] : 0.0f;
      }
    }
  }
  __syncthreads();

  // 7. T = (I + A)^-1: diagonal 16x16 blocks by forward substitution
  //    (lane = (block lg, column lr)), then the off-diagonal blocks
  //    T_IJ = -T_II * sum_{M=J}^{I-1} A_IM T_MJ on MFMA, one level at a time.
  {
    const int I = lg, jc = lr;
    float t[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float* Ar = Aw + (16 * I + i) * AP + 16 * I;
      float a0 = (i == jc) ? 1.0f : 0.0f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
#pragma unroll
      for (int m = 0; m < i; ++m) {
        const float prod = Ar[m] * t[m];
        if ((m & 3) == 0) a0 -= prod; else if ((m & 3) == 1) a1 -= prod; else if ((m & 3) == 2) a2 -= prod; else a3 -= prod;
      }
      t[i] = (a0 + a1) + (a2 + a3);
      Tw[(16 * I + i) * AP + 16 * I + jc] = t[i];
    }
  }
  __syncthreads();
  constexpr int SP = 20;
#pragma unroll
  for (int lvl = 1; lvl <= 3; ++lvl) {
#pragma unroll
    for (int I = lvl; I <= 3; ++I) {
      const int J = I - lvl;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      for (int Mb = J; Mb < I; ++Mb)
        mm16<BF>(acc, Aw + 16 * I * AP + 16 * Mb, AP, Tw + 16 * Mb * AP + 16 * J, AP, lr, lg);
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) scr[(4 * lg + ii) * SP + lr] = acc[ii];
      __syncthreads();
      f32x4 acc2 = {0.f, 0.f, 0.f, 0.f};
      mm16<BF>(acc2, Tw + 16 * I * AP + 16 * I, AP, scr, SP, lr, lg);
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) Tw[(16 * I + 4 * lg + ii) * AP + 16 * J + lr] = -acc2[ii];
      __syncthreads();
    }
  }

  // 8. P into the upper triangle turned by 180 degrees: X[63-i][63-j] = P[i][j], j <= i
#pragma unroll
  for (int p = 0; p < 10; ++p) {
    const int mi = tile_mi(p), mj = tile_mj(p);
    const int j = 16 * mj + lr;
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      const int i = 16 * mi + 4 * lg + ii;
      if (j <= i) Tw[(63 - i) * AP + (63 - j)] = gqk[p][ii];
    }
  }
  __syncthreads();

  // 9. packed tile and scalars to the workspace
  const size_t tile = static_cast<size_t>(c) * nv + h;
  float* X = tp + tile * CH * CH;
#pragma unroll
  for (int it = 0; it < 16; ++it) {
    const int idx = it * 64 + lane, row = idx >> 4, c4 = (idx & 15) * 4;
    const float4 x = *reinterpret_cast<const float4*>(Tw + row * AP + c4);
    if constexpr (BF) {
      // bf16 inputs: the tile is stored as two bf16 planes, hi = bf16(x) and
      // lo = bf16(x - hi), each 64 x 64, in the same 16 KB
      uint16_t* Xh = reinterpret_cast<uint16_t*>(X);
      uint16_t* Xl = Xh + CH * CH;
      uint2 hi, lo;
      split4_packed(x, hi, lo);
      *reinterpret_cast<uint2*>(Xh + row * CH + c4) = hi;
      *reinterpret_cast<uint2*>(Xl + row * CH + c4) = lo;
    } else {
      *reinterpret_cast<float4*>(X + row * CH + c4) = x;
    }
  }
  const float eG = expf(static_cast<float>(G));
  const float rk_i = rk_s[lane], rq_i = rq_s[lane];
  sc[tile * CH + lane] = make_float4(scale * rq_i * eG, bi * rk_i * eG, rk_i * expf(static_cast<float>(GC - G)), bi);
  if (lane == 0) egc[tile] = expf(static_cast<float>(GC));
}

// ------------------------------------------------------------------ state: bf16 inputs, 8 waves per 16 columns
// One workgroup per (sequence, value head, 16 value columns), eight waves with
// two roles over the chunk's four 16-token tiles m = w % 4:
//   waves 0-3 (recurrence side): X = K S, R = beta v - b X, U = R + T R;
//   waves 4-7 (output side):     Y = Q S, O = a Y + P U.
// Wave w also owns rows 16w..16w+15 of S (128 x 16, fp32, one MFMA
// accumulator) and updates them: S_w = e^{G_C} S_w + K[:, rows]^T (c U).
// Waves w and w+4 share a SIMD, so each SIMD interleaves one wave of each
// side. Every fp32 operand is split into bf16 hi + lo once, by the wave that
// produces it, and exchanged through LDS as transposed bf16 planes, so each
// consumer fragment is one 16-byte LDS read feeding an MFMA directly.
constexpr int KTP = 72;   // LDS pitch (bf16) of K^T   [128 rows of dk][64 tokens]
constexpr int SBP = 136;  // LDS pitch (bf16) of S^T   [16 columns][128 rows of dk]
constexpr int TBP = 72;   // LDS pitch (bf16) of R^T, U^T, (cU)^T [16 columns][64 tokens]

struct Prefetch {
  uint4 f[4];       // K (recurrence side) or Q (output side) A-fragments, 4 k-steps over dk
  uint4 x[4];       // T (recurrence) or P (output) fragments: [hi k0, hi k1, lo k0, lo k1]
  // Raw loaded words only: any arithmetic on a prefetched value at load time
  // would force a wait for that load (and every load issued before it).
  uint32_t vv[4];   // V (bf16 in the low half) of this lane's 4 accumulator rows
  uint4 scv;        // per-token scalars (a, b, c, beta) of token lane, fp32 bits (recurrence side)
  uint32_t eg;      // exp(G_C) bits (every wave)
};
// Every loaded word is consumed on every path of every wave that loads it.
// A register whose load is still counted as pending when the compiler reuses
// it makes it wait on the in-order counter, and with it on every load issued
// since -- including the look-ahead loads of later chunks.

__device__ __forceinline__ bf16x8 as_bf16x8(const uint4& u) { return __builtin_bit_cast(bf16x8, u); }
__device__ __forceinline__ uint4 and4(const uint4& a, const uint4& m) {
  return make_uint4(a.x & m.x, a.y & m.y, a.z & m.z, a.w & m.w);
}
// reverse the order of 8 packed bf16
__device__ __forceinline__ uint4 rev8(const uint4& a) {
  auto sw = [](uint32_t d) { return (d >> 16) | (d << 16); };
  return make_uint4(sw(a.w), sw(a.z), sw(a.y), sw(a.x));
}
__device__ __forceinline__ uint4 lds16(const uint16_t* p) { return *reinterpret_cast<const uint4*>(p); }

template <typename TO>
__global__ void __launch_bounds__(512) chunk_state_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v, int64_t qs,
    int64_t ks, int64_t vs, const int32_t* __restrict__ cu, int n_seqs, int64_t T, int nk, int nv,
    const int32_t* __restrict__ chunk_off, const float* __restrict__ tp, const float4* __restrict__ sc,
    const float* __restrict__ egc, const float* __restrict__ S0, float* __restrict__ ST, TO* __restrict__ o) {
  __shared__ __attribute__((aligned(16))) uint16_t Ktt[2][D * KTP];
  __shared__ __attribute__((aligned(16))) uint16_t Sth[16 * SBP];
  __shared__ __attribute__((aligned(16))) uint16_t Stl[16 * SBP];
  __shared__ __attribute__((aligned(16))) uint16_t RTh[16 * TBP];
  __shared__ __attribute__((aligned(16))) uint16_t RTl[16 * TBP];
  __shared__ __attribute__((aligned(16))) uint16_t UTh[16 * TBP];
  __shared__ __attribute__((aligned(16))) uint16_t UTl[16 * TBP];
  __shared__ __attribute__((aligned(16))) uint16_t CTh[16 * TBP];
  __shared__ __attribute__((aligned(16))) uint16_t CTl[16 * TBP];
  __shared__ float4 SCs[2][CH];

  const int bid = xcd_swizzle(blockIdx.x, gridDim.x);
  const int slice = bid & 7;
  const int unit = bid >> 3;               // n * nv + h
  const int n = unit / nv, h = unit % nv;
  const int hk = h / (nv / nk);
  // the wave index is wave-uniform; say so, so that every wave-level value
  // (role, tile, buffer descriptors) lives in scalar registers
  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool rec = w < 4;                  // recurrence side (wave-uniform)
  const int m = w & 3;                     // token tile of this wave
  const int lr = lane & 15, lg = lane >> 4;
  const int col = slice * 16 + lr;
  const int row = 16 * m + lr;             // this lane's token row as an A-operand row

  // masks of the triangular fragments (constant over chunks): T needs
  // token < row, P needs token <= row (P slot j holds token 32s+8lg+7-j)
  uint4 msk[2];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    uint32_t mm[4];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      if (rec) {
        const int k0 = 32 * s + 8 * lg + 2 * d;
        mm[d] = (k0 < row ? 0x0000ffffu : 0u) | (k0 + 1 < row ? 0xffff0000u : 0u);
      } else {
        const int p0 = 32 * s + 8 * lg + 7 - 2 * d;
        mm[d] = (p0 <= row ? 0x0000ffffu : 0u) | (p0 - 1 <= row ? 0xffff0000u : 0u);
      }
    }
    msk[s] = make_uint4(mm[0], mm[1], mm[2], mm[3]);
  }

  int64_t s_begin, s_end;
  seq_bounds(cu, n, T, s_begin, s_end);
  const int cbase = chunk_off[n];
  const int nchunks = chunk_off[n + 1] - cbase;

  f32x4 S = {0.f, 0.f, 0.f, 0.f};        // rows 16w + 4lg + i, column col
  if (S0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) S[i] = S0[(static_cast<int64_t>(unit) * D + 16 * w + 4 * lg + i) * D + col];
  }

  // lane-constant parts of the operand offsets (bytes)
  const uint32_t fo0 = static_cast<uint32_t>(row * (rec ? ks : qs) * 2 + 16 * lg);
  const uint32_t xo0 = rec ? static_cast<uint32_t>((row * CH + 8 * lg) * 2)
                           : static_cast<uint32_t>(((63 - row) * CH + 56 - 8 * lg) * 2);
  const int xstep = rec ? 64 : -64;        // byte step of one k-step along the fragment row
  const uint32_t vo0 = static_cast<uint32_t>(((16 * m + 4 * lg) * vs + col) * 2);

  auto load_chunk = [&](int cc, Prefetch& pf) {
    const int64_t t0 = s_begin + static_cast<int64_t>(cc) * CH;
    const int L = static_cast<int>(min<int64_t>(CH, s_end - t0));
    const size_t tile = static_cast<size_t>(cbase + cc) * nv + h;
    // Per-chunk buffer resources sized to the chunk's valid rows: rows past
    // the sequence end read as zeros, with no branch around any load.
    const uint16_t* fb = rec ? k : q;
    const int64_t fs = rec ? ks : qs;
    const rsrc_t rf = make_rsrc(fb + t0 * fs + static_cast<int64_t>(hk) * D,
                                static_cast<uint32_t>(((L - 1) * fs + D) * 2));
    const rsrc_t rx = make_rsrc(tp + tile * CH * CH, CH * CH * 4);
#pragma unroll
    for (int s = 0; s < 4; ++s) pf.f[s] = bload16(rf, fo0 + 64 * s);
#pragma unroll
    for (int s = 0; s < 2; ++s) {   // hi plane, then lo plane 8 KB further
      pf.x[s] = bload16(rx, xo0 + xstep * s);
      pf.x[2 + s] = bload16(rx, xo0 + xstep * s + CH * CH * 2);
    }
    if (rec) {
      const rsrc_t rv = make_rsrc(v + t0 * vs + static_cast<int64_t>(h) * D,
                                  static_cast<uint32_t>(((L - 1) * vs + D) * 2));
#pragma unroll
      for (int i = 0; i < 4; ++i) pf.vv[i] = bload2(rv, vo0 + static_cast<uint32_t>(i * vs * 2));
      pf.scv = bload16(make_rsrc(sc + tile * CH, CH * 16), static_cast<uint32_t>(lane * 16));
    }
    // exp(G_C) through a vector load: a uniform (scalar) load would share
    // lgkmcnt with LDS traffic and stall the next LDS wait for a full
    // memory round trip
    pf.eg = __builtin_amdgcn_raw_buffer_load_b32(make_rsrc(egc + tile, 4), static_cast<uint32_t>(lane & 0), 0, 0);
  };
  // stage the next chunk: K^T into LDS from the recurrence waves' K fragments
  auto commit = [&](const Prefetch& pf, int buf) {
    if (rec) {
      uint16_t* Kb = Ktt[buf];
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const uint32_t d[4] = {pf.f[s].x, pf.f[s].y, pf.f[s].z, pf.f[s].w};
#pragma unroll
        for (int j = 0; j < 8; ++j)
          Kb[(32 * s + 8 * lg + j) * KTP + row] =
              static_cast<uint16_t>((j & 1) ? (d[j >> 1] >> 16) : (d[j >> 1] & 0xffffu));
      }
      // (all four recurrence waves write the same values: see Prefetch)
      *reinterpret_cast<uint4*>(&SCs[buf][lane]) = pf.scv;
    }
  };
  auto publish_S = [&]() {
    uint2 hi, lo;
    split4_packed(make_float4(S[0], S[1], S[2], S[3]), hi, lo);
    *reinterpret_cast<uint2*>(&Sth[lr * SBP + 16 * w + 4 * lg]) = hi;
    *reinterpret_cast<uint2*>(&Stl[lr * SBP + 16 * w + 4 * lg]) = lo;
  };

  // The output tile of chunk c is stored at the start of chunk c+1, after that
  // chunk's prefetch loads are issued: loads and stores share one in-order
  // completion counter, so a store issued before a load would make every
  // wait on that load also wait for the store to reach memory.
  f32x4 Opend = {0.f, 0.f, 0.f, 0.f};
  int cc_pend = -1;
  const uint32_t oo0 = static_cast<uint32_t>(((16 * m + 4 * lg) * nv * D + col) * sizeof(TO));
  auto store_pending = [&]() {
    const int64_t t0 = s_begin + static_cast<int64_t>(cc_pend) * CH;
    const int L = static_cast<int>(min<int64_t>(CH, s_end - t0));
    const rsrc_t ro = make_rsrc(o + (t0 * nv + h) * static_cast<int64_t>(D),
                                static_cast<uint32_t>(((L - 1) * nv * D + D) * sizeof(TO)));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t off = oo0 + static_cast<uint32_t>(i * nv * D * sizeof(TO));
      if constexpr (sizeof(TO) == 4) bstore4(ro, off, Opend[i]);
      else bstore2(ro, off, f32_to_bf16(Opend[i]));
    }
  };

  // One chunk: issue the loads of chunk cc+2 into `nxt2`, compute chunk cc
  // with `cur`, then stage chunk cc+1 (`nxt`, loaded one chunk ago) in LDS.
  // Three register buffers rotate, so no copy is made between chunks and
  // every load has two chunks of compute to arrive.
  auto step = [&](int cc, const Prefetch& cur, const Prefetch& nxt, Prefetch& nxt2) {
    const int buf = cc & 1;
    // (past the end the last chunk is re-read: unconditional, so loads stay in registers)
    load_chunk(min(cc + 2, nchunks - 1), nxt2);
    if (!rec && cc_pend >= 0) store_pending();

    // X = K S (recurrence side) or Y = Q S (output side) for this wave's tile
    f32x4 XY = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const bf16x8 bh = as_bf16x8(lds16(&Sth[lr * SBP + 32 * s + 8 * lg]));
      const bf16x8 bl = as_bf16x8(lds16(&Stl[lr * SBP + 32 * s + 8 * lg]));
      const bf16x8 a = as_bf16x8(cur.f[s]);
      XY = mfma_bf16(a, bl, XY);
      XY = mfma_bf16(a, bh, XY);
    }
    f32x4 Ra = {0.f, 0.f, 0.f, 0.f};
    if (rec) {   // R = beta v - b X -> R^T planes
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float4 s4 = SCs[buf][16 * m + 4 * lg + i];
        Ra[i] = s4.w * bf16_to_f32(static_cast<uint16_t>(cur.vv[i])) - s4.y * XY[i];
      }
      uint2 hi, lo;
      split4_packed(make_float4(Ra[0], Ra[1], Ra[2], Ra[3]), hi, lo);
      *reinterpret_cast<uint2*>(&RTh[lr * TBP + 16 * m + 4 * lg]) = hi;
      *reinterpret_cast<uint2*>(&RTl[lr * TBP + 16 * m + 4 * lg]) = lo;
    }
    __syncthreads();

    if (rec) {   // U = R + T_strict R -> U^T and (c U)^T planes
      f32x4 Ua = Ra;
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const bf16x8 ah = as_bf16x8(and4(cur.x[s], msk[s]));
        const bf16x8 al = as_bf16x8(and4(cur.x[2 + s], msk[s]));
        const bf16x8 bh = as_bf16x8(lds16(&RTh[lr * TBP + 32 * s + 8 * lg]));
        const bf16x8 bl = as_bf16x8(lds16(&RTl[lr * TBP + 32 * s + 8 * lg]));
        Ua = mfma_bf16(al, bh, Ua);
        Ua = mfma_bf16(ah, bl, Ua);
        Ua = mfma_bf16(ah, bh, Ua);
      }
      uint2 hi, lo;
      split4_packed(make_float4(Ua[0], Ua[1], Ua[2], Ua[3]), hi, lo);
      *reinterpret_cast<uint2*>(&UTh[lr * TBP + 16 * m + 4 * lg]) = hi;
      *reinterpret_cast<uint2*>(&UTl[lr * TBP + 16 * m + 4 * lg]) = lo;
      float cu4[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) cu4[i] = SCs[buf][16 * m + 4 * lg + i].z * Ua[i];
      split4_packed(make_float4(cu4[0], cu4[1], cu4[2], cu4[3]), hi, lo);
      *reinterpret_cast<uint2*>(&CTh[lr * TBP + 16 * m + 4 * lg]) = hi;
      *reinterpret_cast<uint2*>(&CTl[lr * TBP + 16 * m + 4 * lg]) = lo;
    }
    __syncthreads();

    if (!rec) {  // O = a Y + P U (P fragments hold tokens in reversed order: reverse U too)
      f32x4 Oa;
#pragma unroll
      for (int i = 0; i < 4; ++i) Oa[i] = SCs[buf][16 * m + 4 * lg + i].x * XY[i];
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const bf16x8 ah = as_bf16x8(and4(cur.x[s], msk[s]));
        const bf16x8 al = as_bf16x8(and4(cur.x[2 + s], msk[s]));
        const bf16x8 bh = as_bf16x8(rev8(lds16(&UTh[lr * TBP + 32 * s + 8 * lg])));
        const bf16x8 bl = as_bf16x8(rev8(lds16(&UTl[lr * TBP + 32 * s + 8 * lg])));
        Oa = mfma_bf16(al, bh, Oa);
        Oa = mfma_bf16(ah, bl, Oa);
        Oa = mfma_bf16(ah, bh, Oa);
      }
      Opend = Oa;          // stored at the start of the next chunk
      cc_pend = cc;
    }

    // S_w = e^{G_C} S_w + K[:, rows of w]^T (c U)
    {
      const float eGC = __builtin_bit_cast(float, cur.eg);
#pragma unroll
      for (int i = 0; i < 4; ++i) S[i] *= eGC;
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const bf16x8 a = as_bf16x8(lds16(&Ktt[buf][(16 * w + lr) * KTP + 32 * s + 8 * lg]));
        const bf16x8 ch = as_bf16x8(lds16(&CTh[lr * TBP + 32 * s + 8 * lg]));
        const bf16x8 cl = as_bf16x8(lds16(&CTl[lr * TBP + 32 * s + 8 * lg]));
        S = mfma_bf16(a, cl, S);
        S = mfma_bf16(a, ch, S);
      }
    }
    // publish S for the next chunk (every wave has read S^T before the barriers above)
    publish_S();
    commit(nxt, buf ^ 1);
    __syncthreads();
  };

  Prefetch pa, pb, pc;
  if (nchunks > 0) {
    load_chunk(0, pa);
    load_chunk(min(1, nchunks - 1), pb);
    commit(pa, 0);
  }
  publish_S();
  __syncthreads();
  // Whole rotations in the loop, the last one or two chunks after it: a loop
  // body without early exits lets the compiler count exactly which loads are
  // still in flight at every wait.
  int cc = 0;
  for (; cc + 3 <= nchunks; cc += 3) {
    step(cc, pa, pb, pc);
    step(cc + 1, pb, pc, pa);
    step(cc + 2, pc, pa, pb);
  }
  if (cc < nchunks) step(cc, pa, pb, pc);
  if (cc + 1 < nchunks) step(cc + 1, pb, pc, pa);
  if (!rec && cc_pend >= 0) store_pending();

  if (ST) {
#pragma unroll
    for (int i = 0; i < 4; ++i) ST[(static_cast<int64_t>(unit) * D + 16 * w + 4 * lg + i) * D + col] = S[i];
  }
}

// ------------------------------------------------------------------ state: generic (fp32 inputs), one wave per 16 columns
constexpr int KP = 132;    // LDS pitch (floats) of 64 x 128 K/Q tiles
constexpr int RP = 18;     // LDS pitch of the 64 x 16 R / U tiles

template <typename TIn>
__device__ __forceinline__ void load_tile_64x128(const TIn* __restrict__ base, int64_t tok_stride, int L,
                                                 float* __restrict__ dst, int tid, int nthreads) {
  for (int idx = tid; idx < CH * (D / 8); idx += nthreads) {
    const int row = idx >> 4, seg = idx & 15;
    float* d = dst + row * KP + seg * 8;
    if (row < L) {
      float vals[8];
      load8(base + row * tok_stride + seg * 8, vals);
      *reinterpret_cast<float4*>(d) = make_float4(vals[0], vals[1], vals[2], vals[3]);
      *reinterpret_cast<float4*>(d + 4) = make_float4(vals[4], vals[5], vals[6], vals[7]);
    } else {
      *reinterpret_cast<float4*>(d) = make_float4(0.f, 0.f, 0.f, 0.f);
      *reinterpret_cast<float4*>(d + 4) = make_float4(0.f, 0.f, 0.f, 0.f);
    }
  }
}

template <typename TIn, typename TO>
__global__ void __launch_bounds__(64) chunk_state_generic_kernel(
    const TIn* __restrict__ q, const TIn* __restrict__ k, const TIn* __restrict__ v, int64_t qs,
    int64_t ks, int64_t vs, const int32_t* __restrict__ cu, int n_seqs, int64_t T, int nk, int nv,
    const int32_t* __restrict__ chunk_off, const float* __restrict__ tp, const float4* __restrict__ sc,
    const float* __restrict__ egc, const float* __restrict__ S0, float* __restrict__ ST,
    TO* __restrict__ o) {
  constexpr bool BF = sizeof(TIn) == 2;
  constexpr int KS = Mma<BF, true, true>::KS, KPL = Mma<BF, true, true>::KPL;

  extern __shared__ __attribute__((aligned(16))) float smem_f[];
  float* Ks = smem_f;                  // [64][KP]
  float* Qs = Ks + CH * KP;            // [64][KP]
  float* Ts = Qs + CH * KP;            // [64][AP]  packed T | rotated P
  float* Vs = Ts + CH * AP;            // [64][16]
  float4* SCs = reinterpret_cast<float4*>(Vs + CH * 16);   // [64]
  float* Rw = reinterpret_cast<float*>(SCs + CH);           // [64][RP]

  const int bid = xcd_swizzle(blockIdx.x, gridDim.x);
  const int nb = bid & 7;
  const int unit = bid >> 3;
  const int n = unit / nv, h = unit % nv;
  const int hk = h / (nv / nk);
  const int lane = threadIdx.x;
  const int lr = lane & 15, lg = lane >> 4;
  const int col = nb * 16 + lr;

  int64_t s_begin, s_end;
  seq_bounds(cu, n, T, s_begin, s_end);
  const int nchunks = chunk_off[n + 1] - chunk_off[n];

  f32x4 S[8];
#pragma unroll
  for (int t = 0; t < 8; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      S[t][i] = S0 ? S0[(static_cast<int64_t>(unit) * D + 16 * t + 4 * lg + i) * D + col] : 0.0f;

  for (int cc = 0; cc < nchunks; ++cc) {
    const int64_t t0 = s_begin + static_cast<int64_t>(cc) * CH;
    const int L = static_cast<int>(min<int64_t>(CH, s_end - t0));
    const size_t tile = static_cast<size_t>(chunk_off[n] + cc) * nv + h;
    __syncthreads();
    load_tile_64x128(k + t0 * ks + static_cast<int64_t>(hk) * D, ks, L, Ks, lane, 64);
    load_tile_64x128(q + t0 * qs + static_cast<int64_t>(hk) * D, qs, L, Qs, lane, 64);
    for (int idx = lane; idx < CH * CH / 4; idx += 64) {
      const int r = idx >> 4, c4 = (idx & 15) * 4;
      *reinterpret_cast<float4*>(Ts + r * AP + c4) = *reinterpret_cast<const float4*>(tp + tile * CH * CH + r * CH + c4);
    }
    for (int idx = lane; idx < CH * 16; idx += 64) {
      const int r = idx >> 4, cidx = idx & 15;
      Vs[idx] = r < L ? Elem<TIn>::load(v, (t0 + r) * vs + static_cast<int64_t>(h) * D + nb * 16 + cidx) : 0.0f;
    }
    SCs[lane] = sc[tile * CH + lane];
    const float eGC = egc[tile];
    __syncthreads();

    f32x4 Xa[4], Ya[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      Xa[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
      Ya[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < D / KS; ++s) {
        float ak[KPL], aq[KPL], bs[KPL];
#pragma unroll
        for (int j = 0; j < KPL; ++j) {
          const int f = s * KPL + j;
          const int dk = 16 * (f >> 2) + 4 * lg + (f & 3);
          ak[j] = Ks[(16 * mt + lr) * KP + dk];
          aq[j] = Qs[(16 * mt + lr) * KP + dk];
          bs[j] = S[f >> 2][f & 3];
        }
        Mma<BF, true, false>::run(Xa[mt], ak, bs);
        Mma<BF, true, false>::run(Ya[mt], aq, bs);
      }
    }
    f32x4 Ra[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tau = 16 * mt + 4 * lg + i;
        const float4 s4 = SCs[tau];
        Ra[mt][i] = s4.w * Vs[tau * 16 + lr] - s4.y * Xa[mt][i];
        Rw[tau * RP + lr] = Ra[mt][i];
      }
    __syncthreads();
    f32x4 Ua[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      Ua[mt] = Ra[mt];
      const int row = 16 * mt + lr;
#pragma unroll
      for (int s = 0; s <= (16 * mt + 15) / KS; ++s) {
        float a[KPL], b[KPL];
#pragma unroll
        for (int j = 0; j < KPL; ++j) {
          const int kk = s * KS + KPL * lg + j;
          a[j] = kk < row ? Ts[row * AP + kk] : 0.0f;
          b[j] = Rw[kk * RP + lr];
        }
        Mma<BF, false, false>::run(Ua[mt], a, b);
      }
    }
    __syncthreads();
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) Rw[(16 * mt + 4 * lg + i) * RP + lr] = Ua[mt][i];
    __syncthreads();
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      f32x4 Oa;
#pragma unroll
      for (int i = 0; i < 4; ++i) Oa[i] = SCs[16 * mt + 4 * lg + i].x * Ya[mt][i];
      const int row = 16 * mt + lr;
#pragma unroll
      for (int s = 0; s <= (16 * mt + 15) / KS; ++s) {
        float a[KPL], b[KPL];
#pragma unroll
        for (int j = 0; j < KPL; ++j) {
          const int kk = s * KS + KPL * lg + j;
          a[j] = kk <= row ? Ts[(63 - row) * AP + (63 - kk)] : 0.0f;
          b[j] = Rw[kk * RP + lr];
        }
        Mma<BF, false, false>::run(Oa, a, b);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tau = 16 * mt + 4 * lg + i;
        if (tau < L) Elem<TO>::store(o, ((t0 + tau) * nv + h) * static_cast<int64_t>(D) + col, Oa[i]);
      }
    }
#pragma unroll
    for (int t = 0; t < 8; ++t) {
#pragma unroll
      for (int i = 0; i < 4; ++i) S[t][i] *= eGC;
#pragma unroll
      for (int s = 0; s < CH / KS; ++s) {
        float a[KPL], b[KPL];
#pragma unroll
        for (int j = 0; j < KPL; ++j) {
          const int kk = s * KS + KPL * lg + j;
          a[j] = Ks[kk * KP + 16 * t + lr];
          b[j] = SCs[kk].z * Rw[kk * RP + lr];
        }
        Mma<BF, true, false>::run(S[t], a, b);
      }
    }
  }
  if (ST) {
#pragma unroll
    for (int t = 0; t < 8; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        ST[(static_cast<int64_t>(unit) * D + 16 * t + 4 * lg + i) * D + col] = S[t][i];
  }
}

constexpr size_t generic_lds_bytes() {
  return (2 * CH * KP + CH * AP + CH * 16) * sizeof(float) + CH * sizeof(float4) + CH * RP * sizeof(float);
}

template <typename TIn>
hipError_t chunk_dispatch(const void* q, const void* k, const void* v, int64_t qs, int64_t ks, int64_t vs,
                          const float* g, const float* beta, const int32_t* cu, int n_seqs, int64_t T, int nk,
                          int nv, float scale, int l2, const float* S0, float* ST, void* o, int o_bf16, void* ws,
                          hipStream_t s) {
  const WsLayout lay = ws_layout(T, n_seqs, nv);
  char* base = static_cast<char*>(ws);
  int32_t* chunk_off = reinterpret_cast<int32_t*>(base + lay.off_chunk_off);
  float* tp = reinterpret_cast<float*>(base + lay.off_tp);
  float4* sc = reinterpret_cast<float4*>(base + lay.off_sc);
  float* egc = reinterpret_cast<float*>(base + lay.off_egc);

  const int64_t nch = T / CH + n_seqs;
  chunk_offsets_kernel<<<1, 256, 0, s>>>(cu, n_seqs, T, static_cast<int32_t>(nch), chunk_off);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  {
    auto kern = chunk_prep_kernel<TIn>;
    const size_t lds = prep_lds_bytes<TIn>();
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                            static_cast<int>(lds));
    if (e != hipSuccess) return e;
    kern<<<dim3(static_cast<unsigned>(nch), static_cast<unsigned>(nv)), 64, lds, s>>>(
        static_cast<const TIn*>(q), static_cast<const TIn*>(k), qs, ks, g, beta, cu, n_seqs, T, nk, nv, scale, l2,
        chunk_off, tp, sc, egc);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const unsigned grid = static_cast<unsigned>(n_seqs) * nv * (D / 16);
  if constexpr (sizeof(TIn) == 2) {
    if (o_bf16)
      chunk_state_bf16_kernel<uint16_t><<<grid, 512, 0, s>>>(
          static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v), qs, ks,
          vs, cu, n_seqs, T, nk, nv, chunk_off, tp, sc, egc, S0, ST, static_cast<uint16_t*>(o));
    else
      chunk_state_bf16_kernel<float><<<grid, 512, 0, s>>>(
          static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v), qs, ks,
          vs, cu, n_seqs, T, nk, nv, chunk_off, tp, sc, egc, S0, ST, static_cast<float*>(o));
    return hipGetLastError();
  } else {
    const size_t lds = generic_lds_bytes();
    auto launch = [&](auto kern, auto* optr) {
      hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
      if (err != hipSuccess) return err;
      kern<<<grid, 64, lds, s>>>(static_cast<const TIn*>(q), static_cast<const TIn*>(k), static_cast<const TIn*>(v),
                                 qs, ks, vs, cu, n_seqs, T, nk, nv, chunk_off, tp, sc, egc, S0, ST, optr);
      return hipGetLastError();
    };
    if (o_bf16) return launch(chunk_state_generic_kernel<TIn, uint16_t>, static_cast<uint16_t*>(o));
    return launch(chunk_state_generic_kernel<TIn, float>, static_cast<float*>(o));
  }
}

}  // namespace

size_t chunk_workspace_bytes(int64_t T, int n_seqs, int nv) { return ws_layout(T, n_seqs, nv).total; }

hipError_t launch_chunk_fwd(const void* q, const void* k, const void* v, int bf16, int64_t qs, int64_t ks,
                            int64_t vs, const float* g, const float* beta, const int32_t* cu, int n_seqs,
                            int64_t T, int nk, int nv, float scale, int l2, const float* S0, float* ST, void* o,
                            int o_bf16, void* ws, hipStream_t s) {
  if (bf16)
    return chunk_dispatch<uint16_t>(q, k, v, qs, ks, vs, g, beta, cu, n_seqs, T, nk, nv, scale, l2, S0, ST, o,
                                    o_bf16, ws, s);
  return chunk_dispatch<float>(q, k, v, qs, ks, vs, g, beta, cu, n_seqs, T, nk, nv, scale, l2, S0, ST, o, o_bf16,
                               ws, s);
}

}  // namespace gdn
