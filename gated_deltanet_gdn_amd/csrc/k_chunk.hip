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
//   chunk_prep    : one workgroup per (chunk, key head), fully parallel. Grams
//                   K K^T and Q K^T on MFMA from the raw inputs (exact
//                   operands), then per value head: fp64 cumsum of g, A, the
//                   forward substitution for T, P, and the per-token scalars.
//                   Writes a packed 64x64 fp32 tile per (chunk, value head):
//                   T strictly below the diagonal, P^T on and above it.
//   chunk_state   : one wave per (sequence, value head, 16 value columns),
//                   sequential over the sequence's chunks, S (128 x 16) held
//                   in MFMA accumulator registers for the whole sequence.
//                   Products with an fp32 operand split it into bf16 hi + lo.
#include "gdn_device.hpp"
#include "gdn_internal.hpp"

namespace gdn {
namespace {

constexpr int CH = 64;     // chunk length
constexpr int D = 128;     // dk = dv
constexpr int KP = 136;    // LDS row pitch (floats) of 64 x 128 K/Q tiles
constexpr int GP = 65;     // LDS pitch of 64 x 64 Gram tiles
constexpr int AP = 68;     // LDS pitch of 64 x 64 A / T|P tiles (16-byte rows)
constexpr int RP = 18;     // LDS pitch of the per-wave 64 x 16 R / U tiles
constexpr float kEps = 1e-6f;

__device__ __forceinline__ size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

struct WsLayout {
  size_t off_chunk_off, off_tp, off_sc, off_egc, total;
};
__host__ __device__ inline WsLayout ws_layout(int64_t T, int n_seqs, int nv) {
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

template <typename TIn>
__device__ __forceinline__ void load_row8(const TIn* p, float* dst) {
  float v[8];
  load8(p, v);
  *reinterpret_cast<float4*>(dst) = make_float4(v[0], v[1], v[2], v[3]);
  *reinterpret_cast<float4*>(dst + 4) = make_float4(v[4], v[5], v[6], v[7]);
}

// Cooperative load of a 64 x 128 tile (rows >= L zero) into LDS with pitch KP.
template <typename TIn>
__device__ __forceinline__ void load_tile_64x128(const TIn* __restrict__ base, int64_t tok_stride, int L,
                                                 float* __restrict__ dst, int tid, int nthreads) {
  for (int idx = tid; idx < CH * (D / 8); idx += nthreads) {
    const int row = idx >> 4, seg = idx & 15;
    float* d = dst + row * KP + seg * 8;
    if (row < L) {
      load_row8(base + row * tok_stride + seg * 8, d);
    } else {
      *reinterpret_cast<float4*>(d) = make_float4(0.f, 0.f, 0.f, 0.f);
      *reinterpret_cast<float4*>(d + 4) = make_float4(0.f, 0.f, 0.f, 0.f);
    }
  }
}

// ------------------------------------------------------------------ prep
template <typename TIn>
__global__ void __launch_bounds__(256) chunk_prep_kernel(
    const TIn* __restrict__ q, const TIn* __restrict__ k, int64_t qs, int64_t ks,
    const float* __restrict__ g, const float* __restrict__ beta, const int32_t* __restrict__ cu,
    int n_seqs, int64_t T, int nk, int nv, float scale, int l2, const int32_t* __restrict__ chunk_off,
    float* __restrict__ tp, float4* __restrict__ sc, float* __restrict__ egc) {
  constexpr bool BF = sizeof(TIn) == 2;
  using M = Mma<BF, true, true>;
  constexpr int KS = M::KS, KPL = M::KPL;

  extern __shared__ float smem[];
  float* Ks = smem;                       // [64][KP]
  float* Qs = Ks + CH * KP;               // [64][KP]
  float* Gkk = Qs + CH * KP;              // [64][GP]
  float* Gqk = Gkk + CH * GP;             // [64][GP]
  float* rk_s = Gqk + CH * GP;            // [64]
  float* rq_s = rk_s + CH;                // [64]
  float* Aw_all = Ks;                     // after the Grams: 4 x [64][AP] (aliases Ks/Qs)

  const int c = blockIdx.x;
  const int hk = blockIdx.y;
  const int total = chunk_off[n_seqs];
  if (c >= total) return;
  const int n = find_le(chunk_off, n_seqs, c);
  int64_t s_begin, s_end;
  seq_bounds(cu, n, T, s_begin, s_end);
  const int64_t t0 = s_begin + static_cast<int64_t>(c - chunk_off[n]) * CH;
  const int L = static_cast<int>(min<int64_t>(CH, s_end - t0));
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = nv / nk;

  load_tile_64x128(k + t0 * ks + static_cast<int64_t>(hk) * D, ks, L, Ks, tid, 256);
  load_tile_64x128(q + t0 * qs + static_cast<int64_t>(hk) * D, qs, L, Qs, tid, 256);
  __syncthreads();

  {  // row norms: 4 lanes per row, 32 elements each
    const int row = tid >> 2, part = tid & 3;
    float sk = 0.f, sq = 0.f;
#pragma unroll 8
    for (int e = 0; e < 32; ++e) {
      const float kv = Ks[row * KP + part * 32 + e];
      const float qv = Qs[row * KP + part * 32 + e];
      sk = fmaf(kv, kv, sk);
      sq = fmaf(qv, qv, sq);
    }
    sk += __shfl_xor(sk, 1, 64); sk += __shfl_xor(sk, 2, 64);
    sq += __shfl_xor(sq, 1, 64); sq += __shfl_xor(sq, 2, 64);
    if (part == 0) {
      const bool valid = row < L;
      rk_s[row] = valid ? (l2 ? 1.0f / sqrtf(sk + kEps) : 1.0f) : 0.0f;
      rq_s[row] = valid ? (l2 ? 1.0f / sqrtf(sq + kEps) : 1.0f) : 0.0f;
    }
  }

  // Grams on the lower 16x16 tiles: 10 of K K^T and 10 of Q K^T, 5 per wave.
  {
    const int lr = lane & 15, lg = lane >> 4;
    for (int p = wave; p < 20; p += 4) {
      const int pp = p % 10;
      const int mi = pp >= 6 ? 3 : pp >= 3 ? 2 : pp >= 1 ? 1 : 0;
      const int mj = pp - mi * (mi + 1) / 2;
      const float* X = p < 10 ? Ks : Qs;
      float* G = p < 10 ? Gkk : Gqk;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < D / KS; ++s) {
        float a[KPL], b[KPL];
#pragma unroll
        for (int j = 0; j < KPL; ++j) {
          const int kk = s * KS + KPL * lg + j;
          a[j] = X[(16 * mi + lr) * KP + kk];
          b[j] = Ks[(16 * mj + lr) * KP + kk];
        }
        M::run(acc, a, b);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) G[(16 * mi + 4 * lg + i) * GP + 16 * mj + lr] = acc[i];
    }
  }
  __syncthreads();

  // Per value head: one wave each.
  for (int jj = wave; jj < r; jj += 4) {
    const int h = hk * r + jj;
    float* Aw = Aw_all + wave * CH * AP;
    const size_t tile = static_cast<size_t>(c) * nv + h;
    float* X = tp + tile * CH * CH;

    const bool valid = lane < L;
    const float gi = valid ? g[(t0 + lane) * nv + h] : 0.0f;
    const float bi = valid ? beta[(t0 + lane) * nv + h] : 0.0f;
    double G = gi;                      // chunk-local cumulative decay, fp64
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const double y = __shfl_up(G, off, 64);
      if (lane >= off) G += y;
    }
    const double GC = __shfl(G, 63, 64);
    const float rk_i = rk_s[lane], rq_i = rq_s[lane];

    // A, column-oriented (lane = column j); row i broadcast via shuffles
    for (int i = 0; i < CH; ++i) {
      const double Gi = __shfl(G, i, 64);
      const float bi_ = __shfl(bi, i, 64);
      float a = 0.0f;
      if (lane < i) a = bi_ * rk_s[i] * rk_i * expf(static_cast<float>(Gi - G)) * Gkk[i * GP + lane];
      Aw[i * AP + lane] = a;
    }
    // (wave-private LDS: the writes above precede the reads below in program order)
    __builtin_amdgcn_s_waitcnt(0xc07f);
    __builtin_amdgcn_wave_barrier();

    // forward substitution: T[i][j] = delta_ij - sum_{m<i} A[i][m] T[m][j]; lane = j
    float tcol[CH];
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      float acc = (lane == i) ? 1.0f : 0.0f;
      const float* Ar = Aw + i * AP;
#pragma unroll
      for (int m = 0; m < i; ++m) acc = fmaf(-Ar[m], tcol[m], acc);
      tcol[i] = acc;
      if (lane < i) X[i * CH + lane] = acc;     // strictly lower part of T
    }

    // P (row-oriented, lane = i), stored transposed: X[j][i] = P[i][j], j <= i
    for (int j = 0; j < CH; ++j) {
      const double Gj = __shfl(G, j, 64);
      if (j <= lane) {
        const float pij = scale * rq_i * rk_s[j] * expf(static_cast<float>(G - Gj)) * Gqk[lane * GP + j];
        X[j * CH + lane] = pij;
      }
    }
    // per-token scalars: a = scale rq e^G, b = beta rk e^G, c = rk e^{G_C - G}, beta
    const float eG = expf(static_cast<float>(G));
    sc[tile * CH + lane] = make_float4(scale * rq_i * eG, bi * rk_i * eG,
                                       rk_i * expf(static_cast<float>(GC - G)), bi);
    if (lane == 0) egc[tile] = expf(static_cast<float>(GC));
  }
}

// ------------------------------------------------------------------ state recurrence
template <typename TIn, typename TO, int W>
__global__ void __launch_bounds__(64 * W) chunk_state_kernel(
    const TIn* __restrict__ q, const TIn* __restrict__ k, const TIn* __restrict__ v, int64_t qs,
    int64_t ks, int64_t vs, const int32_t* __restrict__ cu, int n_seqs, int64_t T, int nk, int nv,
    const int32_t* __restrict__ chunk_off, const float* __restrict__ tp, const float4* __restrict__ sc,
    const float* __restrict__ egc, const float* __restrict__ S0, float* __restrict__ ST,
    TO* __restrict__ o) {
  constexpr bool BF = sizeof(TIn) == 2;
  constexpr int KS = Mma<BF, true, true>::KS, KPL = Mma<BF, true, true>::KPL;
  constexpr int NT = 64 * W;
  constexpr int VW = 16 * W;           // value columns per workgroup
  constexpr int VP = VW + 4;           // LDS pitch of the V tile

  extern __shared__ float smem[];
  float* Ks = smem;                    // [64][KP]
  float* Qs = Ks + CH * KP;            // [64][KP]
  float* Ts = Qs + CH * KP;            // [64][AP]  packed T | P^T
  float* Vs = Ts + CH * AP;            // [64][VP]
  float4* SCs = reinterpret_cast<float4*>(Vs + CH * VP);   // [64]
  float* Rall = reinterpret_cast<float*>(SCs + CH);        // W x [64][RP]

  const int nblk = D / VW;
  const int bid = xcd_swizzle(blockIdx.x, gridDim.x);
  const int nb = bid % nblk;
  const int unit = bid / nblk;         // n * nv + h
  const int n = unit / nv, h = unit % nv;
  const int hk = h / (nv / nk);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  const int col = nb * VW + wave * 16 + lr;   // this lane's value column
  float* Rw = Rall + wave * CH * RP;

  int64_t s_begin, s_end;
  seq_bounds(cu, n, T, s_begin, s_end);
  const int nchunks = chunk_off[n + 1] - chunk_off[n];

  // S in accumulator layout: tile t covers dk rows 16t..16t+15; lane holds
  // rows 16t + 4*lg + i, column `col`.
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

    __syncthreads();   // previous chunk's LDS reads are complete
    load_tile_64x128(k + t0 * ks + static_cast<int64_t>(hk) * D, ks, L, Ks, tid, NT);
    load_tile_64x128(q + t0 * qs + static_cast<int64_t>(hk) * D, qs, L, Qs, tid, NT);
    for (int idx = tid; idx < CH * CH / 4; idx += NT) {
      const int row = idx >> 4, c4 = (idx & 15) * 4;
      *reinterpret_cast<float4*>(Ts + row * AP + c4) =
          *reinterpret_cast<const float4*>(tp + tile * CH * CH + row * CH + c4);
    }
    for (int idx = tid; idx < CH * (VW / 8); idx += NT) {
      const int row = idx / (VW / 8), seg = idx % (VW / 8);
      float* d = Vs + row * VP + seg * 8;
      if (row < L) {
        load_row8(v + (t0 + row) * vs + static_cast<int64_t>(h) * D + nb * VW + seg * 8, d);
      } else {
        *reinterpret_cast<float4*>(d) = make_float4(0.f, 0.f, 0.f, 0.f);
        *reinterpret_cast<float4*>(d + 4) = make_float4(0.f, 0.f, 0.f, 0.f);
      }
    }
    for (int idx = tid; idx < CH; idx += NT) SCs[idx] = sc[tile * CH + idx];
    const float eGC = egc[tile];
    __syncthreads();

    // X = K S, Y = Q S (64 x 16 per wave); S is the B operand with the
    // contraction index ordered as the accumulator holds it.
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

    // R = beta v - b X  (accumulator layout), to this wave's LDS tile
    f32x4 Ra[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tau = 16 * mt + 4 * lg + i;
        const float4 s4 = SCs[tau];
        const float rv = s4.w * Vs[tau * VP + wave * 16 + lr] - s4.y * Xa[mt][i];
        Ra[mt][i] = rv;
        Rw[tau * RP + lr] = rv;
      }
    __syncthreads();

    // U = R + T_strict R
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

    // O = a Y + P U  (P[i][j] stored at Ts[j][i])
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
          a[j] = kk <= row ? Ts[kk * AP + row] : 0.0f;
          b[j] = Rw[kk * RP + lr];
        }
        Mma<BF, false, false>::run(Oa, a, b);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tau = 16 * mt + 4 * lg + i;
        if (tau < L)
          Elem<TO>::store(o, ((t0 + tau) * nv + h) * static_cast<int64_t>(D) + col, Oa[i]);
      }
    }

    // S = e^{G_C} S + K^T (c U)
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
      for (int i = 0; i < 4; ++i) ST[(static_cast<int64_t>(unit) * D + 16 * t + 4 * lg + i) * D + col] = S[t][i];
  }
}

constexpr size_t prep_lds_bytes() {
  return (2 * CH * KP + 2 * CH * GP + 2 * CH) * sizeof(float);
}
template <int W>
constexpr size_t state_lds_bytes() {
  return (2 * CH * KP + CH * AP + CH * (16 * W + 4)) * sizeof(float) + CH * sizeof(float4) +
         W * CH * RP * sizeof(float);
}
static_assert(4 * CH * AP <= 2 * CH * KP, "A tiles must fit in the K/Q region");

template <typename TIn, typename TO, int W>
hipError_t launch_state(const void* q, const void* k, const void* v, int64_t qs, int64_t ks, int64_t vs,
                        const int32_t* cu, int n_seqs, int64_t T, int nk, int nv, const int32_t* chunk_off,
                        const float* tp, const float4* sc, const float* egc, const float* S0, float* ST,
                        void* o, hipStream_t s) {
  auto kern = chunk_state_kernel<TIn, TO, W>;
  const size_t lds = state_lds_bytes<W>();
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
  if (e != hipSuccess) return e;
  const unsigned grid = static_cast<unsigned>(n_seqs) * nv * (D / (16 * W));
  kern<<<grid, 64 * W, lds, s>>>(static_cast<const TIn*>(q), static_cast<const TIn*>(k),
                                 static_cast<const TIn*>(v), qs, ks, vs, cu, n_seqs, T, nk, nv, chunk_off, tp, sc,
                                 egc, S0, ST, static_cast<TO*>(o));
  return hipGetLastError();
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
    const size_t lds = prep_lds_bytes();
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                            static_cast<int>(lds));
    if (e != hipSuccess) return e;
    kern<<<dim3(static_cast<unsigned>(nch), static_cast<unsigned>(nk)), 256, lds, s>>>(
        static_cast<const TIn*>(q), static_cast<const TIn*>(k), qs, ks, g, beta, cu, n_seqs, T, nk, nv, scale, l2,
        chunk_off, tp, sc, egc);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  // 16 value columns per wave; 4 waves per workgroup when there are enough
  // (sequence, head) units to fill the GPU, else 1 so more CUs share the work.
  const int64_t units = static_cast<int64_t>(n_seqs) * nv;
  const bool wide = units * 2 >= 256;
  if (o_bf16)
    return wide ? launch_state<TIn, uint16_t, 4>(q, k, v, qs, ks, vs, cu, n_seqs, T, nk, nv, chunk_off, tp, sc,
                                                 egc, S0, ST, o, s)
                : launch_state<TIn, uint16_t, 1>(q, k, v, qs, ks, vs, cu, n_seqs, T, nk, nv, chunk_off, tp, sc,
                                                 egc, S0, ST, o, s);
  return wide ? launch_state<TIn, float, 4>(q, k, v, qs, ks, vs, cu, n_seqs, T, nk, nv, chunk_off, tp, sc, egc,
                                            S0, ST, o, s)
              : launch_state<TIn, float, 1>(q, k, v, qs, ks, vs, cu, n_seqs, T, nk, nv, chunk_off, tp, sc, egc,
                                            S0, ST, o, s);
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
