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
//   chunk_prep    : four waves per (chunk, value head), fully parallel. Grams
//                   K K^T and Q K^T on MFMA from the raw inputs (exact
//                   operands), fp64 cumsum of g, A, the blocked inverse T
//                   (16x16 diagonal blocks by substitution, off-diagonal
//                   blocks on MFMA), P and per-token scalars. Output per
//                   (chunk, value head): one packed 64x64 tile X with
//                   X[i][j] = T[i][j] for j < i and X[63-i][63-j] = P[i][j]
//                   for j <= i (P turned by 180 degrees into the upper
//                   triangle), the scalars a, b, c, beta per token and
//                   exp(G_C); for bf16 inputs X is split into bf16 hi + lo
//                   planes and, per (chunk, key head), the raw K and Q rows
//                   are re-laid in MFMA fragment order.
//   chunk_state   : sequential over a sequence's chunks, one workgroup per
//                   (sequence, value head, 16 value columns). bf16 inputs:
//                   four waves, one per SIMD -- two recurrence waves that
//                   each own half of the rows of S (in MFMA accumulators) and
//                   swap partial products K S through LDS once per chunk, and
//                   two output waves one chunk behind. fp32 inputs use a
//                   simple one-wave variant. Products with an fp32 operand
//                   split it into bf16 hi + lo.
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <type_traits>

#include "gdn_device.hpp"
#include "gdn_internal.hpp"

namespace gdn {
namespace {

constexpr int CH = 64;     // chunk length
constexpr int D = 128;     // dk = dv
constexpr int AP = 68;     // LDS pitch (floats) of 64 x 64 fp32 tiles (16-byte rows)
constexpr float kEps = 1e-6f;

constexpr int TILE_ELEMS = CH * D;   // bf16 elements of one 16 KB operand tile

// Workspace: chunk table | sequence order | per (chunk, value head): 16 KB tile, 1 KB of
// per-token scalars, exp(G_C) | bf16 inputs only, per (chunk, key head): K and
// Q operand tiles of 16 KB each.
// Segment-parallel prefill (one sequence, bf16 inputs, at most eight value
// heads, i.e. at most 64 column slices): the sequence is split into up to
// kMaxSeg segments of whole chunks, which the chunk table then treats as
// sequences. The workspace reserves room for it whenever the shape allows it.
constexpr int kMaxSeg = 16;
inline bool seg_eligible(int n_seqs, int nv, bool bf16) { return bf16 && n_seqs == 1 && nv <= 8; }

struct WsLayout {
  size_t off_chunk_off, off_order, off_tp, off_sc, off_egc, off_kf, off_qf, off_segcu, off_sega, off_segs, off_ring,
      total;
};
// ring of the norm epilogue's row partial sums: per (sequence, value head)
// 6 chunk slots x 4 column pairs x 64 rows of 8 bytes (EPI_RING, below)
constexpr size_t kRingBytesPerUnit = size_t(6) * 4 * 64 * 8;
inline WsLayout ws_layout(int64_t T, int n_seqs, int nk, int nv, bool bf16) {
  const int64_t nch = T / CH + n_seqs;   // >= sum_n ceil(len_n / 64), also for segments of whole chunks
  const bool seg = seg_eligible(n_seqs, nv, bf16);
  const size_t ntab = seg ? kMaxSeg : static_cast<size_t>(n_seqs);   // chunk table entries
  const size_t tile_bytes = static_cast<size_t>(TILE_ELEMS) * 2;
  const size_t state_bytes = static_cast<size_t>(nv) * D * D * sizeof(float);
  WsLayout w{};
  size_t o = 0;
  w.off_chunk_off = o; o += (ntab + 1) * sizeof(int32_t); o = (o + 255) & ~size_t(255);
  w.off_order = o;     o += ntab * sizeof(int32_t); o = (o + 255) & ~size_t(255);
  w.off_tp = o;        o += static_cast<size_t>(nch) * nv * tile_bytes;
  w.off_sc = o;        o += static_cast<size_t>(nch) * nv * CH * sizeof(float4);
  w.off_egc = o;       o += static_cast<size_t>(nch) * nv * sizeof(float); o = (o + 255) & ~size_t(255);
  w.off_kf = w.off_qf = o;
  if (bf16) {
    w.off_kf = o;  o += static_cast<size_t>(nch) * nk * tile_bytes;
    w.off_qf = o;  o += static_cast<size_t>(nch) * nk * tile_bytes;
  }
  w.off_segcu = w.off_sega = w.off_segs = o;
  if (seg) {   // segment bounds | final states of the first pass (D, then M) | incoming states
    w.off_segcu = o; o += (kMaxSeg + 1) * sizeof(int32_t); o = (o + 255) & ~size_t(255);
    w.off_sega = o;  o += 2 * kMaxSeg * state_bytes;
    w.off_segs = o;  o += kMaxSeg * state_bytes;
  }
  w.off_ring = o;
  if (bf16) { o += static_cast<size_t>(n_seqs) * nv * kRingBytesPerUnit; o = (o + 255) & ~size_t(255); }
  w.total = o;
  return w;
}

// ------------------------------------------------------------------ chunk table
// Capped at nch (the workspace's chunk capacity) so a malformed cu_seqlens can
// never index past the workspace.
constexpr int ORDER_MAX = 512;   // batches up to this many sequences are ordered longest first
__global__ void __launch_bounds__(256) chunk_offsets_kernel(const int32_t* __restrict__ cu, int n_seqs,
                                                            int64_t T, int32_t nch, int32_t* __restrict__ off,
                                                            int32_t* __restrict__ order) {
  __shared__ int32_t part[256];
  __shared__ int32_t cnt[ORDER_MAX];
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

  // The state kernel takes the sequences in this order: by chunk count,
  // longest first, so that the longest recurrences start first and the short
  // ones fill in behind them (ties by index; a permutation either way).
  if (n_seqs <= ORDER_MAX) {
    for (int n = tid; n < n_seqs; n += 256) {
      int64_t b, e;
      seq_bounds(cu, n, T, b, e);
      cnt[n] = static_cast<int32_t>((e - b + CH - 1) / CH);
    }
    __syncthreads();
    for (int n = tid; n < n_seqs; n += 256) {
      const int32_t c = cnt[n];
      int rank = 0;
      for (int m = 0; m < n_seqs; ++m) rank += (cnt[m] > c) || (cnt[m] == c && m < n);
      order[rank] = n;
    }
  } else {
    for (int n = tid; n < n_seqs; n += 256) order[n] = n;
  }
}

// Segment table of the segment-parallel prefill: segment p covers tokens
// [b + p L, min(b + (p + 1) L, e)) of the one sequence [b, e) (b = 0, e = T
// without cu_seqlens), L = 64 seg_chunks; segments past e are empty. Written
// as the chunk table of P sequences: bounds, first chunk slots (every
// segment but the last non-empty one holds seg_chunks whole chunks) and the
// identity order.
__global__ void __launch_bounds__(64) segment_table_kernel(const int32_t* __restrict__ cu, int64_t T,
                                                           int seg_chunks, int P, int32_t* __restrict__ seg_cu,
                                                           int32_t* __restrict__ off, int32_t* __restrict__ order) {
  const int p = threadIdx.x;
  if (p > P) return;
  int64_t b = 0, e = T;
  if (cu) {
    b = min(max(static_cast<int64_t>(cu[0]), int64_t(0)), T);
    e = min(max(static_cast<int64_t>(cu[1]), b), T);
  }
  const int64_t nc = (e - b + CH - 1) / CH;
  seg_cu[p] = static_cast<int32_t>(p == P ? e : min(b + static_cast<int64_t>(p) * seg_chunks * CH, e));
  off[p] = static_cast<int32_t>(min(static_cast<int64_t>(p) * seg_chunks, nc));
  if (p < P) order[p] = p;
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

// First chunk slot and chunk count of sequence n. Without cu_seqlens there is
// one sequence and no chunk table is built.
__device__ __forceinline__ void chunk_span(const int32_t* chunk_off, const int32_t* cu, int64_t T, int n,
                                           int& first, int& count) {
  if (!cu) {
    first = 0;
    count = static_cast<int>((T + CH - 1) / CH);
    return;
  }
  first = chunk_off[n];
  count = chunk_off[n + 1] - first;
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
__host__ __device__ constexpr int tile_mi(int p) { return p >= 6 ? 3 : p >= 3 ? 2 : p >= 1 ? 1 : 0; }
__host__ __device__ constexpr int tile_mj(int p) { return p - tile_mi(p) * (tile_mi(p) + 1) / 2; }
// The tile pairs of prep wave w (slot u = 0..2, -1 = none). A wave's pairs
// share row tiles, so each K or Q fragment it needs is read from LDS once per
// k-step: w0 (3,0) (3,1) (3,2); w1 (3,3) (2,0) (2,1); w2 (2,2) (1,0);
// w3 (1,1) (0,0).
__device__ __forceinline__ int wave_pair(int w, int u) {
  return w == 0 ? 6 + u : w == 1 ? (u == 0 ? 9 : 2 + u) : w == 2 ? (u == 0 ? 5 : u == 1 ? 1 : -1) : (u == 0 ? 2 : u == 1 ? 0 : -1);
}

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

// ------------------------------------------------------------------ operand blocks (bf16 inputs)
// The state recurrence reads each operand as whole blocks: one wave's MFMA
// fragment, 64 lanes x 16 bytes with lane l at byte 16 l, so every wave load
// is one contiguous kilobyte. Inside a 32-wide k-step, slot j of lane
// (lr, lg) holds index perm32(lg, j) = 16 (j / 4) + 4 lg + j % 4: slots 0-3
// are the four accumulator rows that lane holds in 16-row tile 2s, slots
// 4-7 those of tile 2s + 1. In that order an accumulator tile already is
// this lane's share of a B operand, so tiles pass between waves through LDS
// with no shuffle. The order also commutes with the 180-degree turn of the
// packed T|P tile: 63 - (32 (1-s) + perm32(3-lg, j)) = 32 s + perm32(lg, 7-j).
constexpr int BLK_ELEMS = 64 * 8;    // bf16 elements of one block
__device__ __forceinline__ int perm32(int lg, int j) { return 16 * (j >> 2) + 4 * lg + (j & 3); }

// K or Q tile in LDS (bf16 [64][EP]; rows >= L hold copies) -> blocks (m, s),
// m = 16-token tile, s = k-step over dk: lane (lr, lg) holds
// X[16m + lr][32s + perm32(lg, j)], rows >= L zero. This call writes tile m's
// four blocks.
template <int EP>
__device__ __forceinline__ void write_row_blocks(const uint16_t* tile, int L, uint16_t* __restrict__ dst, int lane,
                                                 int m) {
  const int lr = lane & 15, lg = lane >> 4;
  const int row = 16 * m + lr;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const uint2 a = *reinterpret_cast<const uint2*>(tile + row * EP + 32 * s + 4 * lg);
    const uint2 b = *reinterpret_cast<const uint2*>(tile + row * EP + 32 * s + 16 + 4 * lg);
    *reinterpret_cast<uint4*>(dst + (4 * m + s) * BLK_ELEMS + lane * 8) =
        zero_if(row >= L, make_uint4(a.x, a.y, b.x, b.y));
  }
}
// packed T|P tile in LDS (fp32 [64][AP]) -> blocks (m, s) per plane, hi plane
// then lo: lane (lr, lg) holds X[16m + lr][32s + perm32(lg, j)]. This call
// writes tile m's blocks.
__device__ __forceinline__ void write_tile_blocks(const float* Tw, uint16_t* __restrict__ dst, int lane, int m) {
  const int lr = lane & 15, lg = lane >> 4;
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const float* r = Tw + (16 * m + lr) * AP + 32 * s + 4 * lg;
    uint2 ah, al, bh, bl;
    split4_packed(*reinterpret_cast<const float4*>(r), ah, al);
    split4_packed(*reinterpret_cast<const float4*>(r + 16), bh, bl);
    *reinterpret_cast<uint4*>(dst + (2 * m + s) * BLK_ELEMS + lane * 8) = make_uint4(ah.x, ah.y, bh.x, bh.y);
    *reinterpret_cast<uint4*>(dst + (8 + 2 * m + s) * BLK_ELEMS + lane * 8) = make_uint4(al.x, al.y, bl.x, bl.y);
  }
}

// acc += A(16x16 fp32 in LDS, row pitch lda) * B, with B held in accumulator
// layout (lane (lr, lg) holds B[4 lg + i][lr]). Ordering the k-slots of lane
// group lg as k = 4 lg + slot makes that the B-operand layout, so B needs no
// trip through LDS.
template <bool BF>
__device__ __forceinline__ void mm16_regb(f32x4& acc, const float* A, int lda, const f32x4& B, int lr, int lg) {
  using M = Mma16<BF, false, false>;
  if constexpr (BF) {
    float a[4], b[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      a[j] = A[lr * lda + 4 * lg + j];
      b[j] = B[j];
    }
    M::run(acc, a, b);
  } else {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const float a[1] = {A[lr * lda + 4 * lg + s]}, b[1] = {B[s]};
      M::run(acc, a, b);
    }
  }
}

// e^x for a decay exponent x <= 0 held in fp64: x log2(e) is formed in fp64
// and rounded once to fp32, then the hardware 2^x (about 1 ulp). The result's
// relative error stays near 1e-7 for every |x| at which it is not negligible.
__device__ __forceinline__ float exp_nonpos(double x) {
  return __builtin_amdgcn_exp2f(static_cast<float>(x * 1.4426950408889634));
}

// ------------------------------------------------------------------ prep
// Four waves per (chunk, value head). The ten lower 16x16 tile pairs (mi, mj)
// of the Grams, A and P are dealt out so that a wave's pairs share row tiles
// (wave_pair);
// wave w writes token tile w of every operand block; the off-diagonal blocks
// of T are formed one level at a time with one wave per block.
template <typename TIn>
constexpr int prep_pitch() { return sizeof(TIn) == 2 ? 136 : 132; }   // 16-byte rows
template <typename TIn>
constexpr size_t prep_lds_bytes() {
  constexpr size_t tiles = 2 * CH * prep_pitch<TIn>() * sizeof(TIn);
  constexpr size_t at = 2 * CH * AP * sizeof(float);
  return (tiles > at ? tiles : at) + CH * sizeof(double) + 4 * CH * sizeof(float);
}
constexpr int PREP_WAVES = 4;

// k-step s of the Grams of tile pair P (K K^T and Q K^T, and Q Q^T on the
// diagonal), from the K and Q tiles in LDS (row pitch EP)
template <int P, typename TIn, int EP>
__device__ __forceinline__ void gram_step(const TIn* Ks, const TIn* Qs, int lr, int lg, int s, f32x4& gkk,
                                          f32x4& gqk, f32x4& gqq) {
  if constexpr (P >= 0) {
    constexpr int mi = tile_mi(P), mj = tile_mj(P);
    constexpr bool BF = sizeof(TIn) == 2;
    using MG = Mma<BF, true, true>;
    constexpr int KS = MG::KS, KPL = MG::KPL;
    if constexpr (BF) {   // raw bf16 fragments, one 16-byte LDS read each
      const int kk = s * KS + KPL * lg;
      const bf16x8 ak = *reinterpret_cast<const bf16x8*>(Ks + (16 * mi + lr) * EP + kk);
      const bf16x8 aq = *reinterpret_cast<const bf16x8*>(Qs + (16 * mi + lr) * EP + kk);
      const bf16x8 bk = *reinterpret_cast<const bf16x8*>(Ks + (16 * mj + lr) * EP + kk);
      gkk = mfma_bf16(ak, bk, gkk);
      gqk = mfma_bf16(aq, bk, gqk);
      if constexpr (mi == mj) gqq = mfma_bf16(aq, aq, gqq);
    } else {
      float ak[KPL], aq[KPL], bk[KPL];
#pragma unroll
      for (int j = 0; j < KPL; ++j) {
        const int kk = s * KS + KPL * lg + j;
        ak[j] = tof(Ks[(16 * mi + lr) * EP + kk]);
        aq[j] = tof(Qs[(16 * mi + lr) * EP + kk]);
        bk[j] = tof(Ks[(16 * mj + lr) * EP + kk]);
      }
      MG::run(gkk, ak, bk);
      MG::run(gqk, aq, bk);
      if constexpr (mi == mj) MG::run(gqq, aq, aq);
    }
  }
}
template <int P0, int P1, int P2, typename TIn, int EP>
__device__ __forceinline__ void gram_pairs(const TIn* Ks, const TIn* Qs, int lr, int lg, f32x4 (&gkk)[3],
                                           f32x4 (&gqk)[3], f32x4 (&gqq)[3]) {
  constexpr int KS = Mma<sizeof(TIn) == 2, true, true>::KS;
#pragma unroll
  for (int s = 0; s < D / KS; ++s) {
    gram_step<P0, TIn, EP>(Ks, Qs, lr, lg, s, gkk[0], gqk[0], gqq[0]);
    gram_step<P1, TIn, EP>(Ks, Qs, lr, lg, s, gkk[1], gqk[1], gqq[1]);
    gram_step<P2, TIn, EP>(Ks, Qs, lr, lg, s, gkk[2], gqk[2], gqq[2]);
  }
}

// Causal conv1d (4 taps) + SiLU folded into the chunk kernels: x holds the
// packed q | k | v channels (conv_dim = 2 nk D + nv D, bf16); the conv state
// [n_seqs, conv_dim, state_len] (or none: zero history) supplies the three
// inputs before each sequence's first token. seq_split: the launch's
// sequences are the segments of one sequence (starting at cu[0]), so the
// three inputs before a segment's first token are x rows unless it is the
// first segment.
struct ConvIn {
  const float* w;          // [conv_dim, 4]
  const float* b;          // [conv_dim] or null
  const uint16_t* st;      // conv state in, or null
  int state_len;
  int conv_dim;
  int seq_split;
};

// Gated RMSNorm epilogue inside the wide state kernel (with the conv): the
// kernel writes y = o rms(o)^-1 (1 + w) z sigmoid(z) per (token, value head)
// row of 128 in place of o. A row's 128 columns come from the four workgroups
// (column pairs) of its head: each publishes its row partial sums of squares
// of chunk c in ring slot c % EPI_RING as one 64-bit word (the fp32 bits, and
// c + 1 in the high half, so a reader needs no separate flag or fence), and
// normalizes chunk c, kept in an LDS ring, EPI_LAG chunks later, once the
// four words of each row carry that tag. A workgroup publishes chunk c before
// it waits for chunk c - EPI_LAG, so waits only ever point at older chunks,
// and the launch is cooperative (all workgroups resident). Each wait is
// bounded (EPI_SPIN polls); a row whose partial sums never arrive comes out
// NaN rather than hanging the device. The ring is cleared before each launch.
struct EpiIn {
  const uint16_t* z;             // [T, nv, 128] bf16, dense
  const float* w;                // [128]
  float eps;
  unsigned long long* ring;      // [n_units][EPI_RING][4 pairs][64 rows]
};
constexpr int EPI_LAG = 2;
constexpr int EPI_RING = 6;      // >= 2 EPI_LAG + 1: no slot is rewritten before its last reader read it
static_assert(kRingBytesPerUnit == size_t(EPI_RING) * 4 * CH * 8, "ring size");

__global__ void __launch_bounds__(256) clear_u64_kernel(unsigned long long* __restrict__ p, int64_t n) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i < n) p[i] = 0ull;
}
constexpr int EPI_SPIN = 1 << 20;

// (at most 128 VGPRs: four waves per SIMD, i.e. four blocks per CU, which is
// also what the LDS holds)
// GM selects the per-token gating inputs: 0 = g and beta (fp32) given;
// 1 / 2 = the raw a and b (bf16 / fp32), gated here exactly as the separate
// gating kernel does (same expressions), so both routes give the same bits.
// CV: q is the conv input x (channel 0 of the packed q | k | v) with token
// stride qs; k and ks are unused. The K and Q tiles are then the conv + SiLU
// outputs, rounded to bf16 as a stored conv output would be.
template <typename TIn, int GM, bool CV, bool RG>
__global__ void __launch_bounds__(64 * PREP_WAVES) __attribute__((amdgpu_waves_per_eu(RG ? 3 : 4))) chunk_prep_kernel(
    const TIn* __restrict__ q, const TIn* __restrict__ k, int64_t qs, int64_t ks,
    const void* __restrict__ ga, const void* __restrict__ gb, const float* __restrict__ A_log,
    const float* __restrict__ dt_bias, const int32_t* __restrict__ cu,
    int n_seqs, int64_t T, int nk, int nv, float scale, int l2, const int32_t* __restrict__ chunk_off,
    float* __restrict__ tp, float4* __restrict__ sc, float* __restrict__ egc, uint16_t* __restrict__ kf,
    uint16_t* __restrict__ qf, ConvIn cv, int hg_arg) {
  constexpr bool BF = sizeof(TIn) == 2;
  const int hg = RG ? hg_arg : 1;
  constexpr int EP = prep_pitch<TIn>();
  constexpr size_t tiles = 2 * CH * EP * sizeof(TIn);
  constexpr size_t at = 2 * CH * AP * sizeof(float);
  constexpr size_t head = tiles > at ? tiles : at;
  constexpr int NT = 64 * PREP_WAVES;

  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  TIn* Ks = reinterpret_cast<TIn*>(smem);          // [64][EP]   (input tiles)
  TIn* Qs = Ks + CH * EP;                          // [64][EP]
  float* Aw = reinterpret_cast<float*>(smem);      // [64][AP]   (after the Grams)
  float* Tw = Aw + CH * AP;                        // [64][AP]
  double* Gs = reinterpret_cast<double*>(smem + head);
  float* rk_s = reinterpret_cast<float*>(Gs + CH);
  float* rq_s = rk_s + CH;
  float* b_s = rq_s + CH;

  // !RG: one workgroup per (chunk, value head), heads fastest (the value
  // heads of one key head, and the per-token g and beta of all heads, are
  // read by neighbouring workgroups); RG (hg = nv / nk): one workgroup per
  // (chunk, key head), which forms the K and Q tiles (and their conv), the
  // Grams and the norms once and then runs steps 5-9 for each of the key
  // head's value heads in turn. One-dimensional grid (its y dimension would
  // cap the chunk count at 65536).
  const int nh = nv / hg;   // workgroups per chunk
  const int h0 = static_cast<int>(blockIdx.x % static_cast<unsigned>(nh)) * hg;
  const int c = static_cast<int>(blockIdx.x / static_cast<unsigned>(nh));
  const int hk = h0 / (nv / nk);
  const int total = cu ? chunk_off[n_seqs] : static_cast<int>((T + CH - 1) / CH);
  if (c >= total) return;
  const int n = cu ? find_le(chunk_off, n_seqs, c) : 0;
  int64_t s_begin, s_end;
  seq_bounds(cu, n, T, s_begin, s_end);
  const int64_t t0 = s_begin + static_cast<int64_t>(c - (cu ? chunk_off[n] : 0)) * CH;
  const int L = static_cast<int>(min<int64_t>(CH, s_end - t0));
  const int tid = threadIdx.x, lane = tid & 63, lr = lane & 15, lg = lane >> 4;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  // per-token gating inputs (wave 0, lane = token), issued first so their
  // latency overlaps the tile loads and the Grams
  using TA = std::conditional_t<GM == 1, uint16_t, float>;
  const int64_t gi0 = (t0 + min(lane, L - 1)) * nv + h0;
  TA ga_ld = static_cast<const TA*>(ga)[gi0];
  TA gb_ld = static_cast<const TA*>(gb)[gi0];

  // 1. K and Q tiles into LDS; rows past the sequence end re-read the last
  //    valid row (or are zero after the conv): their norms are forced to 0
  //    below, so they contribute nothing to A, P or the scalars
  if constexpr (CV) {
    static_assert(BF, "the conv prologue takes bf16 inputs");
    // thread -> (K | Q, 8-channel segment, block of 8 rows); its window runs
    // over rows 8 rb - 3 .. 8 rb + 7 of the chunk
    const int grp = tid & 31, rb = tid >> 5;
    const int zq = grp >> 4, seg = grp & 15;
    const int ch0 = (zq ? 0 : nk * D) + hk * D + 8 * seg;
    float wt[4][8], bs[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
#pragma unroll
      for (int j = 0; j < 4; ++j) wt[j][e] = cv.w[(ch0 + e) * 4 + j];
      bs[e] = cv.b ? cv.b[ch0 + e] : 0.0f;
    }
    // the sequence's own first token and conv-state row (a split sequence's)
    const int64_t hb = cv.seq_split ? cu[0] : s_begin;
    const int hn = cv.seq_split ? 0 : n;
    uint4 raw[11];
#pragma unroll
    for (int u = 0; u < 11; ++u) {
      const int r = 8 * rb - 3 + u;
      const int64_t t = t0 + r;
      if (r < L && t >= hb)
        raw[u] = *reinterpret_cast<const uint4*>(q + t * qs + ch0);
      else if (t < hb && cv.st)   // history of the sequence (t - hb in -3 .. -1)
        raw[u] = gather8_bf16(cv.st + (static_cast<int64_t>(hn) * cv.conv_dim + ch0) * cv.state_len + cv.state_len +
                                  (t - hb),
                              cv.state_len);
      else
        raw[u] = make_uint4(0u, 0u, 0u, 0u);
    }
    // each input row is widened once and slides through the window; the
    // arithmetic per output is that of conv4_silu8_bf16 (same bits)
    TIn* dst = zq ? Qs : Ks;
    float win[3][8];
#pragma unroll
    for (int j = 0; j < 3; ++j)
#pragma unroll
      for (int e = 0; e < 8; ++e) win[j][e] = bf16_elem(raw[j], e);
#pragma unroll
    for (int u = 3; u < 11; ++u) {
      const int r = 8 * rb + u - 3;
      float cur[8], y[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        cur[e] = bf16_elem(raw[u], e);
        float acc = bs[e];
        acc = fmaf(wt[0][e], win[0][e], acc);
        acc = fmaf(wt[1][e], win[1][e], acc);
        acc = fmaf(wt[2][e], win[2][e], acc);
        acc = fmaf(wt[3][e], cur[e], acc);
        y[e] = siluf_(acc);
      }
      *reinterpret_cast<uint4*>(dst + r * EP + 8 * seg) = zero_if(r >= L, pack8_bf16(y));
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        win[0][e] = win[1][e];
        win[1][e] = win[2][e];
        win[2][e] = cur[e];
      }
    }
  } else {
    const TIn* kb = k + t0 * ks + static_cast<int64_t>(hk) * D;
    const TIn* qb = q + t0 * qs + static_cast<int64_t>(hk) * D;
#pragma unroll
    for (int it = 0; it < CH * 16 / NT; ++it) {
      const int idx = it * NT + tid, row = idx >> 4, seg = idx & 15;
      const int rr = min(row, L - 1);
      copy8(kb + rr * ks + seg * 8, Ks + row * EP + seg * 8);
      copy8(qb + rr * qs + seg * 8, Qs + row * EP + seg * 8);
    }
  }
  __syncthreads();

  // 2. Grams on this wave's lower 16x16 tile pairs (wave_pair), kept in
  //    registers; on the diagonal pairs also Q Q^T, whose diagonal is |q_i|^2
  //    (|k_i|^2 is the diagonal of K K^T)
  constexpr int NP = 3;
  f32x4 gkk[NP], gqk[NP], gqq[NP];
#pragma unroll
  for (int u = 0; u < NP; ++u) {
    gkk[u] = f32x4{0.f, 0.f, 0.f, 0.f};
    gqk[u] = f32x4{0.f, 0.f, 0.f, 0.f};
    gqq[u] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  if (wv == 0) gram_pairs<6, 7, 8, TIn, EP>(Ks, Qs, lr, lg, gkk, gqk, gqq);
  else if (wv == 1) gram_pairs<9, 3, 4, TIn, EP>(Ks, Qs, lr, lg, gkk, gqk, gqq);
  else if (wv == 2) gram_pairs<5, 1, -1, TIn, EP>(Ks, Qs, lr, lg, gkk, gqk, gqq);
  else gram_pairs<2, 0, -1, TIn, EP>(Ks, Qs, lr, lg, gkk, gqk, gqq);
  // 3. bf16 inputs: K and Q operand blocks of the state recurrence, once
  //     per key head: K by its first value head, Q by its last; wave wv
  //     writes token tile wv
  if constexpr (BF) {
    const int r = nv / nk, rho = h0 % r;
    const size_t kt = (static_cast<size_t>(c) * nk + hk) * TILE_ELEMS;
    if (rho == 0) write_row_blocks<EP>(Ks, L, kf + kt, lane, wv);
    if (rho + hg - 1 == r - 1) write_row_blocks<EP>(Qs, L, qf + kt, lane, wv);
  }
  // 4. |k_i|^2 and |q_i|^2 from the Gram diagonals (pairs 0, 2, 5, 9)
#pragma unroll
  for (int u = 0; u < NP; ++u) {
    const int p = wave_pair(wv, u);
    if (p < 0) break;
    const int mi = tile_mi(p), mj = tile_mj(p);
    if (mi == mj && lr >= 4 * lg && lr < 4 * lg + 4) {
      const int row = 16 * mi + lr;
      const float skk = gkk[u][lr - 4 * lg], sqq = gqq[u][lr - 4 * lg];
      rk_s[row] = row < L ? (l2 ? rsqrtf(skk + kEps) : 1.0f) : 0.0f;
      rq_s[row] = row < L ? (l2 ? rsqrtf(sqq + kEps) : 1.0f) : 0.0f;
    }
  }
  for (int hh = 0; hh < hg; ++hh) {
  const int h = h0 + hh;
  if (hh > 0) {
    __syncthreads();   // the previous head's Aw, Tw, Gs and b_s are read
    if (wv == 0) {
      const int64_t gi = (t0 + min(lane, L - 1)) * nv + h;
      ga_ld = static_cast<const TA*>(ga)[gi];
      gb_ld = static_cast<const TA*>(gb)[gi];
    }
  }
  // 5. chunk-local cumulative decay in fp64 (wave 0, lane = token)
  if (wv == 0) {
    const bool valid = lane < L;
    float g_ld, b_ld;
    if constexpr (GM == 0) {
      g_ld = ga_ld;
      b_ld = gb_ld;
    } else {
      g_ld = -exp_(A_log[h]) * softplusf_(Elem<TA>::cvt(ga_ld) + dt_bias[h]);
      b_ld = sigmoidf_(Elem<TA>::cvt(gb_ld));
    }
    double G = valid ? g_ld : 0.0f;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const double y = __shfl_up(G, off, 64);
      if (lane >= off) G += y;
    }
    Gs[lane] = G;
    b_s[lane] = valid ? b_ld : 0.0f;
  }
  __syncthreads();   // norms, G, beta visible; K/Q tiles no longer read

  // 6. A (into LDS) and P (kept in registers, the QK^T Gram kept for the
  //    next head); per-token values are read before the first write to Aw
  //    (which could alias them as far as the compiler knows)
  f32x4 pq[NP];
  {
    double Gc[NP], Gr[NP][4];
    float rkc[NP], ar[NP][4], pr[NP][4];
#pragma unroll
    for (int u = 0; u < NP; ++u) {
      const int p = max(wave_pair(wv, u), 0);
      const int mi = tile_mi(p), mj = tile_mj(p);
      Gc[u] = Gs[16 * mj + lr];
      rkc[u] = rk_s[16 * mj + lr];
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int i = 16 * mi + 4 * lg + ii;
        Gr[u][ii] = Gs[i];
        ar[u][ii] = b_s[i] * rk_s[i];
        pr[u][ii] = scale * rq_s[i];
      }
    }
#pragma unroll
    for (int u = 0; u < NP; ++u) {
      const int p = wave_pair(wv, u);
      if (p < 0) break;
      const int mi = tile_mi(p), mj = tile_mj(p);
      const int j = 16 * mj + lr;
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int i = 16 * mi + 4 * lg + ii;
        const float dec = (j <= i) ? exp_nonpos(Gr[u][ii] - Gc[u]) : 0.0f;
        Aw[i * AP + j] = (j < i) ? ar[u][ii] * rkc[u] * dec * gkk[u][ii] : 0.0f;
        pq[u][ii] = (j <= i) ? pr[u][ii] * rkc[u] * dec * gqk[u][ii] : 0.0f;
      }
    }
  }
  __syncthreads();

  // 7. T = (I + A)^-1: the four diagonal 16x16 blocks by forward substitution
  //    (wave 0, lane = (block lg, column lr)), then the off-diagonal blocks
  //    T_IJ = -T_II * sum_{M=J}^{I-1} A_IM T_MJ on MFMA, one level at a time,
  //    block (J + lvl, J) on wave J
  if (wv == 0) {
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
    }
    // stored after the loop, so no store sits between the reads of A and
    // they can all be issued ahead of the arithmetic
#pragma unroll
    for (int i = 0; i < 16; ++i) Tw[(16 * I + i) * AP + 16 * I + jc] = t[i];
  }
  __syncthreads();
#pragma unroll
  for (int lvl = 1; lvl <= 3; ++lvl) {
    if (wv <= 3 - lvl) {
      const int J = wv, I = J + lvl;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      for (int Mb = J; Mb < I; ++Mb)
        mm16<BF>(acc, Aw + 16 * I * AP + 16 * Mb, AP, Tw + 16 * Mb * AP + 16 * J, AP, lr, lg);
      f32x4 acc2 = {0.f, 0.f, 0.f, 0.f};
      mm16_regb<BF>(acc2, Tw + 16 * I * AP + 16 * I, AP, acc, lr, lg);
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) Tw[(16 * I + 4 * lg + ii) * AP + 16 * J + lr] = -acc2[ii];
    }
    __syncthreads();
  }

  // 8. P into the upper triangle turned by 180 degrees: X[63-i][63-j] = P[i][j], j <= i
#pragma unroll
  for (int u = 0; u < NP; ++u) {
    const int p = wave_pair(wv, u);
    if (p < 0) break;
    const int mi = tile_mi(p), mj = tile_mj(p);
    const int j = 16 * mj + lr;
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      const int i = 16 * mi + 4 * lg + ii;
      if (j <= i) Tw[(63 - i) * AP + (63 - j)] = pq[u][ii];
    }
  }
  __syncthreads();

  // 9. packed tile and scalars to the workspace (tile rows 16 wv .. +15 per wave)
  const size_t tile = static_cast<size_t>(c) * nv + h;
  if constexpr (BF) {
    write_tile_blocks(Tw, reinterpret_cast<uint16_t*>(tp) + tile * TILE_ELEMS, lane, wv);
  } else {
    float* X = tp + tile * CH * CH;
#pragma unroll
    for (int it = 0; it < CH * CH / 4 / NT; ++it) {
      const int idx = it * NT + tid, row = idx >> 4, c4 = (idx & 15) * 4;
      *reinterpret_cast<float4*>(X + row * CH + c4) = *reinterpret_cast<const float4*>(Tw + row * AP + c4);
    }
  }
  if (wv == 1) {   // per-token scalars (lane = token) and exp(G_C)
    const double G = Gs[lane], GC = Gs[CH - 1];
    const float eG = expf(static_cast<float>(G));
    const float rk_i = rk_s[lane], rq_i = rq_s[lane], bi = b_s[lane];
    const float sa = scale * rq_i * eG, sb = bi * rk_i * eG, scc = rk_i * expf(static_cast<float>(GC - G));
    if constexpr (BF) {   // planes a | b | c | beta
      float* sp = reinterpret_cast<float*>(sc + tile * CH);
      sp[lane] = sa;
      sp[CH + lane] = sb;
      sp[2 * CH + lane] = scc;
      sp[3 * CH + lane] = bi;
    } else {
      sc[tile * CH + lane] = make_float4(sa, sb, scc, bi);
    }
    if (lane == 0) egc[tile] = expf(static_cast<float>(GC));
  }
  }   // value heads
}

// Workgroup -> (unit = sequence slot x nv + value head, 16-column slice) for
// the state kernels. Workgroup b runs on XCD b % 8. The 8 slices of a unit,
// and the r value heads of one key head, go to one XCD (they share that
// chunk's operand blocks in its L2); consecutive key-head groups go to
// consecutive XCDs, so every XCD gets its share of each sequence's units
// (taken longest sequence first). Unit counts that do not split that way fall
// back to one unit per XCD in turn, then to contiguous blocks of units.
__device__ __forceinline__ void state_unit_slice(int b, int n_units, int r, int& unit_slot, int& slice) {
  const int j = b >> 3;          // this workgroup's position on its XCD
  if (n_units % (8 * r) == 0) {
    slice = j & 7;
    const int k = j >> 3;        // unit position on the XCD
    unit_slot = ((k / r) * 8 + (b & 7)) * r + k % r;
  } else if (n_units % 8 == 0) {
    slice = j & 7;
    unit_slot = ((j >> 3) << 3) + (b & 7);
  } else {
    const int bid = xcd_swizzle(b, n_units * 8);
    slice = bid & 7;
    unit_slot = bid >> 3;
  }
}

constexpr int BLK_BYTES = BLK_ELEMS * 2;

__device__ __forceinline__ bf16x8 as_bf16x8(const uint4& u) { return __builtin_bit_cast(bf16x8, u); }
__device__ __forceinline__ uint4 and4(const uint4& a, const uint4& m) {
  return make_uint4(a.x & m.x, a.y & m.y, a.z & m.z, a.w & m.w);
}
// reverse the order of 8 packed bf16
__device__ __forceinline__ uint4 rev8(const uint4& a) {
  auto sw = [](uint32_t d) { return (d >> 16) | (d << 16); };
  return make_uint4(sw(a.w), sw(a.z), sw(a.y), sw(a.x));
}
__device__ __forceinline__ float bits_f(uint32_t u) { return __builtin_bit_cast(float, u); }

// ------------------------------------------------------------------ state: bf16 inputs, 4 waves per 16 columns
// One workgroup per (sequence, value head, 16 value columns), one wave per SIMD.
//   Waves 0 and 1 (recurrence): wave h owns rows 64h .. 64h+63 of S (128 x 16
//     fp32, four MFMA accumulators). Per chunk it forms its partial product
//     X_h = K[:, rows of h] S_h and swaps it with the other half through LDS
//     (the chunk's one barrier); both waves then form X = X_0 + X_1,
//     R = beta v - b X, U = R + T_strict R and c U, bit-identical in both,
//     and update their own rows: S_h = e^{G_C} S_h + K[:, rows of h]^T (c U).
//   Waves 2 and 3 (output), one chunk behind: Y^T = S^T Q^T for two token
//     tiles, then O^T = a Y^T + U^T P^T, from S and U published in LDS; the
//     operands are swapped so that a lane holds 4 consecutive columns of one
//     token row and the tile goes out as one 16-byte store per lane. Wave 2
//     takes tiles 0 and 3, wave 3 tiles 1 and 2 (equal P work).
// The output waves also stage chunk inputs in LDS for the recurrence waves,
// one chunk ahead: wave 2 the masked T blocks (both recurrence waves use all
// of them), wave 3 the per-token scalars, exp(G_C) and beta * v in
// accumulator layout. The K^T operand of the state update is not loaded:
// each recurrence wave writes the K blocks it holds for K S to LDS and reads
// them back transposed.
//
// Barrier B(c) separates: the recurrence waves' S_c (as bf16 hi | lo) and
// partial X_c, and the staged inputs of chunk c, all written before it; after
// it the recurrence waves finish chunk c and start c+1, and the output waves
// form Y of chunk c and O of chunk c-1 (U_{c-1} was written before B(c)).
// Every LDS buffer shared between waves is double-buffered by chunk parity:
// a buffer written between B(c-1) and B(c) is read only between B(c) and
// B(c+1). The K blocks are private to their wave (written and read back by
// it in program order).

constexpr int KL_BLK = 64 * 16 + 4 * 64;   // one padded K block in LDS

// LDS transpose read (ds_read_b64_tr_b16): within each 16-lane group, lane i
// receives in slot j the (i % 4)-th 16-bit element of the 8 bytes addressed
// by lane 4 j + i / 4 of the group.
typedef short i16x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint2 lds_tr16(const unsigned char* p) {
  const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4*)(p));
  return __builtin_bit_cast(uint2, v);
}
// lane l's 16 bytes in a padded LDS K block
__device__ __forceinline__ int kl_lane(int l) { return 16 * l + 64 * (l >> 4); }

// A pass of the segment-parallel prefill (one sequence split into P segments
// of whole chunks, each a sequence of the chunk table). P = 0: an ordinary
// launch. P > 0: launch sequence nn < P runs segment nn from a zero state
// (its local final state D), and nn >= P runs segment nn - P from the
// identity with v = 0 (its transition M); final states go to ST[nn].
// no_out: no output stores. st_only >= 0: only that sequence writes its final
// state, to ST[0].
struct SegRun {
  int P;
  int no_out;
  int st_only;
};

// CV: v is the conv input x at the first value channel (token stride vs); the
// output waves apply the conv + SiLU to the value rows as they stage them,
// wave 2 for tokens 0-31 of a chunk and wave 3 for tokens 32-63.
// DUAL: XPX and SBX single-buffered behind a second barrier per chunk, B'(c)
// (the recurrence waves' end of chunk c; the output waves have read S_c by
// then), so that the LDS of two workgroups fits one CU.
template <typename TO, bool CV, bool DUAL>
__global__ void __launch_bounds__(256) chunk_state_bf16_kernel(
    const uint16_t* __restrict__ v, int64_t vs, const int32_t* __restrict__ cu, int n_seqs, int64_t T, int nk,
    int nv, const int32_t* __restrict__ chunk_off, const uint16_t* __restrict__ xf, const float* __restrict__ scp,
    const float* __restrict__ egc, const uint16_t* __restrict__ kf, const uint16_t* __restrict__ qf,
    const int32_t* __restrict__ order, const float* __restrict__ S0, float* __restrict__ ST, TO* __restrict__ o,
    ConvIn cv, SegRun seg) {
  __shared__ f32x4 XPX[DUAL ? 1 : 2][2][4][64];   // partial X: [parity][half][token tile][lane]
  __shared__ uint4 SBX[DUAL ? 1 : 2][2][4][64];   // S as B operand: [parity][hi | lo][dk k-step][lane]
  constexpr int PB = DUAL ? 0 : 1;       // parity mask of XPX and SBX
  __shared__ f32x4 UXF[2][4][64];        // U, accumulator layout: [parity][token tile][lane]
  __shared__ f32x4 BVS[2][4][64];        // beta * v, accumulator layout
  __shared__ uint4 TSX[2][12][64];       // masked T blocks: [parity][hi (6) | lo (6)][lane]
  // each recurrence wave's K blocks of the current chunk, read back transposed;
  // lane l at byte 16 l + 64 (l / 16) of its block (the pad spreads the
  // transposed reads over all banks)
  __shared__ __attribute__((aligned(16))) unsigned char KLX[2][8][KL_BLK];
  __shared__ __attribute__((aligned(16))) float SCS[2][4 * CH];   // planes a | b | c | beta
  __shared__ float EGS[2];               // exp(G_C)

  int slot, slice;
  state_unit_slice(blockIdx.x, gridDim.x / 8, nv / nk, slot, slice);
  // sequences in the chunk table's order (longest first), value heads fastest
  const int nn = seg.P ? slot / nv : (cu ? order[slot / nv] : 0);
  const bool trans = seg.P && nn >= seg.P;   // transition run: S0 = I, v = 0
  const int n = trans ? nn - seg.P : nn, h = slot % nv;
  const int unit = nn * nv + h;
  const int hk = h / (nv / nk);
  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 15, lg = lane >> 4;
  const int col = slice * 16 + lr;
  const uint32_t lo16 = static_cast<uint32_t>(lane * 16);

  int64_t s_begin, s_end;
  seq_bounds(cu, n, T, s_begin, s_end);
  int cbase, nchunks;
  chunk_span(chunk_off, cu, T, n, cbase, nchunks);
  // with the conv: the sequence's own first token and conv-state row (those
  // of the split sequence when the launch's sequences are its segments)
  const int64_t hb = cv.seq_split ? cu[0] : s_begin;
  const int hn = cv.seq_split ? 0 : n;

  if (w < 2) {
    // ================================================================ recurrence waves
    // The half is a compile-time constant in each instantiation: register
    // arrays are then indexed by constants only (a wave-uniform runtime index
    // into a register array becomes indirect register moves, whose reads of
    // fresh MFMA results the compiler does not protect with wait states).
    auto rec_role = [&](auto hfc) {
      constexpr int hf = decltype(hfc)::value;
      f32x4 S[4];                          // rows 64 hf + 16 tt + 4 lg + i, column col
#pragma unroll
      for (int tt = 0; tt < 4; ++tt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          S[tt][i] = S0 ? S0[(static_cast<int64_t>(unit) * D + 64 * hf + 16 * tt + 4 * lg + i) * D + col]
                        : (trans && 64 * hf + 16 * tt + 4 * lg + i == col ? 1.0f : 0.0f);

      if (nchunks > 0) {
        // operand blocks of one chunk, one register set: each group is reloaded
        // for the next chunk right after its last use
        uint4 kb[4][2];                    // K (token tile m, dk k-step 2 hf + kk)
        auto load_k = [&](int cc) {
          const size_t kt = static_cast<size_t>(cbase + cc) * nk + hk;
          const rsrc_t r = make_rsrc(kf + kt * TILE_ELEMS, TILE_ELEMS * 2);
#pragma unroll
          for (int m = 0; m < 4; ++m)
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) kb[m][kk] = bload16(r, (4 * m + 2 * hf + kk) * BLK_BYTES + lo16);
        };
        f32x4 Xp[4];
        // S_c as B operand (published for the output waves) and this half's X_c
        auto first_half = [&](int c) {
          const int buf = c & 1;
          uint4 sh[2], sl[2];
#pragma unroll
          for (int kk = 0; kk < 2; ++kk) {
            uint2 h0, l0, h1, l1;
            split4_packed(make_float4(S[2 * kk][0], S[2 * kk][1], S[2 * kk][2], S[2 * kk][3]), h0, l0);
            split4_packed(make_float4(S[2 * kk + 1][0], S[2 * kk + 1][1], S[2 * kk + 1][2], S[2 * kk + 1][3]), h1, l1);
            sh[kk] = make_uint4(h0.x, h0.y, h1.x, h1.y);
            sl[kk] = make_uint4(l0.x, l0.y, l1.x, l1.y);
            SBX[buf & PB][0][2 * hf + kk][lane] = sh[kk];
            SBX[buf & PB][1][2 * hf + kk][lane] = sl[kk];
          }
#pragma unroll
          for (int m = 0; m < 4; ++m) {
            f32x4 x = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
              x = mfma_bf16(as_bf16x8(kb[m][kk]), as_bf16x8(sl[kk]), x);
              x = mfma_bf16(as_bf16x8(kb[m][kk]), as_bf16x8(sh[kk]), x);
            }
            Xp[m] = x;
            XPX[buf & PB][hf][m][lane] = x;
#pragma unroll
            for (int kk = 0; kk < 2; ++kk)
              *reinterpret_cast<uint4*>(&KLX[hf][2 * m + kk][kl_lane(lane)]) = kb[m][kk];
          }
          load_k(min(c + 1, nchunks - 1));
        };
        // the rest of chunk c: X, R, U, c U, and the update of this half of S
        auto second_half = [&](int c) {
          const int buf = c & 1;
          // K^T blocks of this wave's rows of S (dk tile 4 hf + tt, token
          // k-step s), read transposed from this chunk's K blocks: addressing
          // lane (lr, lg) points at token 32 s + 16 h + 4 lg + lr / 4, dk
          // 16 tt + 4 (lr % 4) .. +3, which sits in block (2 s + h, tt / 2),
          // block lane 16 (lr % 4) + 4 lg + lr / 4, bytes 8 (tt % 2) ..
          // Issued first: their latency hides under R, U and c U.
          uint4 kta[4][2];
          {
            const int kl = kl_lane(16 * (lr & 3) + 4 * lg + (lr >> 2));
#pragma unroll
            for (int tt = 0; tt < 4; ++tt)
#pragma unroll
              for (int s = 0; s < 2; ++s) {
                const uint2 x0 = lds_tr16(&KLX[hf][2 * (2 * s) + tt / 2][kl + 8 * (tt & 1)]);
                const uint2 x1 = lds_tr16(&KLX[hf][2 * (2 * s + 1) + tt / 2][kl + 8 * (tt & 1)]);
                kta[tt][s] = make_uint4(x0.x, x0.y, x1.x, x1.y);
              }
          }
          f32x4 R[4];
#pragma unroll
          for (int m = 0; m < 4; ++m) {
            const f32x4 xo = XPX[buf & PB][1 - hf][m][lane];
            const f32x4 bv = BVS[buf][m][lane];
            const float4 bb = *reinterpret_cast<const float4*>(&SCS[buf][CH + 16 * m + 4 * lg]);
            const float bbv[4] = {bb.x, bb.y, bb.z, bb.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) R[m][i] = bv[i] - bbv[i] * (Xp[m][i] + xo[i]);
          }
          uint4 rh[2], rl[2];              // R as B operand, token k-steps 0, 1
#pragma unroll
          for (int s = 0; s < 2; ++s) {
            uint2 h0, l0, h1, l1;
            split4_packed(make_float4(R[2 * s][0], R[2 * s][1], R[2 * s][2], R[2 * s][3]), h0, l0);
            split4_packed(make_float4(R[2 * s + 1][0], R[2 * s + 1][1], R[2 * s + 1][2], R[2 * s + 1][3]), h1, l1);
            rh[s] = make_uint4(h0.x, h0.y, h1.x, h1.y);
            rl[s] = make_uint4(l0.x, l0.y, l1.x, l1.y);
          }
          // T blocks (m, s): (0,0) (1,0) (2,0) (2,1) (3,0) (3,1), masked, hi | lo
          uint4 mh[6], ml[6];
#pragma unroll
          for (int b = 0; b < 6; ++b) {
            mh[b] = TSX[buf][b][lane];
            ml[b] = TSX[buf][6 + b][lane];
          }
          // U = R + T_strict R
          f32x4 U[4];
          auto tr = [&](f32x4& acc, int b, int s) {
            acc = mfma_bf16(as_bf16x8(ml[b]), as_bf16x8(rh[s]), acc);
            acc = mfma_bf16(as_bf16x8(mh[b]), as_bf16x8(rl[s]), acc);
            acc = mfma_bf16(as_bf16x8(mh[b]), as_bf16x8(rh[s]), acc);
          };
#pragma unroll
          for (int m = 0; m < 4; ++m) U[m] = R[m];
          tr(U[0], 0, 0);
          tr(U[1], 1, 0);
          tr(U[2], 2, 0);
          tr(U[3], 4, 0);
          tr(U[2], 3, 1);
          tr(U[3], 5, 1);
          // U of this wave's two tiles for the output waves; c U as B operand
#pragma unroll
          for (int u = 0; u < 2; ++u) UXF[buf][2 * hf + u][lane] = U[2 * hf + u];
          f32x4 cU[4];
#pragma unroll
          for (int m = 0; m < 4; ++m) {
            const float4 c4 = *reinterpret_cast<const float4*>(&SCS[buf][2 * CH + 16 * m + 4 * lg]);
            cU[m][0] = c4.x * U[m][0];
            cU[m][1] = c4.y * U[m][1];
            cU[m][2] = c4.z * U[m][2];
            cU[m][3] = c4.w * U[m][3];
          }
          uint4 ch[2], cl[2];
#pragma unroll
          for (int s = 0; s < 2; ++s) {
            uint2 h0, l0, h1, l1;
            split4_packed(make_float4(cU[2 * s][0], cU[2 * s][1], cU[2 * s][2], cU[2 * s][3]), h0, l0);
            split4_packed(make_float4(cU[2 * s + 1][0], cU[2 * s + 1][1], cU[2 * s + 1][2], cU[2 * s + 1][3]), h1, l1);
            ch[s] = make_uint4(h0.x, h0.y, h1.x, h1.y);
            cl[s] = make_uint4(l0.x, l0.y, l1.x, l1.y);
          }
          const float eg = EGS[buf];
#pragma unroll
          for (int tt = 0; tt < 4; ++tt) {
            const uint4* ktb = kta[tt];
#pragma unroll
            for (int i = 0; i < 4; ++i) S[tt][i] *= eg;
#pragma unroll
            for (int s = 0; s < 2; ++s) {
              S[tt] = mfma_bf16(as_bf16x8(ktb[s]), as_bf16x8(cl[s]), S[tt]);
              S[tt] = mfma_bf16(as_bf16x8(ktb[s]), as_bf16x8(ch[s]), S[tt]);
            }
          }
        };

        load_k(0);
        first_half(0);
        // the last pass also runs first_half for a chunk n that does not exist:
        // it writes buffers of parity n that nobody reads afterwards
        for (int c = 0; c < nchunks; ++c) {
          __syncthreads();                 // B(c)
          second_half(c);
          if constexpr (DUAL) __syncthreads();   // B'(c)
          first_half(c + 1);
        }
        __syncthreads();                   // B(n): the last U is in LDS
      }
      if (ST && (seg.st_only < 0 || n == seg.st_only)) {
        const int64_t su = seg.st_only < 0 ? unit : h;
#pragma unroll
        for (int tt = 0; tt < 4; ++tt)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            ST[(su * D + 64 * hf + 16 * tt + 4 * lg + i) * D + col] = S[tt][i];
      }
    };
    if (w == 0)
      rec_role(std::integral_constant<int, 0>{});
    else
      rec_role(std::integral_constant<int, 1>{});
    return;
  }

  // ================================================================ output waves
  if (nchunks == 0) return;
  const int ow = w - 2;
  const int mt[2] = {ow, 3 - ow};        // token tiles: one with one P k-step, one with two
  // P block (tile m, k-step s) is the turned tile's block (3 - m, 1 - s) read
  // in reversed lane order; slot j holds token 32 s + perm32(lg, 7 - j), kept
  // where it is <= the row 16 m + lr
  uint4 pm[3];                           // masks: (tile 0, s 0), (tile 1, s 0), (tile 1, s 1)
  uint32_t po[3];                        // P block offsets (hi plane; lo is 8 blocks further)
#pragma unroll
  for (int b = 0; b < 3; ++b) {
    const int m = b == 0 ? mt[0] : mt[1], s = b == 2 ? 1 : 0;
    const int row = 16 * m + lr;
    uint32_t mm[4];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const bool lo = 32 * s + perm32(lg, 7 - 2 * d) <= row;
      const bool hi = 32 * s + perm32(lg, 6 - 2 * d) <= row;
      mm[d] = (lo ? 0x0000ffffu : 0u) | (hi ? 0xffff0000u : 0u);
    }
    pm[b] = make_uint4(mm[0], mm[1], mm[2], mm[3]);
    po[b] = static_cast<uint32_t>((2 * (3 - m) + 1 - s) * BLK_BYTES + (63 - lane) * 16);
  }
  // V staging: lane l of instruction i loads token 32 i + l / 2, columns 8 (l % 2) .. +7
  const uint32_t vo0 = static_cast<uint32_t>(((lane >> 1) * vs + slice * 16 + 8 * (lane & 1)) * 2);
  // with the conv: output wave ow stages token 32 ow + l / 2 from its window
  // rows (that token and the three before it), the same 8 columns
  const int ctok = 32 * ow + (lane >> 1);
  const int cch = 2 * nk * D + h * D + slice * 16 + 8 * (lane & 1);   // first channel in conv_dim
  float cwt[4][8], cbs[8];
  uint4 cxr[4];                          // staging: window rows
  float cbeta = 0.0f;                    // staging (wave 2): beta of its token
  if constexpr (CV) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
#pragma unroll
      for (int j = 0; j < 4; ++j) cwt[j][e] = cv.w[(cch + e) * 4 + j];
      cbs[e] = cv.b ? cv.b[cch + e] : 0.0f;
    }
  }
  // T staging: block (m, s) of the strictly lower part, slot j = token
  // 32 s + perm32(lg, j) against row 16 m + lr. Blocks (2, 0) and (3, 0) lie
  // wholly below the diagonal; in the others one half is zero or full and the
  // other follows this pattern (slot j < 4 kept where 4 lg + j < lr).
  uint2 dm;
  {
    uint32_t mm[2];
#pragma unroll
    for (int d = 0; d < 2; ++d)
      mm[d] = (4 * lg + 2 * d < lr ? 0x0000ffffu : 0u) | (4 * lg + 2 * d + 1 < lr ? 0xffff0000u : 0u);
    dm = make_uint2(mm[0], mm[1]);
  }

  // One register set: each group is reloaded for the next chunk right after
  // its last use (Q after Y, P after O, staging loads after staging).
  uint4 qb[2][4];                        // Q (tile mt[u], dk k-step)
  uint4 ph[3], pl[3];                    // P blocks as above, hi | lo
  uint4 sg[12];                          // staging: T blocks (T wave), or scalars, V rows
  uint32_t eg = 0;                       // staging: exp(G_C)
  auto load_q = [&](int cc) {
    const size_t kt = static_cast<size_t>(cbase + cc) * nk + hk;
    const rsrc_t r = make_rsrc(qf + kt * TILE_ELEMS, TILE_ELEMS * 2);
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int s = 0; s < 4; ++s) qb[u][s] = bload16(r, static_cast<uint32_t>((4 * mt[u] + s) * BLK_BYTES) + lo16);
  };
  auto load_p = [&](int cc) {
    const size_t ct = static_cast<size_t>(cbase + cc) * nv + h;
    const rsrc_t r = make_rsrc(xf + ct * TILE_ELEMS, TILE_ELEMS * 2);
#pragma unroll
    for (int b = 0; b < 3; ++b) {
      ph[b] = bload16(r, po[b]);
      pl[b] = bload16(r, po[b] + 8 * BLK_BYTES);
    }
  };
  // Y^T = S^T Q^T of chunk c for both tiles, and a of chunk c
  auto out_y = [&](int c, f32x4 (&Y)[2], float (&a)[2]) {
    const int buf = c & 1;
    uint4 sh[4], sl[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      sh[s] = SBX[buf & PB][0][s][lane];
      sl[s] = SBX[buf & PB][1][s][lane];
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      f32x4 y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        y = mfma_bf16(as_bf16x8(sl[s]), as_bf16x8(qb[u][s]), y);
        y = mfma_bf16(as_bf16x8(sh[s]), as_bf16x8(qb[u][s]), y);
      }
      Y[u] = y;
      a[u] = SCS[buf][16 * mt[u] + lr];
    }
  };
  // O^T = a Y^T + U^T P^T of chunk c (U_c in LDS), stored non-temporally
  // (the output is written once and not read back here)
  const uint32_t oo[2] = {static_cast<uint32_t>(((16 * mt[0] + lr) * nv * D + slice * 16 + 4 * lg) * sizeof(TO)),
                          static_cast<uint32_t>(((16 * mt[1] + lr) * nv * D + slice * 16 + 4 * lg) * sizeof(TO))};
  auto out_o = [&](int c, const f32x4 (&Y)[2], const float (&a)[2]) {
    const int buf = c & 1;
    // U^T as A operand (token k-steps 0, 1), slots reversed to match the turned P blocks
    uint4 uh[2], ul[2];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const f32x4 u0 = UXF[buf][2 * s][lane], u1 = UXF[buf][2 * s + 1][lane];
      uint2 h0, l0, h1, l1;
      split4_packed(make_float4(u0[0], u0[1], u0[2], u0[3]), h0, l0);
      split4_packed(make_float4(u1[0], u1[1], u1[2], u1[3]), h1, l1);
      uh[s] = rev8(make_uint4(h0.x, h0.y, h1.x, h1.y));
      ul[s] = rev8(make_uint4(l0.x, l0.y, l1.x, l1.y));
    }
    f32x4 O[2];
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int i = 0; i < 4; ++i) O[u][i] = a[u] * Y[u][i];
    auto up = [&](f32x4& acc, int b, int s) {
      const bf16x8 bh = as_bf16x8(and4(ph[b], pm[b])), bl = as_bf16x8(and4(pl[b], pm[b]));
      acc = mfma_bf16(as_bf16x8(uh[s]), bl, acc);
      acc = mfma_bf16(as_bf16x8(ul[s]), bh, acc);
      acc = mfma_bf16(as_bf16x8(uh[s]), bh, acc);
    };
    up(O[0], 0, 0);
    up(O[1], 1, 0);
    up(O[1], 2, 1);
    const int64_t t0 = s_begin + static_cast<int64_t>(c) * CH;
    const int L = static_cast<int>(min<int64_t>(CH, s_end - t0));
    // (sized to nothing when the pass stores no output: stores past it are dropped)
    const rsrc_t ro = make_rsrc(o + (t0 * nv + h) * static_cast<int64_t>(D),
                                seg.no_out ? 0u : static_cast<uint32_t>(((L - 1) * nv * D + D) * sizeof(TO)));
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      if constexpr (sizeof(TO) == 4) {
        bstore16_nt(ro, oo[u], make_uint4(__float_as_uint(O[u][0]), __float_as_uint(O[u][1]),
                                       __float_as_uint(O[u][2]), __float_as_uint(O[u][3])));
      } else {
        bstore8_nt(ro, oo[u],
                make_uint2(f32_to_bf16(O[u][0]) | (static_cast<uint32_t>(f32_to_bf16(O[u][1])) << 16),
                           f32_to_bf16(O[u][2]) | (static_cast<uint32_t>(f32_to_bf16(O[u][3])) << 16)));
      }
    }
  };

  // wave 2 stages the masked T blocks, wave 3 the scalars, exp(G_C) and beta v
  auto run = [&](auto tstager) {
    constexpr bool TW = decltype(tstager)::value;
    auto last = [&](int c) { return min(c, nchunks - 1); };
    auto load_stage = [&](int cc) {
      const size_t ct = static_cast<size_t>(cbase + cc) * nv + h;
      if constexpr (TW) {
        const rsrc_t r = make_rsrc(xf + ct * TILE_ELEMS, TILE_ELEMS * 2);
        constexpr int blk[6] = {0, 2, 4, 5, 6, 7};   // 2 m + s
#pragma unroll
        for (int b = 0; b < 6; ++b) {
          sg[b] = bload16(r, blk[b] * BLK_BYTES + lo16);
          sg[6 + b] = bload16(r, (8 + blk[b]) * BLK_BYTES + lo16);
        }
      } else {
        sg[0] = bload16(make_rsrc(scp + ct * 4 * CH, 4 * CH * 4), lo16);
        eg = __builtin_amdgcn_raw_buffer_load_b32(make_rsrc(egc + ct, 4), lo16 & 0u, 0, 0);
        if constexpr (!CV) {
          // V rows past the sequence end read as zeros (resource sized to the
          // valid rows; to nothing in a transition run, whose v is zero)
          const int64_t t0 = s_begin + static_cast<int64_t>(cc) * CH;
          const int L = static_cast<int>(min<int64_t>(CH, s_end - t0));
          const rsrc_t rv = make_rsrc(v + t0 * vs + static_cast<int64_t>(h) * D,
                                      trans ? 0u : static_cast<uint32_t>(((L - 1) * vs + D) * 2));
          sg[1] = bload16(rv, vo0);
          sg[2] = bload16(rv, vo0 + static_cast<uint32_t>(32 * vs * 2));
        }
      }
      if constexpr (CV) {
        // window rows ctok - 3 .. ctok of x; the resource starts 3 rows early
        // when those rows lie in the sequence (every chunk but the sequence's
        // first) and ends at the last valid row, so rows before the sequence
        // (offsets that wrap below zero) and after it read as zeros
        const int64_t t0 = s_begin + static_cast<int64_t>(cc) * CH;
        const int L = static_cast<int>(min<int64_t>(CH, s_end - t0));
        const int pre = static_cast<int>(min<int64_t>(3, t0 - hb));
        const rsrc_t rv = make_rsrc(v + (t0 - pre) * vs + static_cast<int64_t>(h) * D,
                                    static_cast<uint32_t>(((L - 1 + pre) * vs + D) * 2));
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int r = ctok - 3 + j + pre;   // row from the resource start (may be < 0)
          cxr[j] = bload16(rv, static_cast<uint32_t>((static_cast<int64_t>(r) * vs + slice * 16 + 8 * (lane & 1)) * 2));
        }
        if constexpr (TW)
          cbeta = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                                make_rsrc(scp + ct * 4 * CH + 3 * CH, CH * 4),
                                                static_cast<uint32_t>(ctok * 4), 0, 0));
      }
    };
    // stage chunk cs (its loads are in sg) in LDS buffer cs & 1
    auto stage = [&](int cs) {
      const int buf = cs & 1;
      if constexpr (TW) {
        auto lowmask = [&](const uint4& x) { return make_uint4(x.x & dm.x, x.y & dm.y, 0u, 0u); };
        auto highmask = [&](const uint4& x) { return make_uint4(x.x, x.y, x.z & dm.x, x.w & dm.y); };
#pragma unroll
        for (int pl2 = 0; pl2 < 2; ++pl2) {
          const uint4* t = sg + 6 * pl2;
          uint4* d = &TSX[buf][6 * pl2][0];
          d[0 * 64 + lane] = lowmask(t[0]);    // (0, 0)
          d[1 * 64 + lane] = highmask(t[1]);   // (1, 0)
          d[2 * 64 + lane] = t[2];             // (2, 0)
          d[3 * 64 + lane] = lowmask(t[3]);    // (2, 1)
          d[4 * 64 + lane] = t[4];             // (3, 0)
          d[5 * 64 + lane] = highmask(t[5]);   // (3, 1)
        }
      } else {
        *reinterpret_cast<uint4*>(&SCS[buf][4 * lane]) = sg[0];
        if (lane == 0) EGS[buf] = bits_f(eg);
      }
      if constexpr (CV) {
        const int t = ctok;
        const float be = TW ? cbeta : SCS[buf][3 * CH + t];   // wave 3 wrote SCS above
        uint4 win[4] = {cxr[0], cxr[1], cxr[2], cxr[3]};
        if (cs == 0 && s_begin == hb && t < 3 && cv.st) {   // the sequence's history from the conv state
#pragma unroll
          for (int j = 0; j < 3; ++j)
            if (t - 3 + j < 0)
              win[j] = gather8_bf16(cv.st + (static_cast<int64_t>(hn) * cv.conv_dim + cch) * cv.state_len +
                                        cv.state_len + (t - 3 + j),
                                    cv.state_len);
        }
        float y[8];
        conv4_silu8_bf16(win, cwt, cbs, y);
        const int64_t t0 = s_begin + static_cast<int64_t>(last(cs)) * CH;
        // rows past the sequence end stage zeros, and so does a transition run (v = 0)
        const bool pad = t0 + t >= s_end || trans;
        float* bvs = reinterpret_cast<float*>(&BVS[buf][0][0]);
        float* base = bvs + ((t >> 4) * 64 + 16 * ((t & 15) >> 2)) * 4 + (t & 3);
#pragma unroll
        for (int e = 0; e < 8; ++e) base[(8 * (lane & 1) + e) * 4] = pad ? 0.0f : be * y[e];
      } else if constexpr (!TW) {
        float* bvs = reinterpret_cast<float*>(&BVS[buf][0][0]);
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const int t = 32 * i + (lane >> 1);
          const float be = SCS[buf][3 * CH + t];   // written above by this wave
          const uint32_t d[4] = {sg[1 + i].x, sg[1 + i].y, sg[1 + i].z, sg[1 + i].w};
          // slot of (t, column c): tile t / 16, lane c + 16 ((t % 16) / 4), row t % 4
          float* base = bvs + ((t >> 4) * 64 + 16 * ((t & 15) >> 2)) * 4 + (t & 3);
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const uint32_t bits = (e & 1) ? (d[e >> 1] & 0xffff0000u) : (d[e >> 1] << 16);
            base[(8 * (lane & 1) + e) * 4] = be * __uint_as_float(bits);
          }
        }
      }
    };
    load_q(0);
    load_p(0);
    load_stage(0);
    stage(0);
    load_stage(last(1));
    __syncthreads();                     // B(0)
    f32x4 Y[2];
    float a[2];
    out_y(0, Y, a);
    if constexpr (DUAL) __syncthreads();   // B'(0)
    load_q(last(1));
    stage(1);
    load_stage(last(2));
    // the pass with c = nchunks (after B(n)) only stores the last chunk's
    // output; its other work re-reads chunk n-1 data or stale buffers that
    // nobody reads afterwards
    for (int c = 1; c <= nchunks; ++c) {
      __syncthreads();                   // B(c)
      f32x4 Yn[2];
      float an[2];
      out_y(last(c), Yn, an);
      load_q(last(c + 1));
      out_o(c - 1, Y, a);
      if constexpr (DUAL)
        if (c < nchunks) __syncthreads();   // B'(c): the recurrence waves have no B'(n)
      load_p(last(c));
      stage(c + 1);
      load_stage(last(c + 2));
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        Y[u] = Yn[u];
        a[u] = an[u];
      }
    }
  };
  if (w == 2)
    run(std::true_type{});
  else
    run(std::false_type{});
}
// ------------------------------------------------------------------ state: bf16 inputs, two 16-column slices per workgroup
// The wide form, for launches with more 16-column slices than CUs (several
// sequences, or many heads), where a CU's throughput matters more than one
// slice's latency. One workgroup per (sequence, value head, 32
// value columns), four waves:
//   Waves 0 and 1 (recurrence): wave j owns all 128 rows of S for the
//     columns of slice 2 p + j (eight MFMA accumulators) and runs the chunk
//     step of the four-wave form on them alone, with no partial products to
//     swap. X is still formed as (K S over dk rows 0-63) + (K S over rows
//     64-127), the sum the four-wave form's two halves exchange, so every
//     result equals that form's bit for bit.
//   Waves 2 and 3 (output, one chunk behind): the four-wave form's output
//     work for both slices (wave 2 token tiles 0 and 3, wave 3 tiles 1 and
//     2); the Q and P blocks of a tile serve both slices.
// Staging: wave 2 the masked T blocks, wave 3 the per-token scalars and
// exp(G_C), both one chunk ahead; wave 2 stages beta v for slice 2 p, wave 3
// for slice 2 p + 1, each for all 64 tokens of a chunk (beta from memory).
// With the conv (CV) the workgroup has eight waves: waves 4-7 stage beta v
// instead, each convolving one token per lane for one slice and half of the
// chunk (waves 4, 5: slice 2 p, tokens 0-31 and 32-63; waves 6, 7: slice
// 2 p + 1), so the output waves, which set the pace when they convolve, keep
// only their products and the T and scalar staging.
// One barrier per chunk; every LDS buffer shared between waves is
// double-buffered by chunk parity as in the four-wave form.
__device__ __forceinline__ void wide_unit_pair(int b, int n_units, int r, int& unit_slot, int& pair) {
  const int j = b >> 3;          // this workgroup's position on its XCD
  if (n_units % (8 * r) == 0) {
    pair = j & 3;
    const int k = j >> 2;        // unit position on the XCD
    unit_slot = ((k / r) * 8 + (b & 7)) * r + k % r;
  } else if (n_units % 8 == 0) {
    pair = j & 3;
    unit_slot = ((j >> 2) << 3) + (b & 7);
  } else {
    const int bid = xcd_swizzle(b, n_units * 4);
    pair = bid & 3;
    unit_slot = bid >> 2;
  }
}

// EPI (with CV only): the gated RMSNorm epilogue described at EpiIn; the
// output waves keep o in an LDS ring and publish row partial sums, and the conv
// waves normalize each chunk EPI_LAG chunks later and store y in place of o.
// One more barrier follows the last chunk.
template <typename TO, bool CV, bool EPI>
__global__ void __launch_bounds__(CV ? 512 : 256) chunk_state_wide_kernel(
    const uint16_t* __restrict__ v, int64_t vs, const int32_t* __restrict__ cu, int n_seqs, int64_t T, int nk,
    int nv, const int32_t* __restrict__ chunk_off, const uint16_t* __restrict__ xf, const float* __restrict__ scp,
    const float* __restrict__ egc, const uint16_t* __restrict__ kf, const uint16_t* __restrict__ qf,
    const int32_t* __restrict__ order, const float* __restrict__ S0, float* __restrict__ ST, TO* __restrict__ o,
    ConvIn cv, EpiIn ep) {
  static_assert(!EPI || CV, "the epilogue runs on the conv waves");
  __shared__ uint4 SBX[2][2][2][4][64];  // S as B operand: [slice][parity][hi | lo][dk k-step][lane]
  __shared__ f32x4 UXF[2][2][4][64];     // U: [slice][parity][token tile][lane]
  __shared__ f32x4 BVS[2][2][4][64];     // beta * v: [slice][parity][token tile][lane]
  __shared__ uint4 TSX[2][12][64];       // masked T blocks: [parity][hi (6) | lo (6)][lane]
  // each recurrence wave's 16 K blocks of the current chunk, read back
  // transposed (lane l at byte 16 l + 64 (l / 16) of its block)
  __shared__ __attribute__((aligned(16))) unsigned char KLX[2][16][KL_BLK];
  __shared__ __attribute__((aligned(16))) float SCS[2][4 * CH];   // planes a | b | c | beta
  __shared__ float EGS[2];               // exp(G_C)
  // epilogue: o of the last EPI_LAG + 1 chunks, [chunk % 3][token][the pair's 32 columns]
  // (rows padded to 36 floats: a 32-float pitch put the 16 rows an output
  // wave writes at once on the same banks)
  __shared__ __attribute__((aligned(16))) float ORX[EPI ? EPI_LAG + 1 : 1][EPI ? CH : 1][EPI ? 36 : 4];

  int slot, pair;
  wide_unit_pair(blockIdx.x, gridDim.x / 4, nv / nk, slot, pair);
  const int n = cu ? order[slot / nv] : 0, h = slot % nv;
  const int unit = n * nv + h;
  const int hk = h / (nv / nk);
  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 15, lg = lane >> 4;
  const uint32_t lo16 = static_cast<uint32_t>(lane * 16);

  int64_t s_begin, s_end;
  seq_bounds(cu, n, T, s_begin, s_end);
  int cbase, nchunks;
  chunk_span(chunk_off, cu, T, n, cbase, nchunks);

  if (w < 2) {
    // ================================================================ recurrence waves
    const int col = (2 * pair + w) * 16 + lr;
    f32x4 S[8];                            // rows 16 tt + 4 lg + i, column col
#pragma unroll
    for (int tt = 0; tt < 8; ++tt)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        S[tt][i] = S0 ? S0[(static_cast<int64_t>(unit) * D + 16 * tt + 4 * lg + i) * D + col] : 0.0f;

    if (nchunks > 0) {
      unsigned char (*kl)[KL_BLK] = KLX[w];
      uint4 kb[4][4];                      // K (token tile m, dk k-step ks)
      auto load_k = [&](int cc) {
        const size_t kt = static_cast<size_t>(cbase + cc) * nk + hk;
        const rsrc_t r = make_rsrc(kf + kt * TILE_ELEMS, TILE_ELEMS * 2);
#pragma unroll
        for (int m = 0; m < 4; ++m)
#pragma unroll
          for (int ks = 0; ks < 4; ++ks) kb[m][ks] = bload16(r, (4 * m + ks) * BLK_BYTES + lo16);
      };
      f32x4 X0[4], X1[4];                  // K S over dk rows 0-63 and 64-127
      // S_c as B operand (published for the output waves) and X_c
      auto first_half = [&](int c) {
        const int buf = c & 1;
        uint4 sh[4], sl[4];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          uint2 h0, l0, h1, l1;
          split4_packed(make_float4(S[2 * ks][0], S[2 * ks][1], S[2 * ks][2], S[2 * ks][3]), h0, l0);
          split4_packed(make_float4(S[2 * ks + 1][0], S[2 * ks + 1][1], S[2 * ks + 1][2], S[2 * ks + 1][3]), h1, l1);
          sh[ks] = make_uint4(h0.x, h0.y, h1.x, h1.y);
          sl[ks] = make_uint4(l0.x, l0.y, l1.x, l1.y);
          SBX[w][buf][0][ks][lane] = sh[ks];
          SBX[w][buf][1][ks][lane] = sl[ks];
        }
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          f32x4 x0 = {0.f, 0.f, 0.f, 0.f}, x1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kk = 0; kk < 2; ++kk) {
            x0 = mfma_bf16(as_bf16x8(kb[m][kk]), as_bf16x8(sl[kk]), x0);
            x0 = mfma_bf16(as_bf16x8(kb[m][kk]), as_bf16x8(sh[kk]), x0);
          }
#pragma unroll
          for (int kk = 2; kk < 4; ++kk) {
            x1 = mfma_bf16(as_bf16x8(kb[m][kk]), as_bf16x8(sl[kk]), x1);
            x1 = mfma_bf16(as_bf16x8(kb[m][kk]), as_bf16x8(sh[kk]), x1);
          }
          X0[m] = x0;
          X1[m] = x1;
#pragma unroll
          for (int ks = 0; ks < 4; ++ks)
            *reinterpret_cast<uint4*>(&kl[4 * m + ks][kl_lane(lane)]) = kb[m][ks];
        }
        load_k(min(c + 1, nchunks - 1));
      };
      // the rest of chunk c: R, U, c U, and the update of S
      auto second_half = [&](int c) {
        const int buf = c & 1;
        // K^T blocks (dk tile tt, token k-step s), read transposed as in the
        // four-wave form: block (token tile 2 s + h, dk k-step tt / 2)
        uint4 kta[8][2];
        {
          const int kll = kl_lane(16 * (lr & 3) + 4 * lg + (lr >> 2));
#pragma unroll
          for (int tt = 0; tt < 8; ++tt)
#pragma unroll
            for (int s = 0; s < 2; ++s) {
              const uint2 y0 = lds_tr16(&kl[4 * (2 * s) + tt / 2][kll + 8 * (tt & 1)]);
              const uint2 y1 = lds_tr16(&kl[4 * (2 * s + 1) + tt / 2][kll + 8 * (tt & 1)]);
              kta[tt][s] = make_uint4(y0.x, y0.y, y1.x, y1.y);
            }
        }
        f32x4 R[4];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const f32x4 bv = BVS[w][buf][m][lane];
          const float4 bb = *reinterpret_cast<const float4*>(&SCS[buf][CH + 16 * m + 4 * lg]);
          const float bbv[4] = {bb.x, bb.y, bb.z, bb.w};
#pragma unroll
          for (int i = 0; i < 4; ++i) R[m][i] = bv[i] - bbv[i] * (X0[m][i] + X1[m][i]);
        }
        uint4 rh[2], rl[2];                // R as B operand, token k-steps 0, 1
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          uint2 h0, l0, h1, l1;
          split4_packed(make_float4(R[2 * s][0], R[2 * s][1], R[2 * s][2], R[2 * s][3]), h0, l0);
          split4_packed(make_float4(R[2 * s + 1][0], R[2 * s + 1][1], R[2 * s + 1][2], R[2 * s + 1][3]), h1, l1);
          rh[s] = make_uint4(h0.x, h0.y, h1.x, h1.y);
          rl[s] = make_uint4(l0.x, l0.y, l1.x, l1.y);
        }
        // T blocks (m, s): (0,0) (1,0) (2,0) (2,1) (3,0) (3,1), masked, hi | lo
        uint4 mh[6], ml[6];
#pragma unroll
        for (int b = 0; b < 6; ++b) {
          mh[b] = TSX[buf][b][lane];
          ml[b] = TSX[buf][6 + b][lane];
        }
        // U = R + T_strict R
        f32x4 U[4];
        auto tr = [&](f32x4& acc, int b, int s) {
          acc = mfma_bf16(as_bf16x8(ml[b]), as_bf16x8(rh[s]), acc);
          acc = mfma_bf16(as_bf16x8(mh[b]), as_bf16x8(rl[s]), acc);
          acc = mfma_bf16(as_bf16x8(mh[b]), as_bf16x8(rh[s]), acc);
        };
#pragma unroll
        for (int m = 0; m < 4; ++m) U[m] = R[m];
        tr(U[0], 0, 0);
        tr(U[1], 1, 0);
        tr(U[2], 2, 0);
        tr(U[3], 4, 0);
        tr(U[2], 3, 1);
        tr(U[3], 5, 1);
        // U for the output waves; c U as B operand
#pragma unroll
        for (int m = 0; m < 4; ++m) UXF[w][buf][m][lane] = U[m];
        f32x4 cU[4];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const float4 c4 = *reinterpret_cast<const float4*>(&SCS[buf][2 * CH + 16 * m + 4 * lg]);
          cU[m][0] = c4.x * U[m][0];
          cU[m][1] = c4.y * U[m][1];
          cU[m][2] = c4.z * U[m][2];
          cU[m][3] = c4.w * U[m][3];
        }
        uint4 ch[2], cl[2];
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          uint2 h0, l0, h1, l1;
          split4_packed(make_float4(cU[2 * s][0], cU[2 * s][1], cU[2 * s][2], cU[2 * s][3]), h0, l0);
          split4_packed(make_float4(cU[2 * s + 1][0], cU[2 * s + 1][1], cU[2 * s + 1][2], cU[2 * s + 1][3]), h1, l1);
          ch[s] = make_uint4(h0.x, h0.y, h1.x, h1.y);
          cl[s] = make_uint4(l0.x, l0.y, l1.x, l1.y);
        }
        const float eg = EGS[buf];
#pragma unroll
        for (int tt = 0; tt < 8; ++tt) {
          const uint4* ktb = kta[tt];
#pragma unroll
          for (int i = 0; i < 4; ++i) S[tt][i] *= eg;
#pragma unroll
          for (int s = 0; s < 2; ++s) {
            S[tt] = mfma_bf16(as_bf16x8(ktb[s]), as_bf16x8(cl[s]), S[tt]);
            S[tt] = mfma_bf16(as_bf16x8(ktb[s]), as_bf16x8(ch[s]), S[tt]);
          }
        }
      };

      load_k(0);
      first_half(0);
      // the last pass also runs first_half for a chunk n that does not exist:
      // it writes buffers of parity n that nobody reads afterwards
      for (int c = 0; c < nchunks; ++c) {
        __syncthreads();                   // B(c)
        second_half(c);
        first_half(c + 1);
      }
      __syncthreads();                     // B(n): the last U is in LDS
    }
    if (ST) {
#pragma unroll
      for (int tt = 0; tt < 8; ++tt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          ST[(static_cast<int64_t>(unit) * D + 16 * tt + 4 * lg + i) * D + col] = S[tt][i];
    }
    if constexpr (EPI)
      if (nchunks > 0) __syncthreads();   // B(n + 1): the conv waves normalize the last chunks
    return;
  }

  auto last = [&](int c) { return min(c, nchunks - 1); };
  if constexpr (CV) {
    if (w >= 4) {
      // ============================================================== conv waves
      if (nchunks == 0) return;
      const int j = (w - 4) >> 1;          // slice 2 pair + j
      const int t = 32 * ((w - 4) & 1) + (lane >> 1);   // this lane's token in a chunk
      const int vcol = (2 * pair + j) * 16 + 8 * (lane & 1);
      const int cch = 2 * nk * D + h * D + vcol;   // first conv channel of those columns
      float cwt[4][8], cbs[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) cwt[q4][e] = cv.w[(cch + e) * 4 + q4];
        cbs[e] = cv.b ? cv.b[cch + e] : 0.0f;
      }
      uint4 cxr[4];                        // window rows t - 3 .. t
      float sb = 0.0f;                     // beta of the token
      // the resource starts 3 rows early when those rows lie in the sequence
      // (every chunk but the first) and ends at the last valid row, so rows
      // before the sequence (offsets that wrap below zero) and after it read
      // as zeros
      auto load_conv = [&](int cc) {
        const size_t ct = static_cast<size_t>(cbase + cc) * nv + h;
        sb = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                           make_rsrc(scp + ct * 4 * CH + 3 * CH, CH * 4),
                                           static_cast<uint32_t>(t * 4), 0, 0));
        const int64_t t0 = s_begin + static_cast<int64_t>(cc) * CH;
        const int L = static_cast<int>(min<int64_t>(CH, s_end - t0));
        const int pre = cc > 0 ? 3 : 0;
        const rsrc_t rv = make_rsrc(v + (t0 - pre) * vs + static_cast<int64_t>(h) * D,
                                    static_cast<uint32_t>(((L - 1 + pre) * vs + D) * 2));
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int r = t - 3 + q4 + pre;   // row from the resource start (may be < 0)
          cxr[q4] = bload16(rv, static_cast<uint32_t>((static_cast<int64_t>(r) * vs + vcol) * 2));
        }
      };
      // beta v of chunk cs (its loads are in cxr, sb) into LDS buffer cs & 1
      auto stage_conv = [&](int cs) {
        const int buf = cs & 1;
        uint4 win[4] = {cxr[0], cxr[1], cxr[2], cxr[3]};
        if (cs == 0 && t < 3 && cv.st) {   // the sequence's history from the conv state
#pragma unroll
          for (int q4 = 0; q4 < 3; ++q4)
            if (t - 3 + q4 < 0)
              win[q4] = gather8_bf16(cv.st + (static_cast<int64_t>(n) * cv.conv_dim + cch) * cv.state_len +
                                         cv.state_len + (t - 3 + q4),
                                     cv.state_len);
        }
        float y[8];
        conv4_silu8_bf16(win, cwt, cbs, y);
        const int64_t t0 = s_begin + static_cast<int64_t>(last(cs)) * CH;
        const bool pad = t0 + t >= s_end;   // rows past the sequence end stage zeros
        float* bvs = reinterpret_cast<float*>(&BVS[j][buf][0][0]);
        // slot of (t, column c): tile t / 16, lane c + 16 ((t % 16) / 4), row t % 4
        float* base = bvs + ((t >> 4) * 64 + 16 * ((t & 15) >> 2)) * 4 + (t & 3);
#pragma unroll
        for (int e = 0; e < 8; ++e) base[(8 * (lane & 1) + e) * 4] = pad ? 0.0f : sb * y[e];
      };
      // epilogue: this wave normalizes token tile w - 4 of a chunk; lane l
      // takes row 16 (w - 4) + l / 4 and the pair's columns 8 (l % 4) .. +7,
      // and polls pair l % 4's partial sum of that row
      const int etok = 16 * (w - 4) + (lane >> 2), eq = lane & 3;
      const int ecol = 32 * pair + 8 * eq;   // first column in the head
      float ew[8];
      if constexpr (EPI) {
#pragma unroll
        for (int e = 0; e < 8; ++e) ew[e] = ep.w[ecol + e];
      }
      // the partial-sum word and z of chunk cn are fetched at the start of
      // period cn + 2, right after its barrier, into register set cn & 1, and
      // used at the end of period cn + 3: the conv loads issued after them in
      // period cn + 2 are waited for at the start of period cn + 3, so by then
      // they have had a whole period and nothing waits on them inside one.
      // Every period issues the same loads (the chunk index clamped into the
      // sequence), so the compiler's waits stay the same from period to
      // period; the loop runs two periods per pass so that each set index is
      // a constant (a run-time select would wait for both sets).
      unsigned long long word[2] = {0ull, 0ull};
      uint4 zr[2] = {make_uint4(0u, 0u, 0u, 0u), make_uint4(0u, 0u, 0u, 0u)};
      auto ring_word = [&](int cn) {
        return ep.ring + ((static_cast<size_t>(unit) * EPI_RING + cn % EPI_RING) * 4 + eq) * CH + etok;
      };
      auto epi_fetch = [&](int cn, auto set) {
        constexpr int SET = decltype(set)::value;
        const int cc = max(0, min(cn, nchunks - 1));
        const unsigned long long wv = __hip_atomic_load(ring_word(cc), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const int64_t t0 = s_begin + static_cast<int64_t>(cc) * CH;
        const int L = static_cast<int>(min<int64_t>(CH, s_end - t0));
        const rsrc_t rz = make_rsrc(ep.z + (t0 * nv + h) * static_cast<int64_t>(D),
                                    static_cast<uint32_t>(((L - 1) * nv * D + D) * 2));
        word[SET] = wv;
        zr[SET] = bload16(rz, static_cast<uint32_t>((etok * nv * D + ecol) * 2));
      };
      auto normalize = [&](int cn, auto set) {
        constexpr int SET = decltype(set)::value;
        const float4 o0 = *reinterpret_cast<const float4*>(&ORX[cn % (EPI_LAG + 1)][etok][8 * eq]);
        const float4 o1 = *reinterpret_cast<const float4*>(&ORX[cn % (EPI_LAG + 1)][etok][8 * eq + 4]);
        const float ov[8] = {o0.x, o0.y, o0.z, o0.w, o1.x, o1.y, o1.z, o1.w};
        unsigned long long* wp = ring_word(cn);
        const uint32_t want = static_cast<uint32_t>(cn) + 1u;
        unsigned long long wd = word[SET];
        const uint4 zc = zr[SET];
        bool ok = static_cast<uint32_t>(wd >> 32) == want;
        for (int it = 0; it < EPI_SPIN && !__all(ok); ++it) {
          __builtin_amdgcn_s_sleep(1);
          if (!ok) {
            wd = __hip_atomic_load(wp, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            ok = static_cast<uint32_t>(wd >> 32) == want;
          }
        }
        // rows' sums in a fixed order, the same in all four lanes of a row
        float ss = ok ? __uint_as_float(static_cast<uint32_t>(wd)) : __builtin_nanf("");
        ss += __shfl_xor(ss, 1, 64);
        ss += __shfl_xor(ss, 2, 64);
        const float inv = 1.0f / sqrtf(ss / static_cast<float>(D) + ep.eps);
        const int64_t t0 = s_begin + static_cast<int64_t>(cn) * CH;
        const int L = static_cast<int>(min<int64_t>(CH, s_end - t0));
        const uint32_t zw[4] = {zc.x, zc.y, zc.z, zc.w};
        float yv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float zv = __uint_as_float((e & 1) ? (zw[e >> 1] & 0xffff0000u) : (zw[e >> 1] << 16));
          yv[e] = ov[e] * inv * (1.0f + ew[e]) * siluf_(zv);
        }
        const rsrc_t ro = make_rsrc(o + (t0 * nv + h) * static_cast<int64_t>(D),
                                    static_cast<uint32_t>(((L - 1) * nv * D + D) * sizeof(TO)));
        const uint32_t oo = static_cast<uint32_t>((etok * nv * D + ecol) * sizeof(TO));
        if constexpr (sizeof(TO) == 4) {
          bstore16_nt(ro, oo, make_uint4(__float_as_uint(yv[0]), __float_as_uint(yv[1]), __float_as_uint(yv[2]),
                                         __float_as_uint(yv[3])));
          bstore16_nt(ro, oo + 16, make_uint4(__float_as_uint(yv[4]), __float_as_uint(yv[5]),
                                              __float_as_uint(yv[6]), __float_as_uint(yv[7])));
        } else {
          bstore16_nt(ro, oo, pack8_bf16(yv));
        }
      };
      // the same staging order as the output waves' (chunk c + 1 between B(c)
      // and B(c + 1)); with the epilogue, chunk c - 1 - EPI_LAG is normalized
      // in step c and the last ones after one more barrier
      load_conv(0);
      stage_conv(0);
      load_conv(last(1));
      __syncthreads();                     // B(0)
      stage_conv(1);
      load_conv(last(2));
      using S0_ = std::integral_constant<int, 0>;
      using S1_ = std::integral_constant<int, 1>;
      // period c; F = (c - EPI_LAG) & 1 = c & 1, the set fetched into
      auto period = [&](int c, auto f) {
        constexpr int F = decltype(f)::value;
        __syncthreads();                   // B(c)
        if constexpr (EPI) {
          epi_fetch(c - EPI_LAG, std::integral_constant<int, F>{});
          __builtin_amdgcn_sched_barrier(0);
        }
        stage_conv(c + 1);
        load_conv(last(c + 2));
        if constexpr (EPI)
          if (c - 1 - EPI_LAG >= 0) normalize(c - 1 - EPI_LAG, std::integral_constant<int, 1 - F>{});
      };
      for (int c = 1; c <= nchunks; c += 2) {
        period(c, S1_{});
        if (c + 1 <= nchunks) period(c + 1, S0_{});
      }
      if constexpr (EPI) {
        __syncthreads();                   // B(n + 1)
        // chunk n - 2 was fetched in period n (when n >= 2); fetch the rest
        for (int cn = max(0, nchunks - EPI_LAG); cn < nchunks; ++cn) {
          if (cn == nchunks - EPI_LAG) continue;
          if (cn & 1)
            epi_fetch(cn, S1_{});
          else
            epi_fetch(cn, S0_{});
        }
        for (int cn = max(0, nchunks - EPI_LAG); cn < nchunks; ++cn) {
          if (cn & 1)
            normalize(cn, S1_{});
          else
            normalize(cn, S0_{});
        }
      }
      return;
    }
  }

  // ================================================================ output waves
  if (nchunks == 0) return;
  const int ow = w - 2;
  const int mt[2] = {ow, 3 - ow};        // token tiles: one with one P k-step, one with two
  // P blocks and their masks as in the four-wave form
  uint4 pm[3];
  uint32_t po[3];
#pragma unroll
  for (int b = 0; b < 3; ++b) {
    const int m = b == 0 ? mt[0] : mt[1], s = b == 2 ? 1 : 0;
    const int row = 16 * m + lr;
    uint32_t mm[4];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const bool lo = 32 * s + perm32(lg, 7 - 2 * d) <= row;
      const bool hi = 32 * s + perm32(lg, 6 - 2 * d) <= row;
      mm[d] = (lo ? 0x0000ffffu : 0u) | (hi ? 0xffff0000u : 0u);
    }
    pm[b] = make_uint4(mm[0], mm[1], mm[2], mm[3]);
    po[b] = static_cast<uint32_t>((2 * (3 - m) + 1 - s) * BLK_BYTES + (63 - lane) * 16);
  }
  // beta v staging for slice 2 p + ow (without the conv): lane l takes tokens
  // l / 2 and 32 + l / 2, columns 8 (l % 2) .. +7 of the head (offsets from
  // the head's first value column)
  const int vcol = (2 * pair + ow) * 16 + 8 * (lane & 1);
  const uint32_t vo0 = static_cast<uint32_t>(((lane >> 1) * vs + vcol) * 2);
  uint4 svr[2];                          // staging: value rows of both tokens
  float sbeta[2];                        // staging: beta of both tokens
  uint2 dm;                              // T staging masks as in the four-wave form
  {
    uint32_t mm[2];
#pragma unroll
    for (int d = 0; d < 2; ++d)
      mm[d] = (4 * lg + 2 * d < lr ? 0x0000ffffu : 0u) | (4 * lg + 2 * d + 1 < lr ? 0xffff0000u : 0u);
    dm = make_uint2(mm[0], mm[1]);
  }

  uint4 qb[2][4];                        // Q (tile mt[u], dk k-step)
  uint4 ph[3], pl[3];                    // P blocks, hi | lo
  uint4 sg[12];                          // staging: T blocks (wave 2), or scalars (wave 3)
  uint32_t eg = 0;                       // staging: exp(G_C)
  auto load_q = [&](int cc) {
    const size_t kt = static_cast<size_t>(cbase + cc) * nk + hk;
    const rsrc_t r = make_rsrc(qf + kt * TILE_ELEMS, TILE_ELEMS * 2);
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int s = 0; s < 4; ++s) qb[u][s] = bload16(r, static_cast<uint32_t>((4 * mt[u] + s) * BLK_BYTES) + lo16);
  };
  auto load_p = [&](int cc) {
    const size_t ct = static_cast<size_t>(cbase + cc) * nv + h;
    const rsrc_t r = make_rsrc(xf + ct * TILE_ELEMS, TILE_ELEMS * 2);
#pragma unroll
    for (int b = 0; b < 3; ++b) {
      ph[b] = bload16(r, po[b]);
      pl[b] = bload16(r, po[b] + 8 * BLK_BYTES);
    }
  };
  // Y^T = S^T Q^T of chunk c for both tiles of both slices, and a of chunk c
  auto out_y = [&](int c, f32x4 (&Y)[2][2], float (&a)[2]) {
    const int buf = c & 1;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      uint4 sh[4], sl[4];
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        sh[s] = SBX[j][buf][0][s][lane];
        sl[s] = SBX[j][buf][1][s][lane];
      }
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        f32x4 y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          y = mfma_bf16(as_bf16x8(sl[s]), as_bf16x8(qb[u][s]), y);
          y = mfma_bf16(as_bf16x8(sh[s]), as_bf16x8(qb[u][s]), y);
        }
        Y[j][u] = y;
      }
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) a[u] = SCS[buf][16 * mt[u] + lr];
  };
  // O^T = a Y^T + U^T P^T of chunk c for both slices, stored non-temporally
  // (with the epilogue: kept in the LDS ring, and the rows' partial sums of
  // squares over the pair's 32 columns published)
  auto out_o = [&](int c, const f32x4 (&Y)[2][2], const float (&a)[2]) {
    const int buf = c & 1;
    const int64_t t0 = s_begin + static_cast<int64_t>(c) * CH;
    const int L = static_cast<int>(min<int64_t>(CH, s_end - t0));
    const rsrc_t ro = make_rsrc(o + (t0 * nv + h) * static_cast<int64_t>(D),
                                static_cast<uint32_t>(((L - 1) * nv * D + D) * sizeof(TO)));
    float ssp[2] = {0.0f, 0.0f};
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      // U^T as A operand (token k-steps 0, 1), slots reversed to match the turned P blocks
      uint4 uh[2], ul[2];
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const f32x4 u0 = UXF[j][buf][2 * s][lane], u1 = UXF[j][buf][2 * s + 1][lane];
        uint2 h0, l0, h1, l1;
        split4_packed(make_float4(u0[0], u0[1], u0[2], u0[3]), h0, l0);
        split4_packed(make_float4(u1[0], u1[1], u1[2], u1[3]), h1, l1);
        uh[s] = rev8(make_uint4(h0.x, h0.y, h1.x, h1.y));
        ul[s] = rev8(make_uint4(l0.x, l0.y, l1.x, l1.y));
      }
      f32x4 O[2];
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int i = 0; i < 4; ++i) O[u][i] = a[u] * Y[j][u][i];
      auto up = [&](f32x4& acc, int b, int s) {
        const bf16x8 bh = as_bf16x8(and4(ph[b], pm[b])), bl = as_bf16x8(and4(pl[b], pm[b]));
        acc = mfma_bf16(as_bf16x8(uh[s]), bl, acc);
        acc = mfma_bf16(as_bf16x8(ul[s]), bh, acc);
        acc = mfma_bf16(as_bf16x8(uh[s]), bh, acc);
      };
      up(O[0], 0, 0);
      up(O[1], 1, 0);
      up(O[1], 2, 1);
      const int ocol = (2 * pair + j) * 16 + 4 * lg;
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        if constexpr (EPI) {
          *reinterpret_cast<float4*>(&ORX[c % (EPI_LAG + 1)][16 * mt[u] + lr][16 * j + 4 * lg]) =
              make_float4(O[u][0], O[u][1], O[u][2], O[u][3]);
#pragma unroll
          for (int i = 0; i < 4; ++i) ssp[u] = fmaf(O[u][i], O[u][i], ssp[u]);
        } else {
          const uint32_t oo = static_cast<uint32_t>(((16 * mt[u] + lr) * nv * D + ocol) * sizeof(TO));
          if constexpr (sizeof(TO) == 4) {
            bstore16_nt(ro, oo, make_uint4(__float_as_uint(O[u][0]), __float_as_uint(O[u][1]),
                                           __float_as_uint(O[u][2]), __float_as_uint(O[u][3])));
          } else {
            bstore8_nt(ro, oo,
                       make_uint2(f32_to_bf16(O[u][0]) | (static_cast<uint32_t>(f32_to_bf16(O[u][1])) << 16),
                                  f32_to_bf16(O[u][2]) | (static_cast<uint32_t>(f32_to_bf16(O[u][3])) << 16)));
          }
        }
      }
    }
    if constexpr (EPI) {
      // a row's 8 values per lane, then its 4 lanes (lanes lr + 16 lg)
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        ssp[u] += __shfl_xor(ssp[u], 16, 64);
        ssp[u] += __shfl_xor(ssp[u], 32, 64);
      }
      if (lg == 0) {
        const unsigned long long tag = static_cast<unsigned long long>(static_cast<uint32_t>(c) + 1u) << 32;
#pragma unroll
        for (int u = 0; u < 2; ++u)
          __hip_atomic_store(ep.ring + ((static_cast<size_t>(unit) * EPI_RING + c % EPI_RING) * 4 + pair) * CH +
                                 16 * mt[u] + lr,
                             tag | __float_as_uint(ssp[u]), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  };

  // wave 2 stages the masked T blocks, wave 3 the scalars and exp(G_C); each
  // stages beta v for its slice
  auto run = [&](auto tstager) {
    constexpr bool TW = decltype(tstager)::value;
    auto load_stage = [&](int cc) {
      const size_t ct = static_cast<size_t>(cbase + cc) * nv + h;
      if constexpr (TW) {
        const rsrc_t r = make_rsrc(xf + ct * TILE_ELEMS, TILE_ELEMS * 2);
        constexpr int blk[6] = {0, 2, 4, 5, 6, 7};   // 2 m + s
#pragma unroll
        for (int b = 0; b < 6; ++b) {
          sg[b] = bload16(r, blk[b] * BLK_BYTES + lo16);
          sg[6 + b] = bload16(r, (8 + blk[b]) * BLK_BYTES + lo16);
        }
      } else {
        sg[0] = bload16(make_rsrc(scp + ct * 4 * CH, 4 * CH * 4), lo16);
        eg = __builtin_amdgcn_raw_buffer_load_b32(make_rsrc(egc + ct, 4), lo16 & 0u, 0, 0);
      }
      if constexpr (!CV) {
        const rsrc_t rb = make_rsrc(scp + ct * 4 * CH + 3 * CH, CH * 4);
#pragma unroll
        for (int i = 0; i < 2; ++i)
          sbeta[i] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                                   rb, static_cast<uint32_t>((32 * i + (lane >> 1)) * 4), 0, 0));
        // V rows past the sequence end read as zeros (resource sized to the valid rows)
        const int64_t t0 = s_begin + static_cast<int64_t>(cc) * CH;
        const int L = static_cast<int>(min<int64_t>(CH, s_end - t0));
        const rsrc_t rv =
            make_rsrc(v + t0 * vs + static_cast<int64_t>(h) * D, static_cast<uint32_t>(((L - 1) * vs + D) * 2));
        svr[0] = bload16(rv, vo0);
        svr[1] = bload16(rv, vo0 + static_cast<uint32_t>(32 * vs * 2));
      }
    };
    // stage chunk cs (its loads are in sg, svr, sbeta) in LDS buffer cs & 1
    auto stage = [&](int cs) {
      const int buf = cs & 1;
      if constexpr (TW) {
        auto lowmask = [&](const uint4& x) { return make_uint4(x.x & dm.x, x.y & dm.y, 0u, 0u); };
        auto highmask = [&](const uint4& x) { return make_uint4(x.x, x.y, x.z & dm.x, x.w & dm.y); };
#pragma unroll
        for (int pl2 = 0; pl2 < 2; ++pl2) {
          const uint4* t = sg + 6 * pl2;
          uint4* d = &TSX[buf][6 * pl2][0];
          d[0 * 64 + lane] = lowmask(t[0]);    // (0, 0)
          d[1 * 64 + lane] = highmask(t[1]);   // (1, 0)
          d[2 * 64 + lane] = t[2];             // (2, 0)
          d[3 * 64 + lane] = lowmask(t[3]);    // (2, 1)
          d[4 * 64 + lane] = t[4];             // (3, 0)
          d[5 * 64 + lane] = highmask(t[5]);   // (3, 1)
        }
      } else {
        *reinterpret_cast<uint4*>(&SCS[buf][4 * lane]) = sg[0];
        if (lane == 0) EGS[buf] = bits_f(eg);
      }
      if constexpr (!CV) {
        float* bvs = reinterpret_cast<float*>(&BVS[ow][buf][0][0]);
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const int t = 32 * i + (lane >> 1);
          // slot of (t, column c): tile t / 16, lane c + 16 ((t % 16) / 4), row t % 4
          float* base = bvs + ((t >> 4) * 64 + 16 * ((t & 15) >> 2)) * 4 + (t & 3);
          const uint32_t d[4] = {svr[i].x, svr[i].y, svr[i].z, svr[i].w};
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const uint32_t bits = (e & 1) ? (d[e >> 1] & 0xffff0000u) : (d[e >> 1] << 16);
            base[(8 * (lane & 1) + e) * 4] = sbeta[i] * __uint_as_float(bits);
          }
        }
      }
    };
    load_q(0);
    load_p(0);
    load_stage(0);
    stage(0);
    load_stage(last(1));
    __syncthreads();                     // B(0)
    f32x4 Y[2][2];
    float a[2];
    out_y(0, Y, a);
    load_q(last(1));
    stage(1);
    load_stage(last(2));
    // the pass with c = nchunks (after B(n)) only stores the last chunk's
    // output; its other work re-reads chunk n-1 data or stale buffers that
    // nobody reads afterwards
    for (int c = 1; c <= nchunks; ++c) {
      __syncthreads();                   // B(c)
      f32x4 Yn[2][2];
      float an[2];
      out_y(last(c), Yn, an);
      load_q(last(c + 1));
      out_o(c - 1, Y, a);
      load_p(last(c));
      stage(c + 1);
      load_stage(last(c + 2));
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int u = 0; u < 2; ++u) Y[j][u] = Yn[j][u];
#pragma unroll
      for (int u = 0; u < 2; ++u) a[u] = an[u];
    }
    if constexpr (EPI) __syncthreads();   // B(n + 1)
  };
  if (w == 2)
    run(std::true_type{});
  else
    run(std::false_type{});
}

// ------------------------------------------------------------------ segment-parallel prefill: incoming states
// A segment's final state is affine in its incoming state, S_out = M S_in + D,
// with D the final state from a zero start and M the one from the identity
// with v = 0 (both from the first pass, D_p = seg_a[p], M_p = seg_a[P + p]).
// One workgroup per (value head, 16 columns) chains them in segment order:
// S_in[0] = S0 (zero if none), S_in[p + 1] = M_p S_in[p] + D_p. The products
// run on MFMA with both fp32 operands split into bf16 hi + lo (three
// passes); wave w forms rows 16 w .. 16 w + 15. M and D do not depend on the
// chain, so their loads run three steps ahead (a ring of three register
// sets; the loop is unrolled by three so that every set index is a constant).
constexpr int SCP = 132;   // LDS pitch (floats) of the transposed 16 x 128 slice
__global__ void __launch_bounds__(512) segment_combine_kernel(const float* __restrict__ seg_a,
                                                              const float* __restrict__ S0, int P, int nv,
                                                              float* __restrict__ seg_s) {
  __shared__ __attribute__((aligned(16))) float St[2][16][SCP];   // S_in[p] of this slice: [column][row]
  const int h = blockIdx.x / 8, slice = blockIdx.x % 8;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, lr = lane & 15, lg = lane >> 4;
  const int col = slice * 16 + lr;
  const size_t st = static_cast<size_t>(D) * D;
  for (int e = tid; e < D * 16; e += 512) {
    const int row = e >> 4, cc = e & 15;
    const size_t idx = static_cast<size_t>(h) * st + static_cast<size_t>(row) * D + slice * 16 + cc;
    const float x = S0 ? S0[idx] : 0.0f;
    St[0][cc][row] = x;
    seg_s[idx] = x;
  }
  // per set: row 16 w + lr of M_p at k-slots 32 s + 8 lg .. +7, and D_p at
  // this lane's rows 16 w + 4 lg + i, column col
  float4 am[3][4][2];
  float dv[3][4];
  auto load = [&](auto setc, int p) {
    constexpr int r3 = decltype(setc)::value;
    if (p + 1 >= P) return;
    const float* r = seg_a + (static_cast<size_t>(P + p) * nv + h) * st + static_cast<size_t>(16 * w + lr) * D + 8 * lg;
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) {
      am[r3][s4][0] = *reinterpret_cast<const float4*>(r + 32 * s4);
      am[r3][s4][1] = *reinterpret_cast<const float4*>(r + 32 * s4 + 4);
    }
    const float* Dp = seg_a + (static_cast<size_t>(p) * nv + h) * st;
#pragma unroll
    for (int i = 0; i < 4; ++i) dv[r3][i] = Dp[static_cast<size_t>(16 * w + 4 * lg + i) * D + col];
  };
  auto step = [&](auto setc, int p) {
    constexpr int r3 = decltype(setc)::value;
    if (p + 1 >= P) return;
    const int buf = p & 1;
    float* out = seg_s + (static_cast<size_t>(p + 1) * nv + h) * st;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) {
      const float4 a0 = am[r3][s4][0], a1 = am[r3][s4][1];
      const float4 b0 = *reinterpret_cast<const float4*>(&St[buf][lr][32 * s4 + 8 * lg]);
      const float4 b1 = *reinterpret_cast<const float4*>(&St[buf][lr][32 * s4 + 8 * lg + 4]);
      const float a[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
      const float b[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
      Mma<true, false, false>::run(acc, a, b);
    }
    float x[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = acc[i] + dv[r3][i];
    load(setc, p + 3);   // this set is free again
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 16 * w + 4 * lg + i;
      out[static_cast<size_t>(row) * D + col] = x[i];
      St[buf ^ 1][lr][row] = x[i];
    }
    __syncthreads();
  };
  using C0 = std::integral_constant<int, 0>;
  using C1 = std::integral_constant<int, 1>;
  using C2 = std::integral_constant<int, 2>;
  load(C0{}, 0);
  load(C1{}, 1);
  load(C2{}, 2);
  __syncthreads();
  for (int p = 0; p + 1 < P; p += 3) {
    step(C0{}, p);
    step(C1{}, p + 1);
    step(C2{}, p + 2);
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
    const float* __restrict__ egc, const int32_t* __restrict__ order, const float* __restrict__ S0,
    float* __restrict__ ST, TO* __restrict__ o) {
  constexpr bool BF = sizeof(TIn) == 2;
  constexpr int KS = Mma<BF, true, true>::KS, KPL = Mma<BF, true, true>::KPL;

  extern __shared__ __attribute__((aligned(16))) float smem_f[];
  float* Ks = smem_f;                  // [64][KP]
  float* Qs = Ks + CH * KP;            // [64][KP]
  float* Ts = Qs + CH * KP;            // [64][AP]  packed T | rotated P
  float* Vs = Ts + CH * AP;            // [64][16]
  float4* SCs = reinterpret_cast<float4*>(Vs + CH * 16);   // [64]
  float* Rw = reinterpret_cast<float*>(SCs + CH);           // [64][RP]

  int slot, nb;
  state_unit_slice(blockIdx.x, gridDim.x / 8, nv / nk, slot, nb);
  const int n = cu ? order[slot / nv] : 0, h = slot % nv;   // as in the bf16 kernel
  const int unit = n * nv + h;
  const int hk = h / (nv / nk);
  const int lane = threadIdx.x;
  const int lr = lane & 15, lg = lane >> 4;
  const int col = nb * 16 + lr;

  int64_t s_begin, s_end;
  seq_bounds(cu, n, T, s_begin, s_end);
  int cbase, nchunks;
  chunk_span(chunk_off, cu, T, n, cbase, nchunks);

  f32x4 S[8];
#pragma unroll
  for (int t = 0; t < 8; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      S[t][i] = S0 ? S0[(static_cast<int64_t>(unit) * D + 16 * t + 4 * lg + i) * D + col] : 0.0f;

  for (int cc = 0; cc < nchunks; ++cc) {
    const int64_t t0 = s_begin + static_cast<int64_t>(cc) * CH;
    const int L = static_cast<int>(min<int64_t>(CH, s_end - t0));
    const size_t tile = static_cast<size_t>(cbase + cc) * nv + h;
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

// Compute units of the current device, asked once per device.
int device_cus() {
  constexpr int kDevs = 64;
  static std::mutex mu;
  static int cus[kDevs] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kDevs) return 256;
  std::lock_guard<std::mutex> lock(mu);
  if (!cus[dev]) {
    int nc = 0;
    if (hipDeviceGetAttribute(&nc, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || nc <= 0) nc = 256;
    cus[dev] = nc;
  }
  return cus[dev];
}

// Which bf16 state kernel runs: the four-wave form (one slice per workgroup,
// the shorter chain) while every slice gets a CU of its own, else the wide
// form (two slices per workgroup): once the four-wave form would need a
// second round of workgroups, one wide round (about 5,000 cycles per chunk)
// beats two four-wave rounds (about 2 x 2,700). GDN_STATE_FORM=narrow or
// =wide in the environment forces one; both give the same bits.
bool use_wide_state(int64_t slices) {
  if (const char* f = std::getenv("GDN_STATE_FORM")) {
    if (std::strcmp(f, "wide") == 0) return true;
    if (std::strcmp(f, "narrow") == 0) return false;
  }
  return slices > static_cast<int64_t>(device_cus());
}

// Value heads per prep workgroup: all of a key head's (r) when a launch has
// at least 4096 (chunk, key head) items, so that the grid still fills the
// CUs many times over; else one. Grouped, the K and Q tiles (and their conv),
// the Grams and the norms are formed once per key head. GDN_PREP_GROUP=0|1
// in the environment forces either; both give the same bits.
int prep_heads_per_group(int64_t nch, int nk, int nv) {
  const int r = nv / nk;
  if (const char* f = std::getenv("GDN_PREP_GROUP")) return std::atoi(f) ? r : 1;
  return nch * nk >= 4096 ? r : 1;
}

// Segments of the segment-parallel prefill for this call (1 = not split).
// The split triples the recurrence work (pass 1 forms a local state and a
// transition per segment and 16-column slice, pass 2 reruns the segment), so
// it pays where 3 x (value heads x 8) slices still fit the 256 CUs of an
// MI355X: eight segments (of at least four chunks) up to four value heads;
// four from five to eight heads, for sequences of at least 256 chunks, where
// the gain (measured 1.12x at 16384 tokens, 1.29x at 262144) outweighs the
// fixed cost of the extra launches. The count depends on the shape only, not
// on the device, so results do not either. GDN_SEGMENTS=<P> in the
// environment forces a count (1 = unsplit).
int segment_count(int64_t T, int n_seqs, int nv, bool bf16, int& seg_chunks) {
  seg_chunks = 0;
  if (!seg_eligible(n_seqs, nv, bf16)) return 1;
  const int64_t nc = (T + CH - 1) / CH;
  int64_t P = nv <= 4 ? std::min<int64_t>(8, nc / 4) : (nc >= 256 ? 4 : 1);
  if (const char* f = std::getenv("GDN_SEGMENTS")) P = std::min<int64_t>(std::atoi(f), nc);
  P = std::min<int64_t>(P, kMaxSeg);
  if (P < 2) return 1;
  seg_chunks = static_cast<int>((nc + P - 1) / P);
  return static_cast<int>((nc + seg_chunks - 1) / seg_chunks);
}

template <typename TIn>
hipError_t chunk_dispatch(const void* q, const void* k, const void* v, int64_t qs, int64_t ks, int64_t vs,
                          const void* ga, const void* gb, int gm, const float* A_log, const float* dt_bias,
                          const int32_t* cu, int n_seqs, int64_t T, int nk,
                          int nv, float scale, int l2, const float* S0, float* ST, void* o, int o_bf16, void* ws,
                          const ConvIn* cvp, const NormEpi* ne, bool* normalized, hipStream_t s) {
  if (normalized) *normalized = false;
  constexpr bool BF = sizeof(TIn) == 2;
  ConvIn cv = cvp ? *cvp : ConvIn{nullptr, nullptr, nullptr, 0, 0, 0};
  const WsLayout lay = ws_layout(T, n_seqs, nk, nv, BF);
  char* base = static_cast<char*>(ws);
  int32_t* chunk_off = reinterpret_cast<int32_t*>(base + lay.off_chunk_off);
  int32_t* order = reinterpret_cast<int32_t*>(base + lay.off_order);
  float* tp = reinterpret_cast<float*>(base + lay.off_tp);
  float4* sc = reinterpret_cast<float4*>(base + lay.off_sc);
  float* egc = reinterpret_cast<float*>(base + lay.off_egc);
  uint16_t* kf = BF ? reinterpret_cast<uint16_t*>(base + lay.off_kf) : nullptr;
  uint16_t* qf = BF ? reinterpret_cast<uint16_t*>(base + lay.off_qf) : nullptr;

  const int64_t nch = T / CH + n_seqs;
  hipError_t e = hipSuccess;
  // segment-parallel prefill: the segments become the sequences of the chunk table
  int seg_chunks = 0;
  const int P = segment_count(T, n_seqs, nv, BF, seg_chunks);
  if (P > 1) {
    cv.seq_split = 1;
    int32_t* seg_cu = reinterpret_cast<int32_t*>(base + lay.off_segcu);
    segment_table_kernel<<<1, 64, 0, s>>>(cu, T, seg_chunks, P, seg_cu, chunk_off, order);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    cu = seg_cu;
    n_seqs = P;
  } else if (cu) {   // varlen chunk table (one sequence needs none)
    chunk_offsets_kernel<<<1, 256, 0, s>>>(cu, n_seqs, T, static_cast<int32_t>(nch), chunk_off, order);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  {
    const int hg = prep_heads_per_group(static_cast<int64_t>(nch), nk, nv);
    auto kern = gm == 1 ? chunk_prep_kernel<TIn, 1, false, false>
                : gm == 2 ? chunk_prep_kernel<TIn, 2, false, false> : chunk_prep_kernel<TIn, 0, false, false>;
    if (hg > 1)
      kern = gm == 1 ? chunk_prep_kernel<TIn, 1, false, true>
             : gm == 2 ? chunk_prep_kernel<TIn, 2, false, true> : chunk_prep_kernel<TIn, 0, false, true>;
    if constexpr (BF) {
      if (cvp)
        kern = hg > 1 ? (gm == 1 ? chunk_prep_kernel<TIn, 1, true, true> : chunk_prep_kernel<TIn, 2, true, true>)
                      : (gm == 1 ? chunk_prep_kernel<TIn, 1, true, false> : chunk_prep_kernel<TIn, 2, true, false>);
    }
    const size_t lds = prep_lds_bytes<TIn>();
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                            static_cast<int>(lds));
    if (e != hipSuccess) return e;
    kern<<<dim3(static_cast<unsigned>((nv / hg) * nch)), 64 * PREP_WAVES, lds, s>>>(
        static_cast<const TIn*>(q), static_cast<const TIn*>(k), qs, ks, ga, gb, A_log, dt_bias, cu, n_seqs, T, nk, nv,
        scale, l2, chunk_off, tp, sc, egc, kf, qf, cv, hg);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const unsigned grid = static_cast<unsigned>(n_seqs) * nv * (D / 16);
  if constexpr (BF) {
    const uint16_t* xf = reinterpret_cast<const uint16_t*>(tp);
    const float* scp = reinterpret_cast<const float*>(sc);
    const uint16_t* vb = static_cast<const uint16_t*>(v);
    auto launch = [&](auto kern, auto* optr) {
      kern<<<grid, 256, 0, s>>>(vb, vs, cu, n_seqs, T, nk, nv, chunk_off, xf, scp, egc, kf, qf, order, S0, ST, optr,
                                cv, SegRun{0, 0, -1});
      return hipGetLastError();
    };
    if (P > 1) {
      // pass 1: every segment from zero (D) and from the identity with v = 0
      // (M), no outputs; then the incoming states; pass 2: every segment from
      // its incoming state, outputs, and the last one's final state
      float* seg_a = reinterpret_cast<float*>(base + lay.off_sega);
      float* seg_s = reinterpret_cast<float*>(base + lay.off_segs);
      auto passes = [&](auto kern, auto* optr) {
        kern<<<2 * grid, 256, 0, s>>>(vb, vs, cu, n_seqs, T, nk, nv, chunk_off, xf, scp, egc, kf, qf, order,
                                      nullptr, seg_a, optr, cv, SegRun{P, 1, -1});
        hipError_t err = hipGetLastError();
        if (err != hipSuccess) return err;
        segment_combine_kernel<<<nv * (D / 16), 512, 0, s>>>(seg_a, S0, P, nv, seg_s);
        err = hipGetLastError();
        if (err != hipSuccess) return err;
        kern<<<grid, 256, 0, s>>>(vb, vs, cu, n_seqs, T, nk, nv, chunk_off, xf, scp, egc, kf, qf, order, seg_s, ST,
                                  optr, cv, SegRun{0, 0, P - 1});
        return hipGetLastError();
      };
      if (cvp) {
        if (o_bf16) return passes(chunk_state_bf16_kernel<uint16_t, true, false>, static_cast<uint16_t*>(o));
        return passes(chunk_state_bf16_kernel<float, true, false>, static_cast<float*>(o));
      }
      if (o_bf16) return passes(chunk_state_bf16_kernel<uint16_t, false, false>, static_cast<uint16_t*>(o));
      return passes(chunk_state_bf16_kernel<float, false, false>, static_cast<float*>(o));
    }
    if (use_wide_state(static_cast<int64_t>(grid))) {
      const unsigned wgrid = grid / 2;   // two slices per workgroup
      if (ne && cvp && !o_bf16) {
        // the norm epilogue inside the kernel when all its workgroups can be
        // resident at once (cooperative launch); else the caller normalizes
        auto kern = chunk_state_wide_kernel<float, true, true>;
        int per_cu = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(kern), 512, 0) ==
                hipSuccess &&
            static_cast<int64_t>(per_cu) * device_cus() >= static_cast<int64_t>(wgrid)) {
          unsigned long long* ring = reinterpret_cast<unsigned long long*>(base + lay.off_ring);
          const int64_t nw = static_cast<int64_t>(n_seqs) * nv * static_cast<int64_t>(kRingBytesPerUnit / 8);
          clear_u64_kernel<<<static_cast<unsigned>((nw + 255) / 256), 256, 0, s>>>(ring, nw);
          e = hipGetLastError();
          if (e != hipSuccess) return e;
          const uint16_t* a_v = vb;
          int64_t a_vs = vs;
          const int32_t* a_cu = cu;
          int a_n = n_seqs;
          int64_t a_T = T;
          int a_nk = nk, a_nv = nv;
          const int32_t* a_off = chunk_off;
          const uint16_t* a_xf = xf;
          const float* a_scp = scp;
          const float* a_egc = egc;
          const uint16_t* a_kf = kf;
          const uint16_t* a_qf = qf;
          const int32_t* a_order = order;
          const float* a_S0 = S0;
          float* a_ST = ST;
          float* a_o = static_cast<float*>(o);
          ConvIn a_cv = cv;
          EpiIn a_ep{ne->z, ne->w, ne->eps, ring};
          void* args[] = {&a_v,   &a_vs,  &a_cu,    &a_n,  &a_T,  &a_nk, &a_nv, &a_off, &a_xf, &a_scp,
                          &a_egc, &a_kf,  &a_qf,    &a_order, &a_S0, &a_ST, &a_o, &a_cv, &a_ep};
          e = hipLaunchCooperativeKernel(reinterpret_cast<const void*>(kern), dim3(wgrid), dim3(512), args, 0, s);
          if (e == hipSuccess) {
            if (normalized) *normalized = true;
            return e;
          }
          // refused: the plain launch below, and the caller normalizes
          (void)hipGetLastError();
        }
      }
      auto launch_wide = [&](auto kern, auto* optr) {   // eight waves with the conv (conv waves), else four
        kern<<<wgrid, cvp ? 512 : 256, 0, s>>>(vb, vs, cu, n_seqs, T, nk, nv, chunk_off, xf, scp, egc, kf, qf, order,
                                              S0, ST, optr, cv, EpiIn{});
        return hipGetLastError();
      };
      if (cvp) {
        if (o_bf16) return launch_wide(chunk_state_wide_kernel<uint16_t, true, false>, static_cast<uint16_t*>(o));
        return launch_wide(chunk_state_wide_kernel<float, true, false>, static_cast<float*>(o));
      }
      if (o_bf16) return launch_wide(chunk_state_wide_kernel<uint16_t, false, false>, static_cast<uint16_t*>(o));
      return launch_wide(chunk_state_wide_kernel<float, false, false>, static_cast<float*>(o));
    }
    // Several sequences (cu_seqlens): two workgroups per CU, so that a CU can
    // take another (sequence, head, slice) while one runs a long sequence;
    // measured on 8 packed sequences of 512-16384 tokens, 11 % less time. One
    // sequence keeps one workgroup per CU: its workgroups all run equally
    // long and a second one per CU only competes (3 % slower at 262,144 tokens).
    const bool dual = cu != nullptr && n_seqs > 1;
    if (cvp) {
      if (dual) {
        if (o_bf16) return launch(chunk_state_bf16_kernel<uint16_t, true, true>, static_cast<uint16_t*>(o));
        return launch(chunk_state_bf16_kernel<float, true, true>, static_cast<float*>(o));
      }
      if (o_bf16) return launch(chunk_state_bf16_kernel<uint16_t, true, false>, static_cast<uint16_t*>(o));
      return launch(chunk_state_bf16_kernel<float, true, false>, static_cast<float*>(o));
    }
    if (dual) {
      if (o_bf16) return launch(chunk_state_bf16_kernel<uint16_t, false, true>, static_cast<uint16_t*>(o));
      return launch(chunk_state_bf16_kernel<float, false, true>, static_cast<float*>(o));
    }
    if (o_bf16) return launch(chunk_state_bf16_kernel<uint16_t, false, false>, static_cast<uint16_t*>(o));
    return launch(chunk_state_bf16_kernel<float, false, false>, static_cast<float*>(o));
  } else {
    const size_t lds = generic_lds_bytes();
    auto launch = [&](auto kern, auto* optr) {
      hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
      if (err != hipSuccess) return err;
      kern<<<grid, 64, lds, s>>>(static_cast<const TIn*>(q), static_cast<const TIn*>(k), static_cast<const TIn*>(v),
                                 qs, ks, vs, cu, n_seqs, T, nk, nv, chunk_off, tp, sc, egc, order, S0, ST, optr);
      return hipGetLastError();
    };
    if (o_bf16) return launch(chunk_state_generic_kernel<TIn, uint16_t>, static_cast<uint16_t*>(o));
    return launch(chunk_state_generic_kernel<TIn, float>, static_cast<float*>(o));
  }
}

// ------------------------------------------------------------------ allocation-free workspace
// A file-scope device array that stands in for the caller's workspace in
// launch_chunk_fwd_noalloc. Every GPU the library runs on holds its own copy
// for the life of the process. In host code `scratch` names a host-side
// stand-in, not a device address: kernels and copies use the per-device
// address from hipGetSymbolAddress instead.
__device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch array, looked up once per
// device with that device current.
hipError_t scratch_ptr(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace

size_t chunk_workspace_bytes(int64_t T, int n_seqs, int nk, int nv, int bf16) {
  return ws_layout(T, n_seqs, nk, nv, bf16 != 0).total;
}

hipError_t launch_chunk_fwd(const void* q, const void* k, const void* v, int bf16, int64_t qs, int64_t ks,
                            int64_t vs, const void* ga, const void* gb, int gm, const float* A_log,
                            const float* dt_bias, const int32_t* cu, int n_seqs, int64_t T, int nk, int nv,
                            float scale, int l2, const float* S0, float* ST, void* o, int o_bf16, void* ws,
                            hipStream_t s) {
  if (bf16)
    return chunk_dispatch<uint16_t>(q, k, v, qs, ks, vs, ga, gb, gm, A_log, dt_bias, cu, n_seqs, T, nk, nv, scale, l2,
                                    S0, ST, o, o_bf16, ws, nullptr, nullptr, nullptr, s);
  return chunk_dispatch<float>(q, k, v, qs, ks, vs, ga, gb, gm, A_log, dt_bias, cu, n_seqs, T, nk, nv, scale, l2, S0,
                               ST, o, o_bf16, ws, nullptr, nullptr, nullptr, s);
}

hipError_t launch_chunk_fwd_noalloc(const void* q, const void* k, const void* v, int bf16, int64_t qs, int64_t ks,
                                    int64_t vs, const void* ga, const void* gb, int gm, const float* A_log,
                                    const float* dt_bias, const int32_t* cu, int n_seqs, int64_t T, int nk, int nv,
                                    float scale, int l2, const float* S0, float* ST, void* o, int o_bf16,
                                    hipStream_t s) {
  // the caller has checked chunk_workspace_bytes(...) <= kNoallocScratchBytes
  void* ws = nullptr;
  const hipError_t e = scratch_ptr(&ws);
  if (e != hipSuccess) return e;
  return launch_chunk_fwd(q, k, v, bf16, qs, ks, vs, ga, gb, gm, A_log, dt_bias, cu, n_seqs, T, nk, nv, scale, l2, S0,
                          ST, o, o_bf16, ws, s);
}

hipError_t launch_chunk_fwd_conv(const void* x, int64_t xs, const float* conv_w, const float* conv_b,
                                 const void* conv_st, int state_len, const void* a, const void* b, int gm,
                                 const float* A_log, const float* dt_bias, const int32_t* cu, int n_seqs, int64_t T,
                                 int nk, int nv, float scale, int l2, const float* S0, float* ST, void* o, int o_bf16,
                                 void* ws, const NormEpi* ne, hipStream_t s) {
  const int conv_dim = (2 * nk + nv) * D;
  const ConvIn cv{conv_w, conv_b, static_cast<const uint16_t*>(conv_st), state_len, conv_dim, 0};
  const uint16_t* xb = static_cast<const uint16_t*>(x);
  bool normalized = false;
  hipError_t e = chunk_dispatch<uint16_t>(xb, xb + nk * D, xb + 2 * nk * D, xs, xs, xs, a, b, gm, A_log, dt_bias, cu,
                                          n_seqs, T, nk, nv, scale, l2, S0, ST, o, o_bf16, ws, &cv, ne, &normalized, s);
  // the epilogue did not run inside the state kernel: o (fp32) is normalized in place
  if (e == hipSuccess && ne && !normalized && T > 0)
    e = launch_gated_rmsnorm(o, 0, ne->z, 1, ne->w, T * nv, D, ne->eps, o, 0, s);
  return e;
}

}  // namespace gdn
