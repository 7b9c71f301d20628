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

constexpr int TILE_ELEMS = CH * D;   // bf16 elements of one 16 KB operand tile

// Workspace: chunk table | per (chunk, value head): 16 KB tile, 1 KB of
// per-token scalars, exp(G_C) | bf16 inputs only, per (chunk, key head): K, Q
// and K^T operand tiles of 16 KB each.
struct WsLayout {
  size_t off_chunk_off, off_tp, off_sc, off_egc, off_kf, off_qf, off_ktf, total;
};
inline WsLayout ws_layout(int64_t T, int n_seqs, int nk, int nv, bool bf16) {
  const int64_t nch = T / CH + n_seqs;   // >= sum_n ceil(len_n / 64)
  const size_t tile_bytes = static_cast<size_t>(TILE_ELEMS) * 2;
  WsLayout w{};
  size_t o = 0;
  w.off_chunk_off = o; o += (static_cast<size_t>(n_seqs) + 1) * sizeof(int32_t); o = (o + 255) & ~size_t(255);
  w.off_tp = o;        o += static_cast<size_t>(nch) * nv * tile_bytes;
  w.off_sc = o;        o += static_cast<size_t>(nch) * nv * CH * sizeof(float4);
  w.off_egc = o;       o += static_cast<size_t>(nch) * nv * sizeof(float); o = (o + 255) & ~size_t(255);
  w.off_kf = w.off_qf = w.off_ktf = o;
  if (bf16) {
    w.off_kf = o;  o += static_cast<size_t>(nch) * nk * tile_bytes;
    w.off_qf = o;  o += static_cast<size_t>(nch) * nk * tile_bytes;
    w.off_ktf = o; o += static_cast<size_t>(nch) * nk * tile_bytes;
  }
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
// K tile in LDS -> transposed blocks (w, s), w = 16 rows of dk, s = 32-token
// k-step: lane (lr, lg) holds K[32s + perm32(lg, j)][16w + lr], tokens >= L
// zero. This call writes w = 2 s2, 2 s2 + 1 (dk step s2). The transpose runs
// on MFMA: with A = 16 token rows x 32 dk of K and B = a 0/1 matrix that picks
// dk 16w + c for column c, D = K[16t + r][16w + c] lands in accumulator order
// (lane (c, lg) holds rows 4 lg .. +3), which is slots 0-3 (t = 2s) or 4-7
// (t = 2s + 1) of the block. Each D entry is a single bf16 product with 1, so
// it converts back to bf16 exactly.
template <int EP>
__device__ __forceinline__ void write_col_blocks(const uint16_t* tile, int L, uint16_t* __restrict__ dst, int lane,
                                                 int s2) {
  const int lr = lane & 15, lg = lane >> 4;
  // sel[hh] picks dk 16 hh + lr out of the 32-wide step (B slot (lg, j) is dk 8 lg + j)
  bf16x8 sel[2];
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    uint32_t d[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int k0 = 8 * lg + 2 * p;
      d[p] = (k0 == 16 * hh + lr ? 0x3f80u : 0u) | (k0 + 1 == 16 * hh + lr ? 0x3f800000u : 0u);
    }
    sel[hh] = __builtin_bit_cast(bf16x8, make_uint4(d[0], d[1], d[2], d[3]));
  }
  f32x4 Dt[2][4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int row = 16 * t + lr;
    const bf16x8 a = __builtin_bit_cast(
        bf16x8, zero_if(row >= L, *reinterpret_cast<const uint4*>(tile + row * EP + 32 * s2 + 8 * lg)));
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) Dt[hh][t] = mfma_bf16(a, sel[hh], f32x4{0.f, 0.f, 0.f, 0.f});
  }
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    const int w = 2 * s2 + hh;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const f32x4& lo = Dt[hh][2 * s];
      const f32x4& hi = Dt[hh][2 * s + 1];
      uint2 p0, p1, unused;
      split4_packed(make_float4(lo[0], lo[1], lo[2], lo[3]), p0, unused);
      split4_packed(make_float4(hi[0], hi[1], hi[2], hi[3]), p1, unused);
      *reinterpret_cast<uint4*>(dst + (2 * w + s) * BLK_ELEMS + lane * 8) = make_uint4(p0.x, p0.y, p1.x, p1.y);
    }
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

// ------------------------------------------------------------------ prep
// Four waves per (chunk, value head). The ten lower 16x16 tile pairs (mi, mj)
// of the Grams, A and P are dealt round-robin (pair p goes to wave p % 4);
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

// (at most 128 VGPRs: four waves per SIMD, i.e. four blocks per CU, which is
// also what the LDS holds)
template <typename TIn>
__global__ void __launch_bounds__(64 * PREP_WAVES) __attribute__((amdgpu_waves_per_eu(4))) chunk_prep_kernel(
    const TIn* __restrict__ q, const TIn* __restrict__ k, int64_t qs, int64_t ks,
    const float* __restrict__ g, const float* __restrict__ beta, const int32_t* __restrict__ cu,
    int n_seqs, int64_t T, int nk, int nv, float scale, int l2, const int32_t* __restrict__ chunk_off,
    float* __restrict__ tp, float4* __restrict__ sc, float* __restrict__ egc, uint16_t* __restrict__ kf,
    uint16_t* __restrict__ qf, uint16_t* __restrict__ ktf) {
  constexpr bool BF = sizeof(TIn) == 2;
  constexpr int EP = prep_pitch<TIn>();
  using MG = Mma<BF, true, true>;
  constexpr int KS = MG::KS, KPL = MG::KPL;
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

  // heads vary fastest: the value heads of one key head, and the per-token
  // g and beta of all heads (one cache line per token), are read by
  // neighbouring workgroups
  const int h = blockIdx.x;
  const int c = blockIdx.y;
  const int hk = h / (nv / nk);
  const int total = cu ? chunk_off[n_seqs] : static_cast<int>((T + CH - 1) / CH);
  if (c >= total) return;
  const int n = cu ? find_le(chunk_off, n_seqs, c) : 0;
  int64_t s_begin, s_end;
  seq_bounds(cu, n, T, s_begin, s_end);
  const int64_t t0 = s_begin + static_cast<int64_t>(c - (cu ? chunk_off[n] : 0)) * CH;
  const int L = static_cast<int>(min<int64_t>(CH, s_end - t0));
  const int tid = threadIdx.x, lane = tid & 63, lr = lane & 15, lg = lane >> 4;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  // per-token g and beta (wave 0, lane = token), issued first so their
  // latency overlaps the tile loads and the Grams
  const float g_ld = g[(t0 + min(lane, L - 1)) * nv + h];
  const float b_ld = beta[(t0 + min(lane, L - 1)) * nv + h];

  // 1. K and Q tiles into LDS; rows past the sequence end re-read the last
  //    valid row: their norms are forced to 0 below, so they contribute
  //    nothing to A, P or the scalars
  {
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

  // 2. |q_i|^2: four threads per row, 32 elements each
  {
    const int row = tid >> 2, part = tid & 3;
    float sqq = 0.f;
#pragma unroll 8
    for (int e = 0; e < D / 4; ++e) {
      const float x = tof(Qs[row * EP + part * (D / 4) + e]);
      sqq = fmaf(x, x, sqq);
    }
    sqq += __shfl_xor(sqq, 1, 64);
    sqq += __shfl_xor(sqq, 2, 64);
    if (part == 0) rq_s[row] = row < L ? (l2 ? 1.0f / sqrtf(sqq + kEps) : 1.0f) : 0.0f;
  }
  // 3. Grams on this wave's lower 16x16 tile pairs p = wv + 4 u, kept in registers
  constexpr int NP = 3;
  f32x4 gkk[NP], gqk[NP];
#pragma unroll
  for (int u = 0; u < NP; ++u) {
    gkk[u] = f32x4{0.f, 0.f, 0.f, 0.f};
    gqk[u] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int p = wv + 4 * u;
    if (p >= 10) break;
    const int mi = tile_mi(p), mj = tile_mj(p);
#pragma unroll
    for (int s = 0; s < D / KS; ++s) {
      if constexpr (BF) {   // raw bf16 fragments, one 16-byte LDS read each
        const int kk = s * KS + KPL * lg;
        const bf16x8 ak = *reinterpret_cast<const bf16x8*>(Ks + (16 * mi + lr) * EP + kk);
        const bf16x8 aq = *reinterpret_cast<const bf16x8*>(Qs + (16 * mi + lr) * EP + kk);
        const bf16x8 bk = *reinterpret_cast<const bf16x8*>(Ks + (16 * mj + lr) * EP + kk);
        gkk[u] = mfma_bf16(ak, bk, gkk[u]);
        gqk[u] = mfma_bf16(aq, bk, gqk[u]);
      } else {
        float ak[KPL], aq[KPL], bk[KPL];
#pragma unroll
        for (int j = 0; j < KPL; ++j) {
          const int kk = s * KS + KPL * lg + j;
          ak[j] = tof(Ks[(16 * mi + lr) * EP + kk]);
          aq[j] = tof(Qs[(16 * mi + lr) * EP + kk]);
          bk[j] = tof(Ks[(16 * mj + lr) * EP + kk]);
        }
        MG::run(gkk[u], ak, bk);
        MG::run(gqk[u], aq, bk);
      }
    }
  }
  // 3b. bf16 inputs: K, Q and K^T operand blocks of the state recurrence,
  //     once per key head: K and Q by its first value head, K^T by its last;
  //     wave wv writes token tile wv (K, Q) and dk step wv (K^T)
  if constexpr (BF) {
    const int r = nv / nk, rho = h % r;
    const size_t kt = (static_cast<size_t>(c) * nk + hk) * TILE_ELEMS;
    if (rho == 0) {
      write_row_blocks<EP>(Ks, L, kf + kt, lane, wv);
      write_row_blocks<EP>(Qs, L, qf + kt, lane, wv);
    }
    if (rho == r - 1) write_col_blocks<EP>(Ks, L, ktf + kt, lane, wv);
  }
  // 4. |k_i|^2 from the Gram diagonals (pairs 0, 2, 5, 9)
#pragma unroll
  for (int u = 0; u < NP; ++u) {
    const int p = wv + 4 * u;
    if (p >= 10) break;
    const int mi = tile_mi(p), mj = tile_mj(p);
    if (mi == mj && lr >= 4 * lg && lr < 4 * lg + 4) {
      const int row = 16 * mi + lr;
      const float skk = gkk[u][lr - 4 * lg];
      rk_s[row] = row < L ? (l2 ? 1.0f / sqrtf(skk + kEps) : 1.0f) : 0.0f;
    }
  }
  // 5. chunk-local cumulative decay in fp64 (wave 0, lane = token)
  if (wv == 0) {
    const bool valid = lane < L;
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

  // 6. A (into LDS) and P (kept in registers, in place of the QK^T Gram);
  //    per-token values are read before the first write to Aw (which could
  //    alias them as far as the compiler knows)
  {
    double Gc[NP], Gr[NP][4];
    float rkc[NP], ar[NP][4], pr[NP][4];
#pragma unroll
    for (int u = 0; u < NP; ++u) {
      const int p = min(wv + 4 * u, 9);
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
      const int p = wv + 4 * u;
      if (p >= 10) break;
      const int mi = tile_mi(p), mj = tile_mj(p);
      const int j = 16 * mj + lr;
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int i = 16 * mi + 4 * lg + ii;
        const float dec = (j <= i) ? expf(static_cast<float>(Gr[u][ii] - Gc[u])) : 0.0f;
        Aw[i * AP + j] = (j < i) ? ar[u][ii] * rkc[u] * dec * gkk[u][ii] : 0.0f;
        gqk[u][ii] = (j <= i) ? pr[u][ii] * rkc[u] * dec * gqk[u][ii] : 0.0f;
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
      Tw[(16 * I + i) * AP + 16 * I + jc] = t[i];
    }
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
    const int p = wv + 4 * u;
    if (p >= 10) break;
    const int mi = tile_mi(p), mj = tile_mj(p);
    const int j = 16 * mj + lr;
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      const int i = 16 * mi + 4 * lg + ii;
      if (j <= i) Tw[(63 - i) * AP + (63 - j)] = gqk[u][ii];
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
}

// ------------------------------------------------------------------ state: bf16 inputs, 8 waves per 16 columns
// One workgroup per (sequence, value head, 16 value columns), eight waves with
// two roles over the chunk's four 16-token tiles m = w % 4:
//   waves 0-3 (recurrence side): X = K S, R = beta v - b X, U = R + T R;
//   waves 4-7 (output side):     Y = Q S, O = a Y + P U, computed transposed
//                                (operands swapped) so a lane holds 4
//                                consecutive columns of one token row, one
//                                phase behind the recurrence side.
// Wave w also owns rows 16w..16w+15 of S (128 x 16, fp32, one MFMA
// accumulator) and updates them: S_w = e^{G_C} S_w + K[:, rows of w]^T (c U).
// Waves w and w+4 share a SIMD, so each SIMD interleaves one wave of each side.
//
// Every operand comes from the workspace as contiguous blocks already in
// fragment order (see the operand-block writers), loaded two chunks ahead
// into three rotating register sets, in three groups spread over the chunk's
// three phases so the memory pipe never backs up into the waves. Tiles
// produced inside the chunk (S, R, U, c U) are split into bf16 hi + lo by
// the producing wave and pass through LDS in the same block order, so a
// consumer reads its share of a B operand with one 16-byte read per plane.
constexpr int BLK_BYTES = BLK_ELEMS * 2;

struct Prefetch {
  uint4 f[4];       // K (recurrence side) or Q (output side) blocks, k-steps 0..3 over dk
  uint4 x[4];       // T (recurrence) or P (output) blocks: hi k0, hi k1, lo k0, lo k1
  uint4 kt[2];      // K^T blocks of this wave's 16 rows of S, token k-steps 0, 1
};
// Tiles 0 and 1 need only k-step 0 of T and P, so x[1] and x[3] are free on
// waves 0, 1, 4, 5; two of those waves carry the per-chunk staging loads there
// (their masks zero x[1] and x[3] wherever T or P blocks are formed).
constexpr int kScalarWave = 4;   // per-token scalars (x[1]) and exp(G_C) (x[3].x)
constexpr int kValueWave = 5;    // the chunk's 64 x 16 slice of V (x[1], x[3])
// Every loaded word is consumed on every path of every wave that loads it: a
// register whose load is still counted as pending when the compiler reuses it
// makes it wait on the in-order counter, and with it on every later load.

__device__ __forceinline__ bf16x8 as_bf16x8(const uint4& u) { return __builtin_bit_cast(bf16x8, u); }
__device__ __forceinline__ uint4 and4(const uint4& a, const uint4& m) {
  return make_uint4(a.x & m.x, a.y & m.y, a.z & m.z, a.w & m.w);
}
// reverse the order of 8 packed bf16
__device__ __forceinline__ uint4 rev8(const uint4& a) {
  auto sw = [](uint32_t d) { return (d >> 16) | (d << 16); };
  return make_uint4(sw(a.w), sw(a.z), sw(a.y), sw(a.x));
}
__device__ __forceinline__ uint4 lds16(const unsigned char* p) { return *reinterpret_cast<const uint4*>(p); }
__device__ __forceinline__ float bits_f(uint32_t u) { return __builtin_bit_cast(float, u); }

// Accumulator tile -> LDS exchange slot: a lane's 4 rows of 16-row tile t
// are slots 4 (t % 2) .. +3 of that lane's 16 bytes in k-step t / 2.
__device__ __forceinline__ void put_tile(unsigned char* X, int planes_off, int t, int lane, const f32x4& v) {
  uint2 hi, lo;
  split4_packed(make_float4(v[0], v[1], v[2], v[3]), hi, lo);
  unsigned char* p = X + (t >> 1) * BLK_BYTES + lane * 16 + (t & 1) * 8;
  *reinterpret_cast<uint2*>(p) = hi;
  *reinterpret_cast<uint2*>(p + planes_off) = lo;
}

template <typename TO>
__global__ void __launch_bounds__(512) chunk_state_bf16_kernel(
    const uint16_t* __restrict__ v, int64_t vs, const int32_t* __restrict__ cu, int n_seqs, int64_t T, int nk,
    int nv, const int32_t* __restrict__ chunk_off, const uint16_t* __restrict__ xf, const float* __restrict__ scp,
    const float* __restrict__ egc, const uint16_t* __restrict__ kf, const uint16_t* __restrict__ qf,
    const uint16_t* __restrict__ ktf, const float* __restrict__ S0, float* __restrict__ ST, TO* __restrict__ o) {
  // exchange tiles, each [plane hi | plane lo][k-step][64 lanes][16 B]
  __shared__ __attribute__((aligned(16))) unsigned char SX[2 * 4 * BLK_BYTES];   // S, 4 dk k-steps
  __shared__ __attribute__((aligned(16))) unsigned char RX[2 * 2 * BLK_BYTES];   // R, 2 token k-steps
  __shared__ __attribute__((aligned(16))) unsigned char UX[2 * 2 * BLK_BYTES];   // U
  __shared__ __attribute__((aligned(16))) unsigned char CX[2 * 2 * BLK_BYTES];   // c U
  constexpr int SXP = 4 * BLK_BYTES, TXP = 2 * BLK_BYTES;                        // plane offsets
  // per-chunk inputs staged by one wave each, double-buffered by chunk parity:
  // scalar planes a | b | c | beta over the 64 tokens, exp(G_C) (every entry),
  // and V of the four recurrence tiles in accumulator order [tile][lane][row]
  __shared__ __attribute__((aligned(16))) float SCS[2][4 * CH];
  __shared__ float EGS[2][64];
  __shared__ __attribute__((aligned(16))) uint16_t VS[2][4 * 64 * 4];

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

  // masks of the triangular blocks (constant over chunks): T needs token <
  // row; P slot j holds token 32s + perm32(lg, 7 - j) and needs it <= row
  uint4 msk[2];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    uint32_t mm[4];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      bool lo, hi;
      if (rec) {
        lo = 32 * s + perm32(lg, 2 * d) < row;
        hi = 32 * s + perm32(lg, 2 * d + 1) < row;
      } else {
        lo = 32 * s + perm32(lg, 7 - 2 * d) <= row;
        hi = 32 * s + perm32(lg, 6 - 2 * d) <= row;
      }
      mm[d] = (lo ? 0x0000ffffu : 0u) | (hi ? 0xffff0000u : 0u);
    }
    msk[s] = make_uint4(mm[0], mm[1], mm[2], mm[3]);
  }

  int64_t s_begin, s_end;
  seq_bounds(cu, n, T, s_begin, s_end);
  int cbase, nchunks;
  chunk_span(chunk_off, cu, T, n, cbase, nchunks);

  f32x4 S = {0.f, 0.f, 0.f, 0.f};        // rows 16w + 4lg + i, column col
  if (S0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) S[i] = S0[(static_cast<int64_t>(unit) * D + 16 * w + 4 * lg + i) * D + col];
  }

  // lane-constant block offsets (bytes). The T block of k-step s is (m, s);
  // the P block is the turned tile's (3 - m, 1 - s) read in reversed lane
  // order. Tiles 0 and 1 need only k-step 0 of either: their second block
  // reads as zeros from past the resource, so no branch guards any load.
  const uint32_t lo16 = static_cast<uint32_t>(lane * 16);
  uint32_t xo[2];
#pragma unroll
  for (int s = 0; s < 2; ++s)
    xo[s] = rec ? static_cast<uint32_t>((2 * m + s) * BLK_BYTES) + lo16
                : static_cast<uint32_t>((2 * (3 - m) + 1 - s) * BLK_BYTES + (63 - lane) * 16);
  const bool two_k = m >= 2;               // tiles 0, 1 need only k-step 0 of T and P
  const uint32_t fo = static_cast<uint32_t>(4 * m * BLK_BYTES) + lo16;
  const uint32_t kto = static_cast<uint32_t>(2 * w * BLK_BYTES) + lo16;
  // V staging: lane l of instruction i loads token 32i + l / 2, columns 8 (l % 2) .. +7
  const uint32_t vo0 = static_cast<uint32_t>(((lane >> 1) * vs + slice * 16 + 8 * (lane & 1)) * 2);

  // group 0: T/P blocks (and the scalar block on the scalar wave); group 1:
  // K^T blocks (and V on the value wave); group 2: K/Q blocks -- the larger
  // groups go to the phases with less LDS traffic
  auto load_chunk = [&](int cc, Prefetch& pf, int part) {
    const size_t ct = static_cast<size_t>(cbase + cc) * nv + h;    // (chunk, value head)
    const size_t kt = static_cast<size_t>(cbase + cc) * nk + hk;   // (chunk, key head)
    if (part == 0) {
      const rsrc_t rx = make_rsrc(xf + ct * TILE_ELEMS, TILE_ELEMS * 2);
      pf.x[0] = bload16(rx, xo[0]);
      pf.x[2] = bload16(rx, xo[0] + 8 * BLK_BYTES);
      if (two_k) {
        pf.x[1] = bload16(rx, xo[1]);
        pf.x[3] = bload16(rx, xo[1] + 8 * BLK_BYTES);
      }
      if (w == kScalarWave) {
        // exp(G_C) through a vector load: a uniform (scalar) load would share
        // lgkmcnt with LDS traffic and stall the next LDS wait for a full
        // memory round trip
        pf.x[1] = bload16(make_rsrc(scp + ct * 4 * CH, 4 * CH * 4), lo16);
        pf.x[3].x = __builtin_amdgcn_raw_buffer_load_b32(make_rsrc(egc + ct, 4), lo16 & 0u, 0, 0);
      }
    } else if (part == 1) {
      const rsrc_t rk = make_rsrc(ktf + kt * TILE_ELEMS, TILE_ELEMS * 2);
      pf.kt[0] = bload16(rk, kto);
      pf.kt[1] = bload16(rk, kto + BLK_BYTES);
      if (w == kValueWave) {
        // V rows past the sequence end read as zeros (resource sized to the valid rows)
        const int64_t t0 = s_begin + static_cast<int64_t>(cc) * CH;
        const int L = static_cast<int>(min<int64_t>(CH, s_end - t0));
        const rsrc_t rv = make_rsrc(v + t0 * vs + static_cast<int64_t>(h) * D,
                                    static_cast<uint32_t>(((L - 1) * vs + D) * 2));
        pf.x[1] = bload16(rv, vo0);
        pf.x[3] = bload16(rv, vo0 + static_cast<uint32_t>(32 * vs * 2));
      }
    } else {
      const rsrc_t rf = make_rsrc((rec ? kf : qf) + kt * TILE_ELEMS, TILE_ELEMS * 2);
#pragma unroll
      for (int s = 0; s < 4; ++s) pf.f[s] = bload16(rf, fo + s * BLK_BYTES);
    }
  };
  // stage a chunk's scalars, exp(G_C) and V slice in LDS buffer `buf`
  auto commit = [&](const Prefetch& pf, int buf) {
    if (w == kScalarWave) {
      *reinterpret_cast<uint4*>(&SCS[buf][4 * lane]) = pf.x[1];
      EGS[buf][lane] = bits_f(pf.x[3].x);
    }
    if (w == kValueWave) {
      // lane holds V[t][8 (lane % 2) + e], e = 0..7, for t = 32i + lane / 2;
      // slot of (t, c): tile t / 16, lane c + 16 ((t % 16) / 4), row t % 4
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const uint4& vi = pf.x[2 * i + 1];
        const uint32_t d[4] = {vi.x, vi.y, vi.z, vi.w};
        const int t = 32 * i + (lane >> 1);
        uint16_t* base = &VS[buf][((t >> 4) * 64 + 16 * ((t & 15) >> 2)) * 4 + (t & 3)];
#pragma unroll
        for (int e = 0; e < 8; ++e)
          base[(8 * (lane & 1) + e) * 4] = static_cast<uint16_t>((e & 1) ? (d[e >> 1] >> 16) : (d[e >> 1] & 0xffffu));
      }
    }
  };
  auto publish_S = [&]() { put_tile(SX, SXP, w, lane, S); };

  // The output side runs one phase behind the recurrence side: Y of chunk c
  // is formed in phase 2 of chunk c and kept in registers with chunk c's
  // masked P blocks, and the O tile of chunk c in phase 1 of chunk c+1, from
  // those, U of chunk c (still in LDS) and its scalars. The recurrence chain
  // X -> R -> U -> S then never waits on output work, and the S reads split
  // over two phases.
  f32x4 Yprev = {0.f, 0.f, 0.f, 0.f};
  uint4 Pprev[4] = {};
  // O^T tile: lane (lr, lg) holds O[token 16m + lr][columns 16 slice + 4lg + i]
  const uint32_t oo0 = static_cast<uint32_t>((row * nv * D + slice * 16 + 4 * lg) * sizeof(TO));
  // O^T = a Y^T + U^T P^T for chunk co (P slots hold tokens in reversed order:
  // reverse U too), stored at once: the chunk's loads are already issued, and
  // a store issued before a load would make every wait on that load also wait
  // for the store (one in-order completion counter)
  auto out_tile = [&](int co, const uint4 (&xp)[4]) {
    f32x4 O0, O1 = {0.f, 0.f, 0.f, 0.f};
    const float ar = SCS[co & 1][row];     // a of this lane's token row
#pragma unroll
    for (int i = 0; i < 4; ++i) O0[i] = ar * Yprev[i];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      if (s == 1 && !two_k) break;
      const bf16x8 ah = as_bf16x8(xp[s]), al = as_bf16x8(xp[2 + s]);
      const bf16x8 bh = as_bf16x8(rev8(lds16(UX + s * BLK_BYTES + lane * 16)));
      const bf16x8 bl = as_bf16x8(rev8(lds16(UX + TXP + s * BLK_BYTES + lane * 16)));
      f32x4& Oa = s == 0 ? O0 : O1;
      Oa = mfma_bf16(bh, al, Oa);
      Oa = mfma_bf16(bl, ah, Oa);
      Oa = mfma_bf16(bh, ah, Oa);
    }
    float Ov[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) Ov[i] = O0[i] + O1[i];
    const int64_t t0 = s_begin + static_cast<int64_t>(co) * CH;
    const int L = static_cast<int>(min<int64_t>(CH, s_end - t0));
    const rsrc_t ro = make_rsrc(o + (t0 * nv + h) * static_cast<int64_t>(D),
                                static_cast<uint32_t>(((L - 1) * nv * D + D) * sizeof(TO)));
    if constexpr (sizeof(TO) == 4) {
      bstore16(ro, oo0, make_uint4(__float_as_uint(Ov[0]), __float_as_uint(Ov[1]), __float_as_uint(Ov[2]),
                                   __float_as_uint(Ov[3])));
    } else {
      bstore8(ro, oo0, make_uint2(f32_to_bf16(Ov[0]) | (static_cast<uint32_t>(f32_to_bf16(Ov[1])) << 16),
                                  f32_to_bf16(Ov[2]) | (static_cast<uint32_t>(f32_to_bf16(Ov[3])) << 16)));
    }
  };
  auto masked = [&](const Prefetch& pf, uint4 (&xa)[4]) {
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      xa[s] = and4(pf.x[s], msk[s]);
      xa[2 + s] = and4(pf.x[2 + s], msk[s]);
    }
  };

  // One chunk with `cur`; the loads of chunk cc+2 go into `nxt2` (the set in
  // between is in flight). Three register sets rotate, so nothing is copied
  // between chunks and every load has about two chunks of compute to arrive.
  auto step = [&](int cc, const Prefetch& cur, const Prefetch& nxt, Prefetch& nxt2) {
    const int ln = min(cc + 2, nchunks - 1);   // past the end the last chunk is re-read
    const int buf = cc & 1;
    // masked T or P blocks of this chunk. The k-step 1 blocks of tiles 0 and 1
    // are not loaded (or carry staging loads) but are consumed here on every
    // path (their mask is zero).
    uint4 xa[4];
    masked(cur, xa);
    load_chunk(ln, nxt2, 0);

    // phase 1: X = K S and R = beta v - b X (recurrence side); O of the
    // previous chunk (output side)
    f32x4 Ra = {0.f, 0.f, 0.f, 0.f};
    const int srow = 16 * m + 4 * lg;      // first of this lane's 4 accumulator rows
    if (rec) {
      f32x4 XH = {0.f, 0.f, 0.f, 0.f}, XL = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const bf16x8 a = as_bf16x8(cur.f[s]);
        XL = mfma_bf16(a, as_bf16x8(lds16(SX + SXP + s * BLK_BYTES + lane * 16)), XL);
        XH = mfma_bf16(a, as_bf16x8(lds16(SX + s * BLK_BYTES + lane * 16)), XH);
      }
      const float4 bb = *reinterpret_cast<const float4*>(&SCS[buf][CH + srow]);
      const float4 be = *reinterpret_cast<const float4*>(&SCS[buf][3 * CH + srow]);
      const uint2 vv = *reinterpret_cast<const uint2*>(&VS[buf][(m * 64 + lane) * 4]);
      Ra[0] = be.x * bf16_to_f32(static_cast<uint16_t>(vv.x)) - bb.x * (XH[0] + XL[0]);
      Ra[1] = be.y * bf16_to_f32(static_cast<uint16_t>(vv.x >> 16)) - bb.y * (XH[1] + XL[1]);
      Ra[2] = be.z * bf16_to_f32(static_cast<uint16_t>(vv.y)) - bb.z * (XH[2] + XL[2]);
      Ra[3] = be.w * bf16_to_f32(static_cast<uint16_t>(vv.y >> 16)) - bb.w * (XH[3] + XL[3]);
      put_tile(RX, TXP, m, lane, Ra);
    } else if (cc > 0) {
      out_tile(cc - 1, Pprev);
    }
    __syncthreads();
    load_chunk(ln, nxt2, 1);

    // phase 2: U = R + T_strict R -> U and c U tiles (recurrence side);
    // Y^T = S^T Q^T of this chunk, hi and lo parts of S in two accumulators
    // (output side)
    if (rec) {
      f32x4 U0 = Ra, U1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        if (s == 1 && !two_k) break;
        const bf16x8 ah = as_bf16x8(xa[s]), al = as_bf16x8(xa[2 + s]);
        const bf16x8 bh = as_bf16x8(lds16(RX + s * BLK_BYTES + lane * 16));
        const bf16x8 bl = as_bf16x8(lds16(RX + TXP + s * BLK_BYTES + lane * 16));
        f32x4& Ua = s == 0 ? U0 : U1;
        Ua = mfma_bf16(al, bh, Ua);
        Ua = mfma_bf16(ah, bl, Ua);
        Ua = mfma_bf16(ah, bh, Ua);
      }
      f32x4 Ua, cU;
      const float4 cb = *reinterpret_cast<const float4*>(&SCS[buf][2 * CH + srow]);
      const float cbv[4] = {cb.x, cb.y, cb.z, cb.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        Ua[i] = U0[i] + U1[i];
        cU[i] = cbv[i] * Ua[i];
      }
      put_tile(UX, TXP, m, lane, Ua);
      put_tile(CX, TXP, m, lane, cU);
    } else {
      f32x4 YH = {0.f, 0.f, 0.f, 0.f}, YL = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const bf16x8 a = as_bf16x8(cur.f[s]);
        YL = mfma_bf16(as_bf16x8(lds16(SX + SXP + s * BLK_BYTES + lane * 16)), a, YL);
        YH = mfma_bf16(as_bf16x8(lds16(SX + s * BLK_BYTES + lane * 16)), a, YH);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) Yprev[i] = YH[i] + YL[i];
#pragma unroll
      for (int s = 0; s < 4; ++s) Pprev[s] = xa[s];
    }
    __syncthreads();
    load_chunk(ln, nxt2, 2);

    // phase 3: S_w = e^{G_C} S_w + K[:, rows of w]^T (c U), the two token
    // k-steps in two accumulators
    {
      const float eGC = EGS[buf][0];
      f32x4 S1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < 4; ++i) S[i] *= eGC;
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const bf16x8 a = as_bf16x8(cur.kt[s]);
        const bf16x8 ch = as_bf16x8(lds16(CX + s * BLK_BYTES + lane * 16));
        const bf16x8 cl = as_bf16x8(lds16(CX + TXP + s * BLK_BYTES + lane * 16));
        f32x4& Sa = s == 0 ? S : S1;
        Sa = mfma_bf16(a, cl, Sa);
        Sa = mfma_bf16(a, ch, Sa);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) S[i] += S1[i];
    }
    // publish S for the next chunk (every wave has read S before the barriers above)
    publish_S();
    commit(nxt, buf ^ 1);
    __syncthreads();
  };

  Prefetch pa{}, pb{}, pc{};
  if (nchunks > 0) {
#pragma unroll
    for (int p = 0; p < 3; ++p) {
      load_chunk(0, pa, p);
      load_chunk(min(1, nchunks - 1), pb, p);
    }
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
  if (!rec && nchunks > 0) out_tile(nchunks - 1, Pprev);   // the last chunk's output

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

template <typename TIn>
hipError_t chunk_dispatch(const void* q, const void* k, const void* v, int64_t qs, int64_t ks, int64_t vs,
                          const float* g, const float* beta, const int32_t* cu, int n_seqs, int64_t T, int nk,
                          int nv, float scale, int l2, const float* S0, float* ST, void* o, int o_bf16, void* ws,
                          hipStream_t s) {
  constexpr bool BF = sizeof(TIn) == 2;
  const WsLayout lay = ws_layout(T, n_seqs, nk, nv, BF);
  char* base = static_cast<char*>(ws);
  int32_t* chunk_off = reinterpret_cast<int32_t*>(base + lay.off_chunk_off);
  float* tp = reinterpret_cast<float*>(base + lay.off_tp);
  float4* sc = reinterpret_cast<float4*>(base + lay.off_sc);
  float* egc = reinterpret_cast<float*>(base + lay.off_egc);
  uint16_t* kf = BF ? reinterpret_cast<uint16_t*>(base + lay.off_kf) : nullptr;
  uint16_t* qf = BF ? reinterpret_cast<uint16_t*>(base + lay.off_qf) : nullptr;
  uint16_t* ktf = BF ? reinterpret_cast<uint16_t*>(base + lay.off_ktf) : nullptr;

  const int64_t nch = T / CH + n_seqs;
  hipError_t e = hipSuccess;
  if (cu) {   // varlen chunk table (one sequence needs none)
    chunk_offsets_kernel<<<1, 256, 0, s>>>(cu, n_seqs, T, static_cast<int32_t>(nch), chunk_off);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  {
    auto kern = chunk_prep_kernel<TIn>;
    const size_t lds = prep_lds_bytes<TIn>();
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                            static_cast<int>(lds));
    if (e != hipSuccess) return e;
    kern<<<dim3(static_cast<unsigned>(nv), static_cast<unsigned>(nch)), 64 * PREP_WAVES, lds, s>>>(
        static_cast<const TIn*>(q), static_cast<const TIn*>(k), qs, ks, g, beta, cu, n_seqs, T, nk, nv, scale, l2,
        chunk_off, tp, sc, egc, kf, qf, ktf);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const unsigned grid = static_cast<unsigned>(n_seqs) * nv * (D / 16);
  if constexpr (BF) {
    const uint16_t* xf = reinterpret_cast<const uint16_t*>(tp);
    const float* scp = reinterpret_cast<const float*>(sc);
    const uint16_t* vb = static_cast<const uint16_t*>(v);
    if (o_bf16)
      chunk_state_bf16_kernel<uint16_t><<<grid, 512, 0, s>>>(vb, vs, cu, n_seqs, T, nk, nv, chunk_off, xf, scp, egc,
                                                             kf, qf, ktf, S0, ST, static_cast<uint16_t*>(o));
    else
      chunk_state_bf16_kernel<float><<<grid, 512, 0, s>>>(vb, vs, cu, n_seqs, T, nk, nv, chunk_off, xf, scp, egc,
                                                          kf, qf, ktf, S0, ST, static_cast<float*>(o));
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

size_t chunk_workspace_bytes(int64_t T, int n_seqs, int nk, int nv, int bf16) {
  return ws_layout(T, n_seqs, nk, nv, bf16 != 0).total;
}

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
