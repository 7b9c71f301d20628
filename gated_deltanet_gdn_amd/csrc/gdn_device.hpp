// gdn_device.hpp -- device helpers shared by the gfx950 kernels of libgdn.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

// ---------------------------------------------------------------- bf16 <-> fp32
// bf16 is stored as raw 16-bit words in global memory. Widening is exact;
// narrowing rounds to nearest even (the hardware conversion on gfx950).
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float(static_cast<uint32_t>(h) << 16); }
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  __bf16 b = static_cast<__bf16>(f);
  return __builtin_bit_cast(uint16_t, b);
}

template <typename T> struct Elem;
template <> struct Elem<float> {
  __device__ static __forceinline__ float cvt(float x) { return x; }
  __device__ static __forceinline__ float load(const float* p, int64_t i) { return p[i]; }
  __device__ static __forceinline__ void store(float* p, int64_t i, float v) { p[i] = v; }
};
template <> struct Elem<uint16_t> {
  __device__ static __forceinline__ float cvt(uint16_t x) { return bf16_to_f32(x); }
  __device__ static __forceinline__ float load(const uint16_t* p, int64_t i) { return bf16_to_f32(p[i]); }
  __device__ static __forceinline__ void store(uint16_t* p, int64_t i, float v) { p[i] = f32_to_bf16(v); }
};

// Load 8 consecutive elements (16-byte aligned for bf16, 32-byte for fp32) as fp32.
__device__ __forceinline__ void load8(const uint16_t* p, float (&out)[8]) {
  const uint4 u = *reinterpret_cast<const uint4*>(p);
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    out[2 * i] = __uint_as_float(w[i] << 16);
    out[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}
__device__ __forceinline__ void load8(const float* p, float (&out)[8]) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  out[0] = a.x; out[1] = a.y; out[2] = a.z; out[3] = a.w;
  out[4] = b.x; out[5] = b.y; out[6] = b.z; out[7] = b.w;
}

// ---------------------------------------------------------------- math
// sigmoid and SiLU from e^{-x} = 2^{-x log2(e)} with the hardware 2^x and
// reciprocal (each about 1 ulp); the product -x log2(e) rounds once, so the
// relative error stays below about 1e-6 for |x| < 20 and the results saturate
// correctly (e^{-x} = inf gives sigmoid 0 and SiLU -0). The library's
// elementwise passes are bound by these instructions, not by memory, with the
// correctly rounded expf and division.
__device__ __forceinline__ float exp_(float x) { return __builtin_amdgcn_exp2f(x * 1.4426950408889634f); }
__device__ __forceinline__ float exp_neg_(float x) { return exp_(-x); }
__device__ __forceinline__ float sigmoidf_(float x) { return __builtin_amdgcn_rcpf(1.0f + exp_neg_(x)); }
// log1p(y) for y >= 0 from the hardware log2 and reciprocal: with u = 1 + y
// rounded, log1p(y) = ln(u) * y / (u - 1), or y when u rounds to 1. Dividing
// by the rounded u - 1 cancels the rounding of u (Goldberg, "What Every
// Computer Scientist Should Know About Floating-Point Arithmetic", 1991,
// Theorem 4); with the about-1-ulp log2 and reciprocal the result stays
// within a few ulps.
__device__ __forceinline__ float log1p_pos_(float y) {
  const float u = 1.0f + y;
  const float d = u - 1.0f;
  return d == 0.0f ? y : (__builtin_amdgcn_logf(u) * 0.6931471805599453f) * (y * __builtin_amdgcn_rcpf(d));
}
// log(1 + e^s) without overflow: max(s, 0) + log1p(e^{-|s|}).
__device__ __forceinline__ float softplusf_(float s) { return fmaxf(s, 0.0f) + log1p_pos_(exp_neg_(fabsf(s))); }
__device__ __forceinline__ float siluf_(float x) { return x * __builtin_amdgcn_rcpf(1.0f + exp_neg_(x)); }

// ---------------------------------------------------------------- conv taps
// Element e (0..7) of 8 packed bf16.
__device__ __forceinline__ float bf16_elem(const uint4& u, int e) {
  const uint32_t d = e < 2 ? u.x : e < 4 ? u.y : e < 6 ? u.z : u.w;
  return __uint_as_float((e & 1) ? (d & 0xffff0000u) : (d << 16));
}
// Causal depthwise conv (4 taps) + SiLU of 8 channels of one token from its
// raw bf16 window rows (w[3] the token, w[0] three tokens back), rounded to
// bf16 as a stored conv output is. The bias comes first, then the taps
// oldest first, one fma each: the order of the prefill conv kernel, so both
// give the same bits.
__device__ __forceinline__ void conv4_silu8_bf16(const uint4 (&w)[4], const float (&wt)[4][8], const float (&bs)[8],
                                                 float (&out)[8]) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    float acc = bs[e];
#pragma unroll
    for (int j = 0; j < 4; ++j) acc = fmaf(wt[j][e], bf16_elem(w[j], e), acc);
    out[e] = bf16_to_f32(f32_to_bf16(siluf_(acc)));
  }
}
// 8 bf16 values at stride `stride` elements, packed as a row of 8.
__device__ __forceinline__ uint4 gather8_bf16(const uint16_t* p, int64_t stride) {
  uint32_t d[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    d[i] = static_cast<uint32_t>(p[2 * i * stride]) | (static_cast<uint32_t>(p[(2 * i + 1) * stride]) << 16);
  return make_uint4(d[0], d[1], d[2], d[3]);
}
// 8 fp32 values rounded to bf16 (nearest even) and packed, element 0 lowest.
__device__ __forceinline__ uint4 pack8_bf16(const float (&v)[8]) {
  typedef float f2 __attribute__((ext_vector_type(2)));
  typedef __bf16 b2 __attribute__((ext_vector_type(2)));
  uint32_t d[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) d[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f2{v[2 * i], v[2 * i + 1]}, b2));
  return make_uint4(d[0], d[1], d[2], d[3]);
}

// ---------------------------------------------------------------- wave helpers (wave64)
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// ---------------------------------------------------------------- MFMA fragments
// v_mfma_f32_16x16x32_bf16 (gfx950): per lane, A holds 8 bf16 of one row
// (row = lane % 16, k-slots 8*(lane/16) .. +7), B holds 8 bf16 of one column
// (col = lane % 16, same k-slots), D holds 4 fp32 (rows 4*(lane/16) + i,
// col = lane % 16). v_mfma_f32_16x16x4_f32 uses the same row/col mapping with
// one k-slot per lane (k = lane / 16).
typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef float f32x4 __attribute__((__vector_size__(4 * sizeof(float))));

__device__ __forceinline__ f32x4 mfma_bf16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_f32(float a, float b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 to_bf16x8(const float (&v)[8]) {
  bf16x8 r;
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = static_cast<__bf16>(v[i]);
  return r;
}
// x = hi + lo + O(2^-17 |x|): hi = bf16(x), lo = bf16(x - hi).
__device__ __forceinline__ void split_bf16x8(const float (&v)[8], bf16x8& hi, bf16x8& lo) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const __bf16 h = static_cast<__bf16>(v[i]);
    hi[i] = h;
    lo[i] = static_cast<__bf16>(v[i] - static_cast<float>(h));
  }
}

// Accumulate A(16 x KS) * B(KS x 16) for one k-step, given per-lane operand
// values (KPL = 8 slots for bf16 MFMA, 1 slot for fp32 MFMA). EXACT_A / EXACT_B
// say whether that operand's values are exactly representable in bf16 (raw bf16
// inputs); other operands are split into hi + lo, giving 1, 2 or 3 MFMA passes.
template <bool BF16, bool EXACT_A, bool EXACT_B> struct Mma;

template <bool EA, bool EB> struct Mma<false, EA, EB> {
  static constexpr int KS = 4, KPL = 1;
  __device__ static __forceinline__ void run(f32x4& acc, const float (&a)[1], const float (&b)[1]) {
    acc = mfma_f32(a[0], b[0], acc);
  }
};
template <bool EA, bool EB> struct Mma<true, EA, EB> {
  static constexpr int KS = 32, KPL = 8;
  __device__ static __forceinline__ void run(f32x4& acc, const float (&a)[8], const float (&b)[8]) {
    if constexpr (EA && EB) {
      acc = mfma_bf16(to_bf16x8(a), to_bf16x8(b), acc);
    } else if constexpr (EA) {
      bf16x8 bh, bl;
      split_bf16x8(b, bh, bl);
      const bf16x8 aa = to_bf16x8(a);
      acc = mfma_bf16(aa, bl, acc);
      acc = mfma_bf16(aa, bh, acc);
    } else if constexpr (EB) {
      bf16x8 ah, al;
      split_bf16x8(a, ah, al);
      const bf16x8 bb = to_bf16x8(b);
      acc = mfma_bf16(al, bb, acc);
      acc = mfma_bf16(ah, bb, acc);
    } else {
      bf16x8 ah, al, bh, bl;
      split_bf16x8(a, ah, al);
      split_bf16x8(b, bh, bl);
      acc = mfma_bf16(al, bh, acc);
      acc = mfma_bf16(ah, bl, acc);
      acc = mfma_bf16(ah, bh, acc);
    }
  }
};

// ---------------------------------------------------------------- packed sequences
// Token range [b, e) of sequence n, clamped into [0, T] so that a malformed
// cu_seqlens can give wrong results but never an out-of-range token index.
// cu == nullptr means one sequence of T tokens.
__device__ __forceinline__ void seq_bounds(const int32_t* cu, int n, int64_t T, int64_t& b, int64_t& e) {
  if (!cu) { b = 0; e = T; return; }
  b = min(max(static_cast<int64_t>(cu[n]), int64_t(0)), T);
  e = min(max(static_cast<int64_t>(cu[n + 1]), b), T);
}

// Contractions of length 16 (the blocked triangular inverse): bf16 uses
// v_mfma_f32_16x16x16_bf16 (4 k-slots per lane: 4*(lane/16) .. +3), fp32
// uses v_mfma_f32_16x16x4_f32 four times. Operands split into hi + lo as above.
typedef __bf16 bf16x4 __attribute__((__vector_size__(4 * sizeof(__bf16))));
template <bool BF16, bool EXACT_A, bool EXACT_B> struct Mma16;
template <bool EA, bool EB> struct Mma16<false, EA, EB> : Mma<false, EA, EB> {};
template <bool EA, bool EB> struct Mma16<true, EA, EB> {
  static constexpr int KS = 16, KPL = 4;
  __device__ static __forceinline__ void split4(const float (&v)[4], bf16x4& hi, bf16x4& lo) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const __bf16 h = static_cast<__bf16>(v[i]);
      hi[i] = h;
      lo[i] = static_cast<__bf16>(v[i] - static_cast<float>(h));
    }
  }
  __device__ static __forceinline__ void run(f32x4& acc, const float (&a)[4], const float (&b)[4]) {
    bf16x4 ah, al, bh, bl;
    split4(a, ah, al);
    split4(b, bh, bl);
    if constexpr (EA && EB) {
      acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ah, bh, acc, 0, 0, 0);
    } else if constexpr (EA) {
      acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ah, bl, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ah, bh, acc, 0, 0, 0);
    } else if constexpr (EB) {
      acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(al, bh, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ah, bh, acc, 0, 0, 0);
    } else {
      acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(al, bh, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ah, bl, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ah, bh, acc, 0, 0, 0);
    }
  }
};

// ---------------------------------------------------------------- buffer loads
// Raw buffer loads: a 128-bit resource in SGPRs plus a 32-bit VGPR offset per
// lane. Loads past num_records bytes return 0.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0), bytes, 0x00020000);
}
__device__ __forceinline__ uint4 bload16(rsrc_t r, uint32_t off) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
  return make_uint4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ uint16_t bload2(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
}

__device__ __forceinline__ void bstore4(rsrc_t r, uint32_t off, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), r, off, 0, 0);
}
__device__ __forceinline__ void bstore2(rsrc_t r, uint32_t off, uint16_t v) {
  __builtin_amdgcn_raw_buffer_store_b16(v, r, off, 0, 0);
}
__device__ __forceinline__ void bstore16(rsrc_t r, uint32_t off, uint4 v) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  u32x4 d;
  d.x = v.x; d.y = v.y; d.z = v.z; d.w = v.w;
  __builtin_amdgcn_raw_buffer_store_b128(d, r, off, 0, 0);
}
__device__ __forceinline__ void bstore8(rsrc_t r, uint32_t off, uint2 v) {
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  u32x2 d;
  d.x = v.x; d.y = v.y;
  __builtin_amdgcn_raw_buffer_store_b64(d, r, off, 0, 0);
}
// Non-temporal stores (cache policy bit "nt") for write-once output streams.
__device__ __forceinline__ void bstore16_nt(rsrc_t r, uint32_t off, uint4 v) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  u32x4 d;
  d.x = v.x; d.y = v.y; d.z = v.z; d.w = v.w;
  __builtin_amdgcn_raw_buffer_store_b128(d, r, off, 0, 2);
}
__device__ __forceinline__ void bstore8_nt(rsrc_t r, uint32_t off, uint2 v) {
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  u32x2 d;
  d.x = v.x; d.y = v.y;
  __builtin_amdgcn_raw_buffer_store_b64(d, r, off, 0, 2);
}

// ---------------------------------------------------------------- XCD-aware block order
// Workgroups are dispatched round-robin over the 8 XCDs (block b -> XCD b % 8).
// Remap so that logically consecutive work items land on the same XCD and
// share its L2. Identity when the grid is not a multiple of 8.
__device__ __forceinline__ int xcd_swizzle(int b, int nblocks) {
  if (nblocks % 8 != 0) return b;
  const int per = nblocks / 8;
  return (b % 8) * per + b / 8;
}

}  // namespace gdn
