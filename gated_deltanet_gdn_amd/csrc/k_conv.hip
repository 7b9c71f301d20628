// k_conv.hip -- causal depthwise conv1d (+SiLU): prefill conv body and decode update.
//
// "Qwen3.5 Simulation Support Design Document" 2.4 splits the conv into a body
// (prefill) and a state update (decode); "Qwen3.5 Dense Model Architecture",
// Linear Attention, applies a depthwise Conv1d of kernel size
// linear_conv_kernel_dim to the packed QKV and then SiLU, prepending the cached
// conv state when one exists. Cross-correlation orientation: tap K-1 multiplies
// the newest input.
#include "gdn_device.hpp"
#include "gdn_internal.hpp"

namespace gdn {
namespace {

constexpr int KW = 4;        // conv taps (the only width built)
constexpr int CPT = 8;       // channels per thread (one 16-byte bf16 vector)
constexpr int TB = 64;       // tokens per thread (sliding window in registers)

__device__ __forceinline__ int find_seq(const int32_t* cu, int n_seqs, int64_t t) {
  // largest n with cu[n] <= t (sequences may be empty)
  int lo = 0, hi = n_seqs - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (cu[mid] <= t) lo = mid; else hi = mid - 1;
  }
  return lo;
}

constexpr int UB = 1;        // tokens whose loads are issued together (more measured slower)

template <typename T>
__device__ __forceinline__ void load_vec(const T* p, float (&v)[CPT]) { load8(p, v); }

// CPT elements as raw 16-byte words (1 for bf16, 2 for fp32), converted later
__device__ __forceinline__ void load_raw(const uint16_t* p, uint4 (&r)[1]) { r[0] = *reinterpret_cast<const uint4*>(p); }
__device__ __forceinline__ void load_raw(const float* p, uint4 (&r)[2]) {
  r[0] = *reinterpret_cast<const uint4*>(p);
  r[1] = *reinterpret_cast<const uint4*>(p + 4);
}
__device__ __forceinline__ void unpack_raw(const uint4 (&r)[1], float (&v)[CPT]) {
  const uint32_t w[4] = {r[0].x, r[0].y, r[0].z, r[0].w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(w[i] << 16);
    v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}
__device__ __forceinline__ void unpack_raw(const uint4 (&r)[2], float (&v)[CPT]) {
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    v[4 * h] = __uint_as_float(r[h].x);
    v[4 * h + 1] = __uint_as_float(r[h].y);
    v[4 * h + 2] = __uint_as_float(r[h].z);
    v[4 * h + 3] = __uint_as_float(r[h].w);
  }
}

template <typename T>
__device__ __forceinline__ void store_vec(T* p, const float (&v)[CPT]);
template <>
__device__ __forceinline__ void store_vec<float>(float* p, const float (&v)[CPT]) {
  *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
  *reinterpret_cast<float4*>(p + 4) = make_float4(v[4], v[5], v[6], v[7]);
}
template <>
__device__ __forceinline__ void store_vec<uint16_t>(uint16_t* p, const float (&v)[CPT]) {
  uint4 u;
  u.x = f32_to_bf16(v[0]) | (static_cast<uint32_t>(f32_to_bf16(v[1])) << 16);
  u.y = f32_to_bf16(v[2]) | (static_cast<uint32_t>(f32_to_bf16(v[3])) << 16);
  u.z = f32_to_bf16(v[4]) | (static_cast<uint32_t>(f32_to_bf16(v[5])) << 16);
  u.w = f32_to_bf16(v[6]) | (static_cast<uint32_t>(f32_to_bf16(v[7])) << 16);
  *reinterpret_cast<uint4*>(p) = u;
}

// Window slot j (0..KW-2) holds the input at relative position j-(KW-1), i.e.
// slot KW-2 is the previous token. Fill it for a sequence start from the
// conv state history (its last KW-1 entries) or zeros.
template <typename T>
__device__ __forceinline__ void history_from_state(const T* st_in, int n, int C, int c0, int state_len,
                                                   float (&win)[KW - 1][CPT]) {
#pragma unroll
  for (int j = 0; j < KW - 1; ++j)
#pragma unroll
    for (int e = 0; e < CPT; ++e)
      win[j][e] = st_in ? Elem<T>::load(st_in, (static_cast<int64_t>(n) * C + c0 + e) * state_len +
                                                   (state_len - (KW - 1) + j))
                        : 0.0f;
}

template <typename T>
__global__ void __launch_bounds__(256) causal_conv1d_kernel(const T* __restrict__ x, int64_t xs,
                                                            const float* __restrict__ w,
                                                            const float* __restrict__ bias,
                                                            const int32_t* __restrict__ cu, int n_seqs,
                                                            int64_t T_tot, int C, const T* __restrict__ st_in,
                                                            int state_len, int silu, T* __restrict__ y) {
  const int c0 = (blockIdx.y * blockDim.x + threadIdx.x) * CPT;
  if (c0 >= C) return;
  const int64_t t_begin = static_cast<int64_t>(blockIdx.x) * TB;
  if (t_begin >= T_tot) return;
  const int64_t t_end = min(t_begin + TB, T_tot);

  float wt[KW][CPT], bs[CPT];
#pragma unroll
  for (int e = 0; e < CPT; ++e) {
#pragma unroll
    for (int j = 0; j < KW; ++j) wt[j][e] = w[static_cast<int64_t>(c0 + e) * KW + j];
    bs[e] = bias ? bias[c0 + e] : 0.0f;
  }

  int n = cu ? find_seq(cu, n_seqs, t_begin) : 0;
  int64_t s_begin, s_end;
  seq_bounds(cu, n, T_tot, s_begin, s_end);

  float win[KW - 1][CPT];
  // inputs t_begin-3 .. t_begin-1: from x inside the sequence, else from history
#pragma unroll
  for (int j = 0; j < KW - 1; ++j) {
    const int64_t tt = t_begin - (KW - 1) + j;
    if (tt >= s_begin) {
      load_vec(x + tt * xs + c0, win[j]);
    } else {
      const int p = static_cast<int>(max(tt - s_begin, int64_t(-(KW - 1))));  // -(KW-1) .. -1
#pragma unroll
      for (int e = 0; e < CPT; ++e)
        win[j][e] = st_in ? Elem<T>::load(st_in, (static_cast<int64_t>(n) * C + c0 + e) * state_len + state_len + p)
                          : 0.0f;
    }
  }

  // UB tokens' inputs are loaded before any of them is used, so every wave
  // keeps UB loads in flight (t is uniform over the workgroup: the branches
  // below do not diverge)
  for (int64_t tb = t_begin; tb < t_end; tb += UB) {
    uint4 raw[UB][CPT * sizeof(T) / 16];
#pragma unroll
    for (int u = 0; u < UB; ++u)
      if (tb + u < t_end) load_raw(x + (tb + u) * xs + c0, raw[u]);
#pragma unroll
    for (int u = 0; u < UB; ++u) {
      const int64_t t = tb + u;
      if (t >= t_end) break;
      if (t >= s_end) {  // next non-empty sequence starts at t
        while (n + 1 < n_seqs && cu[n + 1] <= t) ++n;
        seq_bounds(cu, n, T_tot, s_begin, s_end);
        history_from_state(st_in, n, C, c0, state_len, win);
      }
      float xv[CPT];
      unpack_raw(raw[u], xv);
      float out[CPT];
#pragma unroll
      for (int e = 0; e < CPT; ++e) {
        float acc = bs[e];
#pragma unroll
        for (int j = 0; j < KW - 1; ++j) acc = fmaf(wt[j][e], win[j][e], acc);
        acc = fmaf(wt[KW - 1][e], xv[e], acc);
        out[e] = silu ? siluf_(acc) : acc;
      }
      store_vec(y + t * static_cast<int64_t>(C) + c0, out);
#pragma unroll
      for (int e = 0; e < CPT; ++e) {
#pragma unroll
        for (int j = 0; j < KW - 2; ++j) win[j][e] = win[j + 1][e];
        win[KW - 2][e] = xv[e];
      }
    }
  }
}

// conv_state_out[n,c,s] = ext[L + s], ext = concat(state_in[n,c,:] or 0, x[seq n, c]).
template <typename T>
__global__ void __launch_bounds__(256) conv_state_out_kernel(const T* __restrict__ x, int64_t xs,
                                                             const int32_t* __restrict__ cu, int n_seqs,
                                                             int64_t T_tot, int C, const T* __restrict__ st_in,
                                                             T* __restrict__ st_out, int state_len) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= static_cast<int64_t>(n_seqs) * C) return;
  const int n = static_cast<int>(i / C);
  const int c = static_cast<int>(i % C);
  int64_t sb, se;
  seq_bounds(cu, n, T_tot, sb, se);
  const int64_t L = se - sb;
  for (int s = 0; s < state_len; ++s) {
    const int64_t p = L - state_len + s;
    float v;
    if (p >= 0) v = Elem<T>::load(x, (sb + p) * xs + c);
    else v = st_in ? Elem<T>::load(st_in, i * state_len + state_len + p) : 0.0f;
    Elem<T>::store(st_out, i * state_len + s, v);
  }
}

// One thread per (sequence, channel): y = act(bias + w . [state[-3:], x]);
// state <- [state[1:], x] (an exact copy of the stored values).
template <typename T>
__global__ void __launch_bounds__(256) conv_update_kernel(const T* __restrict__ x, T* __restrict__ st,
                                                          int state_len, const float* __restrict__ w,
                                                          const float* __restrict__ bias, int64_t n_units,
                                                          int C, int silu, T* __restrict__ y) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= n_units) return;
  const int c = static_cast<int>(i % C);
  T* sp = st + i * state_len;
  const T xr = x[i];
  float acc = bias ? bias[c] : 0.0f;
#pragma unroll
  for (int j = 0; j < KW - 1; ++j)
    acc = fmaf(w[static_cast<int64_t>(c) * KW + j], Elem<T>::load(sp, state_len - (KW - 1) + j), acc);
  acc = fmaf(w[static_cast<int64_t>(c) * KW + KW - 1], Elem<T>::load(&xr, 0), acc);
  Elem<T>::store(y, i, silu ? siluf_(acc) : acc);
  for (int s = 0; s + 1 < state_len; ++s) sp[s] = sp[s + 1];
  sp[state_len - 1] = xr;
}

// The same update for state_len == K - 1, one thread per (sequence, 8
// channels): x, the 8 x 3 state entries (contiguous) and the 8 x 4 weights
// move as 16-byte vectors. Same per-channel arithmetic as above.
template <typename T>
__global__ void __launch_bounds__(256) conv_update_vec_kernel(const T* __restrict__ x, T* __restrict__ st,
                                                              const float* __restrict__ w,
                                                              const float* __restrict__ bias, int64_t n_vec, int C,
                                                              int silu, T* __restrict__ y) {
  constexpr int SL = KW - 1;
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;   // (sequence, 8 channels)
  if (i >= n_vec) return;
  const int64_t e0 = i * CPT;                  // first (sequence, channel) element
  const int c0 = static_cast<int>(e0 % C);
  float xv[CPT], sv[CPT * SL], wv[CPT * KW], bv[CPT];
  load_vec(x + e0, xv);
#pragma unroll
  for (int q = 0; q < SL; ++q) {
    float t8[CPT];
    load_vec(st + e0 * SL + q * CPT, t8);
#pragma unroll
    for (int e = 0; e < CPT; ++e) sv[q * CPT + e] = t8[e];
  }
#pragma unroll
  for (int q = 0; q < CPT * KW / 4; ++q) {
    const float4 f = *reinterpret_cast<const float4*>(w + static_cast<int64_t>(c0) * KW + 4 * q);
    wv[4 * q] = f.x; wv[4 * q + 1] = f.y; wv[4 * q + 2] = f.z; wv[4 * q + 3] = f.w;
  }
#pragma unroll
  for (int e = 0; e < CPT; ++e) bv[e] = bias ? bias[c0 + e] : 0.0f;
  float out[CPT], ns[CPT * SL];
#pragma unroll
  for (int e = 0; e < CPT; ++e) {
    float acc = bv[e];
#pragma unroll
    for (int j = 0; j < SL; ++j) acc = fmaf(wv[e * KW + j], sv[e * SL + j], acc);
    acc = fmaf(wv[e * KW + KW - 1], xv[e], acc);
    out[e] = silu ? siluf_(acc) : acc;
#pragma unroll
    for (int j = 0; j + 1 < SL; ++j) ns[e * SL + j] = sv[e * SL + j + 1];
    ns[e * SL + SL - 1] = xv[e];
  }
  store_vec(y + e0, out);
#pragma unroll
  for (int q = 0; q < SL; ++q) {
    float t8[CPT];
#pragma unroll
    for (int e = 0; e < CPT; ++e) t8[e] = ns[q * CPT + e];
    store_vec(st + e0 * SL + q * CPT, t8);
  }
}

}  // namespace

hipError_t launch_causal_conv1d(const void* x, int bf16, int64_t x_stride, const float* w, const float* bias,
                                const int32_t* cu, int n_seqs, int64_t T, int C, const void* st_in,
                                void* st_out, int state_len, int silu, void* y, hipStream_t s) {
  if (T > 0) {
    const dim3 grid(static_cast<unsigned>((T + TB - 1) / TB), static_cast<unsigned>((C / CPT + 255) / 256));
    if (bf16)
      causal_conv1d_kernel<uint16_t><<<grid, 256, 0, s>>>(
          static_cast<const uint16_t*>(x), x_stride, w, bias, cu, n_seqs, T, C,
          static_cast<const uint16_t*>(st_in), state_len, silu, static_cast<uint16_t*>(y));
    else
      causal_conv1d_kernel<float><<<grid, 256, 0, s>>>(static_cast<const float*>(x), x_stride, w, bias, cu,
                                                       n_seqs, T, C, static_cast<const float*>(st_in),
                                                       state_len, silu, static_cast<float*>(y));
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (st_out) return launch_conv_state_out(x, bf16, x_stride, cu, n_seqs, T, C, st_in, st_out, state_len, s);
  return hipSuccess;
}

hipError_t launch_conv_state_out(const void* x, int bf16, int64_t x_stride, const int32_t* cu, int n_seqs,
                                 int64_t T, int C, const void* st_in, void* st_out, int state_len, hipStream_t s) {
  const int64_t units = static_cast<int64_t>(n_seqs) * C;
  const dim3 grid(static_cast<unsigned>((units + 255) / 256));
  if (bf16)
    conv_state_out_kernel<uint16_t><<<grid, 256, 0, s>>>(static_cast<const uint16_t*>(x), x_stride, cu, n_seqs, T,
                                                         C, static_cast<const uint16_t*>(st_in),
                                                         static_cast<uint16_t*>(st_out), state_len);
  else
    conv_state_out_kernel<float><<<grid, 256, 0, s>>>(static_cast<const float*>(x), x_stride, cu, n_seqs, T, C,
                                                      static_cast<const float*>(st_in), static_cast<float*>(st_out),
                                                      state_len);
  return hipGetLastError();
}

hipError_t launch_causal_conv1d_update(const void* x, int bf16, void* state, int state_len, const float* w,
                                       const float* bias, int n_seqs, int C, int silu, void* y, hipStream_t s) {
  const int64_t units = static_cast<int64_t>(n_seqs) * C;
  const uintptr_t al = reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(state) |
                       reinterpret_cast<uintptr_t>(y) | reinterpret_cast<uintptr_t>(w);
  if (state_len == KW - 1 && C % CPT == 0 && (al & 15) == 0) {
    const int64_t nvec = units / CPT;
    const dim3 grid(static_cast<unsigned>((nvec + 255) / 256));
    if (bf16)
      conv_update_vec_kernel<uint16_t><<<grid, 256, 0, s>>>(static_cast<const uint16_t*>(x),
                                                            static_cast<uint16_t*>(state), w, bias, nvec, C, silu,
                                                            static_cast<uint16_t*>(y));
    else
      conv_update_vec_kernel<float><<<grid, 256, 0, s>>>(static_cast<const float*>(x), static_cast<float*>(state), w,
                                                         bias, nvec, C, silu, static_cast<float*>(y));
    return hipGetLastError();
  }
  const dim3 grid(static_cast<unsigned>((units + 255) / 256));
  if (bf16)
    conv_update_kernel<uint16_t><<<grid, 256, 0, s>>>(static_cast<const uint16_t*>(x),
                                                      static_cast<uint16_t*>(state), state_len, w, bias, units,
                                                      C, silu, static_cast<uint16_t*>(y));
  else
    conv_update_kernel<float><<<grid, 256, 0, s>>>(static_cast<const float*>(x), static_cast<float*>(state),
                                                   state_len, w, bias, units, C, silu, static_cast<float*>(y));
  return hipGetLastError();
}

}  // namespace gdn
