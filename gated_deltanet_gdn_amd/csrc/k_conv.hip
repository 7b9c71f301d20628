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

template <typename T>
__device__ __forceinline__ void load_vec(const T* p, float (&v)[CPT]) { load8(p, v); }

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

  for (int64_t t = t_begin; t < t_end; ++t) {
    if (t >= s_end) {  // next non-empty sequence starts at t
      while (n + 1 < n_seqs && cu[n + 1] <= t) ++n;
      seq_bounds(cu, n, T_tot, s_begin, s_end);
      history_from_state(st_in, n, C, c0, state_len, win);
    }
    float xv[CPT];
    load_vec(x + t * xs + c0, xv);
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
  if (st_out) {
    const int64_t units = static_cast<int64_t>(n_seqs) * C;
    const dim3 grid(static_cast<unsigned>((units + 255) / 256));
    if (bf16)
      conv_state_out_kernel<uint16_t><<<grid, 256, 0, s>>>(static_cast<const uint16_t*>(x), x_stride, cu, n_seqs,
                                                           T, C, static_cast<const uint16_t*>(st_in),
                                                           static_cast<uint16_t*>(st_out), state_len);
    else
      conv_state_out_kernel<float><<<grid, 256, 0, s>>>(static_cast<const float*>(x), x_stride, cu, n_seqs, T, C,
                                                        static_cast<const float*>(st_in),
                                                        static_cast<float*>(st_out), state_len);
    return hipGetLastError();
  }
  return hipSuccess;
}

hipError_t launch_causal_conv1d_update(const void* x, int bf16, void* state, int state_len, const float* w,
                                       const float* bias, int n_seqs, int C, int silu, void* y, hipStream_t s) {
  const int64_t units = static_cast<int64_t>(n_seqs) * C;
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
