// k_elementwise.hip -- gating and gated RMSNorm (HBM-bound elementwise/row kernels).
//
// Gating follows the beta / g lines of the minimal forward example in
// "Qwen3.5 Dense Model Architecture" (Linear Attention), computed in fp32.
// Gated RMSNorm follows "Qwen3.5 Simulation Support Design Document" 1.1 and
// Appendix B (scale by 1 + weight) with the SiLU(z) gate of its op table (2.2).
#include "gdn_device.hpp"
#include "gdn_internal.hpp"

namespace gdn {
namespace {

// One thread per VEC consecutive (token, head) elements of one token when
// nv % VEC == 0 (VEC = 8 or 4: the inputs arrive as one 16- or 8-byte vector
// load each, the head index is formed once per thread), else one element per
// thread. Bytes per element: 2*sizeof(in) + 8.
template <typename TIn, int VEC>
__device__ __forceinline__ void load_vecn(const TIn* p, float (&v)[VEC]) {
  if constexpr (sizeof(TIn) == 2 && VEC == 8) {
    load8(p, v);
  } else if constexpr (sizeof(TIn) == 2 && VEC == 4) {
    const uint2 u = *reinterpret_cast<const uint2*>(p);
    v[0] = __uint_as_float(u.x << 16); v[1] = __uint_as_float(u.x & 0xffff0000u);
    v[2] = __uint_as_float(u.y << 16); v[3] = __uint_as_float(u.y & 0xffff0000u);
  } else {
#pragma unroll
    for (int q = 0; q < VEC / 4; ++q) {
      const float4 f = *reinterpret_cast<const float4*>(p + 4 * q);
      v[4 * q] = f.x; v[4 * q + 1] = f.y; v[4 * q + 2] = f.z; v[4 * q + 3] = f.w;
    }
  }
}

template <typename TIn, int VEC>
__global__ void __launch_bounds__(256) gating_kernel(const TIn* __restrict__ a, const TIn* __restrict__ b,
                                                     const float* __restrict__ A_log,
                                                     const float* __restrict__ dt_bias, int64_t n,
                                                     int nv, float* __restrict__ g,
                                                     float* __restrict__ beta) {
  const int64_t base = (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) * VEC;
  if (base >= n) return;
  if constexpr (VEC == 1) {
    const int h = static_cast<int>(base % nv);
    const float av = Elem<TIn>::load(a, base);
    const float bv = Elem<TIn>::load(b, base);
    beta[base] = sigmoidf_(bv);
    g[base] = -exp_(A_log[h]) * softplusf_(av + dt_bias[h]);
  } else {
    const int h0 = static_cast<int>(base % nv);   // the VEC elements share one token
    float av[VEC], bv[VEC], gv[VEC], be[VEC];
    load_vecn<TIn, VEC>(a + base, av);
    load_vecn<TIn, VEC>(b + base, bv);
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      be[e] = sigmoidf_(bv[e]);
      gv[e] = -exp_(A_log[h0 + e]) * softplusf_(av[e] + dt_bias[h0 + e]);
    }
#pragma unroll
    for (int q = 0; q < VEC / 4; ++q) {
      *reinterpret_cast<float4*>(beta + base + 4 * q) = make_float4(be[4 * q], be[4 * q + 1], be[4 * q + 2], be[4 * q + 3]);
      *reinterpret_cast<float4*>(g + base + 4 * q) = make_float4(gv[4 * q], gv[4 * q + 1], gv[4 * q + 2], gv[4 * q + 3]);
    }
  }
}

// A half-wave (32 lanes) per row; each lane owns 4 consecutive elements per
// 128-element slab. Rows are independent; one read of x and z, one write of y.
template <typename TX, typename TZ, typename TY>
__global__ void __launch_bounds__(256) gated_rmsnorm_kernel(const TX* __restrict__ x, const TZ* __restrict__ z,
                                                            const float* __restrict__ w, int64_t rows,
                                                            int D, float eps, TY* __restrict__ y) {
  const int lane32 = threadIdx.x & 31;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * 8 + (threadIdx.x >> 5);
  if (row >= rows) return;
  const int64_t off = row * D;
  float ss = 0.0f;
  for (int c = lane32 * 4; c < D; c += 128) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float xv = Elem<TX>::load(x, off + c + e);
      ss = fmaf(xv, xv, ss);
    }
  }
#pragma unroll
  for (int o = 16; o >= 1; o >>= 1) ss += __shfl_xor(ss, o, 32);
  const float inv = 1.0f / sqrtf(ss / static_cast<float>(D) + eps);
  for (int c = lane32 * 4; c < D; c += 128) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float xv = Elem<TX>::load(x, off + c + e);
      const float zv = Elem<TZ>::load(z, off + c + e);
      Elem<TY>::store(y, off + c + e, xv * inv * (1.0f + w[c + e]) * siluf_(zv));
    }
  }
}

template <typename TX, typename TZ>
hipError_t rms_dispatch_y(const void* x, const void* z, const float* w, int64_t rows, int D, float eps,
                          void* y, int y_bf16, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>((rows + 7) / 8));
  if (y_bf16)
    gated_rmsnorm_kernel<TX, TZ, uint16_t><<<grid, 256, 0, s>>>(
        static_cast<const TX*>(x), static_cast<const TZ*>(z), w, rows, D, eps, static_cast<uint16_t*>(y));
  else
    gated_rmsnorm_kernel<TX, TZ, float><<<grid, 256, 0, s>>>(
        static_cast<const TX*>(x), static_cast<const TZ*>(z), w, rows, D, eps, static_cast<float*>(y));
  return hipGetLastError();
}

}  // namespace

template <typename TIn, int VEC>
hipError_t gating_launch(const void* a, const void* b, const float* A_log, const float* dt_bias, int64_t n, int nv,
                         float* g, float* beta, hipStream_t s) {
  const int64_t threads = n / VEC;
  const dim3 grid(static_cast<unsigned>((threads + 255) / 256));
  gating_kernel<TIn, VEC><<<grid, 256, 0, s>>>(static_cast<const TIn*>(a), static_cast<const TIn*>(b), A_log, dt_bias,
                                               n, nv, g, beta);
  return hipGetLastError();
}

template <typename TIn>
hipError_t gating_dispatch(const void* a, const void* b, const float* A_log, const float* dt_bias, int64_t n, int nv,
                           float* g, float* beta, hipStream_t s) {
  // vector accesses need 16-byte aligned tensors (the ABI does not require it)
  const uintptr_t al = reinterpret_cast<uintptr_t>(a) | reinterpret_cast<uintptr_t>(b) |
                       reinterpret_cast<uintptr_t>(g) | reinterpret_cast<uintptr_t>(beta);
  if ((al & 15) == 0) {
    if (nv % 8 == 0) return gating_launch<TIn, 8>(a, b, A_log, dt_bias, n, nv, g, beta, s);
    if (nv % 4 == 0) return gating_launch<TIn, 4>(a, b, A_log, dt_bias, n, nv, g, beta, s);
  }
  return gating_launch<TIn, 1>(a, b, A_log, dt_bias, n, nv, g, beta, s);
}

hipError_t launch_gating(const void* a, const void* b, int bf16, const float* A_log, const float* dt_bias,
                         int64_t T, int nv, float* g, float* beta, hipStream_t s) {
  const int64_t n = T * nv;
  if (n == 0) return hipSuccess;
  return bf16 ? gating_dispatch<uint16_t>(a, b, A_log, dt_bias, n, nv, g, beta, s)
              : gating_dispatch<float>(a, b, A_log, dt_bias, n, nv, g, beta, s);
}

hipError_t launch_gated_rmsnorm(const void* x, int x_bf16, const void* z, int z_bf16, const float* w,
                                int64_t rows, int D, float eps, void* y, int y_bf16, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  if (x_bf16) {
    return z_bf16 ? rms_dispatch_y<uint16_t, uint16_t>(x, z, w, rows, D, eps, y, y_bf16, s)
                  : rms_dispatch_y<uint16_t, float>(x, z, w, rows, D, eps, y, y_bf16, s);
  }
  return z_bf16 ? rms_dispatch_y<float, uint16_t>(x, z, w, rows, D, eps, y, y_bf16, s)
                : rms_dispatch_y<float, float>(x, z, w, rows, D, eps, y, y_bf16, s);
}

}  // namespace gdn
