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

// One thread per 4 consecutive (token, head) elements when nv % 4 == 0,
// else one element per thread. Bytes per element: 2*sizeof(in) + 8.
template <typename TIn, int VEC>
__global__ void __launch_bounds__(256) gating_kernel(const TIn* __restrict__ a, const TIn* __restrict__ b,
                                                     const float* __restrict__ A_log,
                                                     const float* __restrict__ dt_bias, int64_t n,
                                                     int nv, float* __restrict__ g,
                                                     float* __restrict__ beta) {
  const int64_t base = (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) * VEC;
  if (base >= n) return;
#pragma unroll
  for (int e = 0; e < VEC; ++e) {
    const int64_t i = base + e;
    if (VEC > 1 || i < n) {
      const int h = static_cast<int>(i % nv);
      const float av = Elem<TIn>::load(a, i);
      const float bv = Elem<TIn>::load(b, i);
      beta[i] = sigmoidf_(bv);
      g[i] = -expf(A_log[h]) * softplusf_(av + dt_bias[h]);
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

hipError_t launch_gating(const void* a, const void* b, int bf16, const float* A_log, const float* dt_bias,
                         int64_t T, int nv, float* g, float* beta, hipStream_t s) {
  const int64_t n = T * nv;
  if (n == 0) return hipSuccess;
  const bool vec4 = (nv % 4) == 0;
  const int64_t threads = vec4 ? n / 4 : n;
  const dim3 grid(static_cast<unsigned>((threads + 255) / 256));
  if (bf16) {
    if (vec4)
      gating_kernel<uint16_t, 4><<<grid, 256, 0, s>>>(static_cast<const uint16_t*>(a),
                                                      static_cast<const uint16_t*>(b), A_log, dt_bias, n, nv, g, beta);
    else
      gating_kernel<uint16_t, 1><<<grid, 256, 0, s>>>(static_cast<const uint16_t*>(a),
                                                      static_cast<const uint16_t*>(b), A_log, dt_bias, n, nv, g, beta);
  } else {
    if (vec4)
      gating_kernel<float, 4><<<grid, 256, 0, s>>>(static_cast<const float*>(a), static_cast<const float*>(b),
                                                   A_log, dt_bias, n, nv, g, beta);
    else
      gating_kernel<float, 1><<<grid, 256, 0, s>>>(static_cast<const float*>(a), static_cast<const float*>(b),
                                                   A_log, dt_bias, n, nv, g, beta);
  }
  return hipGetLastError();
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
