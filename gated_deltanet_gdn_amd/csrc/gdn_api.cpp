// gdn_api.cpp -- the C ABI of libgdn.so (declared in include/gdn.h).
//
// Every entry point validates its arguments on the host first and returns a
// status without touching the HIP runtime when they are invalid, so the
// error paths are testable on a machine without a GPU. Valid calls enqueue
// kernels on the caller's stream and return without synchronising.
#include "gdn.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <string>

#include "gdn_internal.hpp"

namespace {

thread_local std::string g_last_error;

int fail(int status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

int ok() {
  g_last_error.clear();
  return GDN_OK;
}

int launched(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(GDN_ERR_LAUNCH, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }
bool valid_dtype(int d) { return d == GDN_F32 || d == GDN_BF16; }
size_t dsize(int d) { return d == GDN_BF16 ? 2 : 4; }

// Shared checks of the two delta-rule entry points.
int check_core(const char* fn, const void* q, const void* k, const void* v, int in_dtype, int64_t& qs,
               int64_t& ks, int64_t& vs, const float* g, const float* beta, int n_seqs, int64_t T, int nk, int nv,
               int dk, int dv, const void* o, int o_dtype) {
  if (!valid_dtype(in_dtype)) return fail(GDN_ERR_INVALID_ARGUMENT, "%s: in_dtype %d is not f32/bf16", fn, in_dtype);
  if (!valid_dtype(o_dtype)) return fail(GDN_ERR_INVALID_ARGUMENT, "%s: o_dtype %d is not f32/bf16", fn, o_dtype);
  if (n_seqs <= 0) return fail(GDN_ERR_INVALID_ARGUMENT, "%s: n_seqs must be >= 1 (got %d)", fn, n_seqs);
  if (T < 0) return fail(GDN_ERR_INVALID_ARGUMENT, "%s: T_tot must be >= 0", fn);
  if (nk <= 0 || nv <= 0) return fail(GDN_ERR_INVALID_ARGUMENT, "%s: head counts must be positive", fn);
  if (nv % nk != 0)
    return fail(GDN_ERR_INVALID_ARGUMENT, "%s: nv (%d) must be a multiple of nk (%d)", fn, nv, nk);
  if (dk <= 0 || dv <= 0) return fail(GDN_ERR_INVALID_ARGUMENT, "%s: head dims must be positive", fn);
  if (dk != 128 || dv != 128)
    return fail(GDN_ERR_UNSUPPORTED, "%s: only dk = dv = 128 is built (got %d, %d)", fn, dk, dv);
  if (T > INT32_MAX) return fail(GDN_ERR_UNSUPPORTED, "%s: T_tot above 2^31-1", fn);
  if (qs == 0) qs = static_cast<int64_t>(nk) * dk;
  if (ks == 0) ks = static_cast<int64_t>(nk) * dk;
  if (vs == 0) vs = static_cast<int64_t>(nv) * dv;
  if (qs < static_cast<int64_t>(nk) * dk || ks < static_cast<int64_t>(nk) * dk || vs < static_cast<int64_t>(nv) * dv)
    return fail(GDN_ERR_INVALID_ARGUMENT, "%s: a token stride is smaller than one token's row", fn);
  // chunk rows are addressed through 32-bit buffer offsets (64 rows of a stride)
  constexpr int64_t kMaxStride = int64_t(1) << 24;
  if (qs > kMaxStride || ks > kMaxStride || vs > kMaxStride)
    return fail(GDN_ERR_UNSUPPORTED, "%s: token strides above 2^24 elements are not supported", fn);
  if (T > 0) {
    if (!q || !k || !v || !g || !beta || !o)
      return fail(GDN_ERR_INVALID_ARGUMENT, "%s: q, k, v, g, beta and o are required", fn);
    if (qs % 8 || ks % 8 || vs % 8)
      return fail(GDN_ERR_UNSUPPORTED, "%s: token strides must be multiples of 8 elements", fn);
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16))
      return fail(GDN_ERR_UNSUPPORTED, "%s: q, k, v, o must be 16-byte aligned", fn);
  }
  return GDN_OK;
}

// One dispatch holds at most 2^32 - 1 work-items and 2^31 - 1 workgroups in
// its one-dimensional grid.
bool grid_fits(int64_t blocks, int64_t threads) {
  return blocks <= INT32_MAX && blocks * threads <= static_cast<int64_t>(UINT32_MAX);
}

// The chunk kernels launch 256 threads per (chunk slot, value head) and per
// (sequence, value head, 16 columns), in one-dimensional grids.
int check_chunk_grid(const char* fn, int64_t T, int n_seqs, int nv) {
  const int64_t slots = T / 64 + n_seqs;
  if (!grid_fits(slots * nv, 256) || !grid_fits(static_cast<int64_t>(n_seqs) * nv * 8, 256))
    return fail(GDN_ERR_UNSUPPORTED, "%s: too many (chunk, head) units for one launch", fn);
  return GDN_OK;
}

// Checks shared by the two entry points of the chunked rule with the gating
// folded in; qs, ks, vs and scale come back resolved (0 = dense, <= 0 = dk^-1/2).
int check_chunk_gated(const char* fn, const void* q, const void* k, const void* v, int in_dtype, int64_t& qs,
                      int64_t& ks, int64_t& vs, const void* a, const void* b, int ab_dtype, const float* A_log,
                      const float* dt_bias, const int32_t* cu_seqlens, int n_seqs, int64_t T_tot, int nk, int nv,
                      int dk, int dv, float& scale, const void* o, int o_dtype) {
  if (!valid_dtype(ab_dtype)) return fail(GDN_ERR_INVALID_ARGUMENT, "%s: ab_dtype %d is not f32/bf16", fn, ab_dtype);
  // a and b stand where g and beta stand in the shared checks
  const int st = check_core(fn, q, k, v, in_dtype, qs, ks, vs, static_cast<const float*>(a),
                            static_cast<const float*>(b), n_seqs, T_tot, nk, nv, dk, dv, o, o_dtype);
  if (st != GDN_OK) return st;
  if (!A_log || !dt_bias) return fail(GDN_ERR_INVALID_ARGUMENT, "%s: A_log and dt_bias are required", fn);
  if (!cu_seqlens && n_seqs != 1) return fail(GDN_ERR_INVALID_ARGUMENT, "%s: cu_seqlens is required when n_seqs > 1", fn);
  if (const int gst = check_chunk_grid(fn, T_tot, n_seqs, nv); gst != GDN_OK) return gst;
  if (!(scale > 0.0f)) scale = 1.0f / sqrtf(static_cast<float>(dk));
  return GDN_OK;
}

}  // namespace

extern "C" {

int gdn_abi_version(void) { return GDN_ABI_VERSION; }

const char* gdn_status_string(int status) {
  switch (status) {
    case GDN_OK: return "GDN_OK";
    case GDN_ERR_INVALID_ARGUMENT: return "GDN_ERR_INVALID_ARGUMENT";
    case GDN_ERR_UNSUPPORTED: return "GDN_ERR_UNSUPPORTED";
    case GDN_ERR_WORKSPACE_TOO_SMALL: return "GDN_ERR_WORKSPACE_TOO_SMALL";
    case GDN_ERR_LAUNCH: return "GDN_ERR_LAUNCH";
    default: return "GDN_ERR_UNKNOWN";
  }
}

const char* gdn_last_error(void) { return g_last_error.c_str(); }

int gdn_gating(const void* a, const void* b, int ab_dtype, const float* A_log, const float* dt_bias, int64_t T_tot,
               int nv, float* g, float* beta, void* stream) {
  if (!valid_dtype(ab_dtype)) return fail(GDN_ERR_INVALID_ARGUMENT, "gdn_gating: ab_dtype %d is not f32/bf16", ab_dtype);
  if (T_tot < 0 || nv <= 0) return fail(GDN_ERR_INVALID_ARGUMENT, "gdn_gating: need T_tot >= 0 and nv > 0");
  if (!A_log || !dt_bias) return fail(GDN_ERR_INVALID_ARGUMENT, "gdn_gating: A_log and dt_bias are required");
  if (T_tot > 0 && (!a || !b || !g || !beta))
    return fail(GDN_ERR_INVALID_ARGUMENT, "gdn_gating: a, b, g and beta are required");
  if (T_tot == 0) return ok();
  if (!grid_fits((T_tot * nv + 255) / 256, 256))
    return fail(GDN_ERR_UNSUPPORTED, "gdn_gating: too many (token, head) elements for one launch");
  return launched(gdn::launch_gating(a, b, ab_dtype == GDN_BF16, A_log, dt_bias, T_tot, nv, g, beta,
                                     static_cast<hipStream_t>(stream)),
                  "gdn_gating");
}

size_t gdn_chunk_fwd_workspace_size(int64_t T_tot, int n_seqs, int nk, int nv, int dk, int dv, int in_dtype) {
  (void)dk; (void)dv;
  if (T_tot < 0 || n_seqs <= 0 || nk <= 0 || nv <= 0) return 0;
  return gdn::chunk_workspace_bytes(T_tot, n_seqs, nk, nv, in_dtype == GDN_BF16);
}

int gdn_chunk_fwd(const void* q, const void* k, const void* v, int in_dtype, int64_t q_tok_stride,
                  int64_t k_tok_stride, int64_t v_tok_stride, const float* g, const float* beta,
                  const int32_t* cu_seqlens, int n_seqs, int64_t T_tot, int nk, int nv, int dk, int dv, float scale,
                  int qk_l2norm, const float* initial_state, float* final_state, void* o, int o_dtype,
                  void* workspace, size_t workspace_bytes, void* stream) {
  const char* fn = "gdn_chunk_fwd";
  int64_t qs = q_tok_stride, ks = k_tok_stride, vs = v_tok_stride;
  const int st = check_core(fn, q, k, v, in_dtype, qs, ks, vs, g, beta, n_seqs, T_tot, nk, nv, dk, dv, o, o_dtype);
  if (st != GDN_OK) return st;
  if (!cu_seqlens && n_seqs != 1) return fail(GDN_ERR_INVALID_ARGUMENT, "%s: cu_seqlens is required when n_seqs > 1", fn);
  if (!workspace) return fail(GDN_ERR_INVALID_ARGUMENT, "%s: workspace is required", fn);
  if (!aligned(workspace, 256)) return fail(GDN_ERR_INVALID_ARGUMENT, "%s: workspace must be 256-byte aligned", fn);
  if (const int gst = check_chunk_grid(fn, T_tot, n_seqs, nv); gst != GDN_OK) return gst;
  const size_t need = gdn::chunk_workspace_bytes(T_tot, n_seqs, nk, nv, in_dtype == GDN_BF16);
  if (workspace_bytes < need)
    return fail(GDN_ERR_WORKSPACE_TOO_SMALL, "%s: workspace of %zu bytes, need %zu", fn, workspace_bytes, need);
  if (!(scale > 0.0f)) scale = 1.0f / sqrtf(static_cast<float>(dk));
  return launched(gdn::launch_chunk_fwd(q, k, v, in_dtype == GDN_BF16, qs, ks, vs, g, beta, 0, nullptr, nullptr,
                                        cu_seqlens, n_seqs, T_tot, nk, nv, scale, qk_l2norm != 0, initial_state,
                                        final_state, o, o_dtype == GDN_BF16, workspace,
                                        static_cast<hipStream_t>(stream)),
                  fn);
}

int gdn_chunk_fwd_gated(const void* q, const void* k, const void* v, int in_dtype, int64_t q_tok_stride,
                        int64_t k_tok_stride, int64_t v_tok_stride, const void* a, const void* b, int ab_dtype,
                        const float* A_log, const float* dt_bias, const int32_t* cu_seqlens, int n_seqs,
                        int64_t T_tot, int nk, int nv, int dk, int dv, float scale, int qk_l2norm,
                        const float* initial_state, float* final_state, void* o, int o_dtype, void* workspace,
                        size_t workspace_bytes, void* stream) {
  const char* fn = "gdn_chunk_fwd_gated";
  int64_t qs = q_tok_stride, ks = k_tok_stride, vs = v_tok_stride;
  const int st = check_chunk_gated(fn, q, k, v, in_dtype, qs, ks, vs, a, b, ab_dtype, A_log, dt_bias, cu_seqlens,
                                   n_seqs, T_tot, nk, nv, dk, dv, scale, o, o_dtype);
  if (st != GDN_OK) return st;
  if (!workspace) return fail(GDN_ERR_INVALID_ARGUMENT, "%s: workspace is required", fn);
  if (!aligned(workspace, 256)) return fail(GDN_ERR_INVALID_ARGUMENT, "%s: workspace must be 256-byte aligned", fn);
  const size_t need = gdn::chunk_workspace_bytes(T_tot, n_seqs, nk, nv, in_dtype == GDN_BF16);
  if (workspace_bytes < need)
    return fail(GDN_ERR_WORKSPACE_TOO_SMALL, "%s: workspace of %zu bytes, need %zu", fn, workspace_bytes, need);
  return launched(gdn::launch_chunk_fwd(q, k, v, in_dtype == GDN_BF16, qs, ks, vs, a, b, ab_dtype == GDN_BF16 ? 1 : 2,
                                        A_log, dt_bias, cu_seqlens, n_seqs, T_tot, nk, nv, scale, qk_l2norm != 0,
                                        initial_state, final_state, o, o_dtype == GDN_BF16, workspace,
                                        static_cast<hipStream_t>(stream)),
                  fn);
}

size_t gdn_chunk_fwd_noalloc_max_bytes(void) { return gdn::kNoallocScratchBytes; }

int gdn_chunk_fwd_gated_noalloc(const void* q, const void* k, const void* v, int in_dtype, int64_t q_tok_stride,
                                int64_t k_tok_stride, int64_t v_tok_stride, const void* a, const void* b,
                                int ab_dtype, const float* A_log, const float* dt_bias, const int32_t* cu_seqlens,
                                int n_seqs, int64_t T_tot, int nk, int nv, int dk, int dv, float scale,
                                int qk_l2norm, const float* initial_state, float* final_state, void* o,
                                int o_dtype, void* stream) {
  const char* fn = "gdn_chunk_fwd_gated_noalloc";
  int64_t qs = q_tok_stride, ks = k_tok_stride, vs = v_tok_stride;
  const int st = check_chunk_gated(fn, q, k, v, in_dtype, qs, ks, vs, a, b, ab_dtype, A_log, dt_bias, cu_seqlens,
                                   n_seqs, T_tot, nk, nv, dk, dv, scale, o, o_dtype);
  if (st != GDN_OK) return st;
  const size_t need = gdn::chunk_workspace_bytes(T_tot, n_seqs, nk, nv, in_dtype == GDN_BF16);
  if (need > gdn::kNoallocScratchBytes)
    return fail(GDN_ERR_WORKSPACE_TOO_SMALL,
                "%s: this call needs %zu bytes of scratch, above the %zu bytes the library holds per device; "
                "use gdn_chunk_fwd_gated with a caller-allocated workspace",
                fn, need, gdn::kNoallocScratchBytes);
  return launched(gdn::launch_chunk_fwd_noalloc(q, k, v, in_dtype == GDN_BF16, qs, ks, vs, a, b,
                                                ab_dtype == GDN_BF16 ? 1 : 2, A_log, dt_bias, cu_seqlens, n_seqs,
                                                T_tot, nk, nv, scale, qk_l2norm != 0, initial_state, final_state, o,
                                                o_dtype == GDN_BF16, static_cast<hipStream_t>(stream)),
                  fn);
}

}  // extern "C"

namespace {
// gdn_prefill_fused and gdn_prefill_fused_norm: the same checks and launches;
// ne (the norm epilogue) is null for the former.
int prefill_fused_impl(const char* fn, const void* x, int dtype, int64_t x_tok_stride, const float* conv_weight,
                       const float* conv_bias, int K, const void* conv_state_in, void* conv_state_out, int state_len,
                       const void* a, const void* b, int ab_dtype, const float* A_log, const float* dt_bias,
                       const int32_t* cu_seqlens, int n_seqs, int64_t T_tot, int nk, int nv, int dk, int dv,
                       float scale, int qk_l2norm, const float* initial_state, float* final_state, void* o,
                       int o_dtype, const gdn::NormEpi* ne, void* workspace, size_t workspace_bytes, void* stream) {
  if (!valid_dtype(dtype)) return fail(GDN_ERR_INVALID_ARGUMENT, "%s: dtype %d is not f32/bf16", fn, dtype);
  if (dtype != GDN_BF16) return fail(GDN_ERR_UNSUPPORTED, "%s: only bf16 x is built", fn);
  if (!valid_dtype(ab_dtype)) return fail(GDN_ERR_INVALID_ARGUMENT, "%s: ab_dtype %d is not f32/bf16", fn, ab_dtype);
  if (K <= 0) return fail(GDN_ERR_INVALID_ARGUMENT, "%s: K must be positive", fn);
  if (state_len < K - 1) return fail(GDN_ERR_INVALID_ARGUMENT, "%s: state_len (%d) < K - 1", fn, state_len);
  if (K != 4) return fail(GDN_ERR_UNSUPPORTED, "%s: only K = 4 is built (got %d)", fn, K);
  if (nk <= 0 || nv <= 0 || dk <= 0 || dv <= 0)
    return fail(GDN_ERR_INVALID_ARGUMENT, "%s: head counts and dims must be positive", fn);
  const int64_t conv_dim = 2 * static_cast<int64_t>(nk) * dk + static_cast<int64_t>(nv) * dv;
  if (x_tok_stride == 0) x_tok_stride = conv_dim;
  if (x_tok_stride < conv_dim) return fail(GDN_ERR_INVALID_ARGUMENT, "%s: x token stride smaller than conv_dim", fn);
  // q, k, v are the views of x at channel offsets 0, nk dk and 2 nk dk
  const uint16_t* xb = static_cast<const uint16_t*>(x);
  const void* qv = xb;
  const void* kv = xb ? xb + static_cast<int64_t>(nk) * dk : nullptr;
  const void* vv = xb ? xb + 2 * static_cast<int64_t>(nk) * dk : nullptr;
  int64_t qs = x_tok_stride, ks = x_tok_stride, vs = x_tok_stride;
  const int st = check_core(fn, qv, kv, vv, dtype, qs, ks, vs, static_cast<const float*>(a),
                            static_cast<const float*>(b), n_seqs, T_tot, nk, nv, dk, dv, o, o_dtype);
  if (st != GDN_OK) return st;
  if (!conv_weight) return fail(GDN_ERR_INVALID_ARGUMENT, "%s: conv_weight is required", fn);
  if (!A_log || !dt_bias) return fail(GDN_ERR_INVALID_ARGUMENT, "%s: A_log and dt_bias are required", fn);
  if (!cu_seqlens && n_seqs != 1) return fail(GDN_ERR_INVALID_ARGUMENT, "%s: cu_seqlens is required when n_seqs > 1", fn);
  if (!workspace) return fail(GDN_ERR_INVALID_ARGUMENT, "%s: workspace is required", fn);
  if (!aligned(workspace, 256)) return fail(GDN_ERR_INVALID_ARGUMENT, "%s: workspace must be 256-byte aligned", fn);
  if (const int gst = check_chunk_grid(fn, T_tot, n_seqs, nv); gst != GDN_OK) return gst;
  if (ne && !grid_fits((T_tot * nv + 7) / 8, 256))
    return fail(GDN_ERR_UNSUPPORTED, "%s: too many rows for one launch", fn);
  const size_t need = gdn::chunk_workspace_bytes(T_tot, n_seqs, nk, nv, 1);
  if (workspace_bytes < need)
    return fail(GDN_ERR_WORKSPACE_TOO_SMALL, "%s: workspace of %zu bytes, need %zu", fn, workspace_bytes, need);
  if (conv_state_out && !grid_fits((static_cast<int64_t>(n_seqs) * conv_dim + 255) / 256, 256))
    return fail(GDN_ERR_UNSUPPORTED, "%s: too many (seq, channel) units for one launch", fn);
  if (conv_state_in && conv_state_out) {
    const size_t bytes = static_cast<size_t>(n_seqs) * conv_dim * state_len * 2;
    const char* a0 = static_cast<const char*>(conv_state_in);
    const char* b0 = static_cast<const char*>(conv_state_out);
    if (a0 < b0 + bytes && b0 < a0 + bytes)
      return fail(GDN_ERR_INVALID_ARGUMENT, "%s: conv_state_out must not overlap conv_state_in", fn);
  }
  if (!(scale > 0.0f)) scale = 1.0f / sqrtf(static_cast<float>(dk));
  const hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = gdn::launch_chunk_fwd_conv(x, x_tok_stride, conv_weight, conv_bias, conv_state_in, state_len, a, b,
                                            ab_dtype == GDN_BF16 ? 1 : 2, A_log, dt_bias, cu_seqlens, n_seqs, T_tot,
                                            nk, nv, scale, qk_l2norm != 0, initial_state, final_state, o,
                                            o_dtype == GDN_BF16, workspace, ne, s);
  if (e == hipSuccess && conv_state_out)   // after the chunk kernels, which read conv_state_in
    e = gdn::launch_conv_state_out(x, 1, x_tok_stride, cu_seqlens, n_seqs, T_tot, static_cast<int>(conv_dim),
                                   conv_state_in, conv_state_out, state_len, s);
  return launched(e, fn);
}
}  // namespace

extern "C" {

int gdn_prefill_fused(const void* x, int dtype, int64_t x_tok_stride, const float* conv_weight,
                      const float* conv_bias, int K, const void* conv_state_in, void* conv_state_out, int state_len,
                      const void* a, const void* b, int ab_dtype, const float* A_log, const float* dt_bias,
                      const int32_t* cu_seqlens, int n_seqs, int64_t T_tot, int nk, int nv, int dk, int dv,
                      float scale, int qk_l2norm, const float* initial_state, float* final_state, void* o,
                      int o_dtype, void* workspace, size_t workspace_bytes, void* stream) {
  return prefill_fused_impl("gdn_prefill_fused", x, dtype, x_tok_stride, conv_weight, conv_bias, K, conv_state_in,
                            conv_state_out, state_len, a, b, ab_dtype, A_log, dt_bias, cu_seqlens, n_seqs, T_tot, nk,
                            nv, dk, dv, scale, qk_l2norm, initial_state, final_state, o, o_dtype, nullptr, workspace,
                            workspace_bytes, stream);
}

int gdn_prefill_fused_norm(const void* x, int dtype, int64_t x_tok_stride, const float* conv_weight,
                           const float* conv_bias, int K, const void* conv_state_in, void* conv_state_out,
                           int state_len, const void* a, const void* b, int ab_dtype, const float* A_log,
                           const float* dt_bias, const int32_t* cu_seqlens, int n_seqs, int64_t T_tot, int nk, int nv,
                           int dk, int dv, float scale, int qk_l2norm, const float* initial_state, float* final_state,
                           const void* z, int z_dtype, const float* norm_weight, float eps, float* y,
                           void* workspace, size_t workspace_bytes, void* stream) {
  const char* fn = "gdn_prefill_fused_norm";
  if (!valid_dtype(z_dtype)) return fail(GDN_ERR_INVALID_ARGUMENT, "%s: z_dtype %d is not f32/bf16", fn, z_dtype);
  if (z_dtype != GDN_BF16) return fail(GDN_ERR_UNSUPPORTED, "%s: only bf16 z is built", fn);
  if (!norm_weight) return fail(GDN_ERR_INVALID_ARGUMENT, "%s: norm_weight is required", fn);
  if (!(eps >= 0.0f)) return fail(GDN_ERR_INVALID_ARGUMENT, "%s: eps must be >= 0", fn);
  if (T_tot > 0 && !z) return fail(GDN_ERR_INVALID_ARGUMENT, "%s: z is required", fn);
  if (z && !aligned(z, 16)) return fail(GDN_ERR_UNSUPPORTED, "%s: z must be 16-byte aligned", fn);
  const gdn::NormEpi ne{static_cast<const uint16_t*>(z), norm_weight, eps};
  return prefill_fused_impl(fn, x, dtype, x_tok_stride, conv_weight, conv_bias, K, conv_state_in, conv_state_out,
                            state_len, a, b, ab_dtype, A_log, dt_bias, cu_seqlens, n_seqs, T_tot, nk, nv, dk, dv,
                            scale, qk_l2norm, initial_state, final_state, y, GDN_F32, &ne, workspace,
                            workspace_bytes, stream);
}

int gdn_recurrent_fwd(const void* q, const void* k, const void* v, int in_dtype, int64_t q_tok_stride,
                      int64_t k_tok_stride, int64_t v_tok_stride, const float* g, const float* beta,
                      const int32_t* cu_seqlens, int n_seqs, int64_t T_tot, int nk, int nv, int dk, int dv,
                      float scale, int qk_l2norm, float* state, void* o, int o_dtype, void* stream) {
  const char* fn = "gdn_recurrent_fwd";
  int64_t qs = q_tok_stride, ks = k_tok_stride, vs = v_tok_stride;
  const int st = check_core(fn, q, k, v, in_dtype, qs, ks, vs, g, beta, n_seqs, T_tot, nk, nv, dk, dv, o, o_dtype);
  if (st != GDN_OK) return st;
  if (!state) return fail(GDN_ERR_INVALID_ARGUMENT, "%s: state is required", fn);
  if (!aligned(state, 16)) return fail(GDN_ERR_UNSUPPORTED, "%s: state must be 16-byte aligned", fn);
  if (!cu_seqlens && T_tot != n_seqs)
    return fail(GDN_ERR_INVALID_ARGUMENT, "%s: without cu_seqlens T_tot must equal n_seqs (one token each)", fn);
  // 256 threads per (sequence, value head) state
  if (!grid_fits(static_cast<int64_t>(n_seqs) * nv, 256))
    return fail(GDN_ERR_UNSUPPORTED, "%s: too many (seq, head) units for one launch", fn);
  if (!(scale > 0.0f)) scale = 1.0f / sqrtf(static_cast<float>(dk));
  return launched(gdn::launch_recurrent(q, k, v, in_dtype == GDN_BF16, qs, ks, vs, g, beta, cu_seqlens, n_seqs, T_tot, nk,
                                        nv, scale, qk_l2norm != 0, state, o, o_dtype == GDN_BF16,
                                        static_cast<hipStream_t>(stream)),
                  fn);
}

int gdn_decode_step_fused(const void* x, int dtype, int64_t x_tok_stride, void* conv_state, int state_len,
                          const float* conv_weight, const float* conv_bias, int K, const void* a, const void* b,
                          const float* A_log, const float* dt_bias, const int32_t* cu_seqlens, int n_seqs,
                          int64_t T_tot, int nk, int nv, int dk, int dv, float scale, int qk_l2norm, float* state,
                          const int32_t* state_indices, int n_slots, float* state_snapshots, void* o, int o_dtype,
                          void* stream) {
  const char* fn = "gdn_decode_step_fused";
  if (!valid_dtype(dtype)) return fail(GDN_ERR_INVALID_ARGUMENT, "%s: dtype %d is not f32/bf16", fn, dtype);
  if (!valid_dtype(o_dtype)) return fail(GDN_ERR_INVALID_ARGUMENT, "%s: o_dtype %d is not f32/bf16", fn, o_dtype);
  if (n_seqs <= 0) return fail(GDN_ERR_INVALID_ARGUMENT, "%s: n_seqs must be >= 1 (got %d)", fn, n_seqs);
  if (T_tot < 0) return fail(GDN_ERR_INVALID_ARGUMENT, "%s: T_tot must be >= 0", fn);
  if (nk <= 0 || nv <= 0) return fail(GDN_ERR_INVALID_ARGUMENT, "%s: head counts must be positive", fn);
  if (nv % nk != 0)
    return fail(GDN_ERR_INVALID_ARGUMENT, "%s: nv (%d) must be a multiple of nk (%d)", fn, nv, nk);
  if (dk <= 0 || dv <= 0 || K <= 0) return fail(GDN_ERR_INVALID_ARGUMENT, "%s: dk, dv and K must be positive", fn);
  if (state_len < K - 1) return fail(GDN_ERR_INVALID_ARGUMENT, "%s: state_len (%d) < K - 1", fn, state_len);
  if (!cu_seqlens && T_tot != n_seqs)
    return fail(GDN_ERR_INVALID_ARGUMENT, "%s: without cu_seqlens T_tot must equal n_seqs (one token each)", fn);
  if (!conv_state || !conv_weight || !A_log || !dt_bias || !state)
    return fail(GDN_ERR_INVALID_ARGUMENT, "%s: conv_state, conv_weight, A_log, dt_bias and state are required", fn);
  if (T_tot > 0 && (!x || !a || !b || !o))
    return fail(GDN_ERR_INVALID_ARGUMENT, "%s: x, a, b and o are required", fn);
  if (dk != 128 || dv != 128)
    return fail(GDN_ERR_UNSUPPORTED, "%s: only dk = dv = 128 is built (got %d, %d)", fn, dk, dv);
  if (K != 4) return fail(GDN_ERR_UNSUPPORTED, "%s: only K = 4 is built (got %d)", fn, K);
  const int r = nv / nk;
  if (r != 1 && r != 2 && r != 4)
    return fail(GDN_ERR_UNSUPPORTED, "%s: nv / nk must be 1, 2 or 4 (got %d)", fn, r);
  const int64_t conv_dim = static_cast<int64_t>(2 * nk) * dk + static_cast<int64_t>(nv) * dv;
  if (conv_dim > INT32_MAX / 8) return fail(GDN_ERR_UNSUPPORTED, "%s: conv_dim too large", fn);
  if (x_tok_stride == 0) x_tok_stride = conv_dim;
  if (x_tok_stride < conv_dim)
    return fail(GDN_ERR_INVALID_ARGUMENT, "%s: x token stride smaller than conv_dim (%lld)", fn,
                static_cast<long long>(conv_dim));
  if (T_tot > INT32_MAX) return fail(GDN_ERR_UNSUPPORTED, "%s: T_tot above 2^31-1", fn);
  // one workgroup of 256 threads per value head for each (sequence, key head)
  if (!grid_fits(static_cast<int64_t>(n_seqs) * nk, 256LL * (nv / nk)))
    return fail(GDN_ERR_UNSUPPORTED, "%s: too many (seq, head) units for one launch", fn);
  if (!aligned(state, 16)) return fail(GDN_ERR_UNSUPPORTED, "%s: state must be 16-byte aligned", fn);
  if (state_indices) {
    if (n_slots <= 0) return fail(GDN_ERR_INVALID_ARGUMENT, "%s: n_slots must be >= 1 with state_indices", fn);
  } else if (n_slots != n_seqs) {
    return fail(GDN_ERR_INVALID_ARGUMENT, "%s: without state_indices n_slots must equal n_seqs", fn);
  }
  if (state_snapshots && !aligned(state_snapshots, 16))
    return fail(GDN_ERR_UNSUPPORTED, "%s: state_snapshots must be 16-byte aligned", fn);
  if (!(scale > 0.0f)) scale = 1.0f / sqrtf(static_cast<float>(dk));
  return launched(gdn::launch_decode_fused(x, dtype == GDN_BF16, x_tok_stride, conv_state, state_len, conv_weight,
                                           conv_bias, a, b, A_log, dt_bias, cu_seqlens, n_seqs, T_tot, nk, nv, scale,
                                           qk_l2norm != 0, state, state_indices, n_slots, state_snapshots, o,
                                           o_dtype == GDN_BF16, static_cast<hipStream_t>(stream)),
                  fn);
}

int gdn_causal_conv1d(const void* x, int dtype, int64_t x_tok_stride, const float* weight, const float* bias,
                      const int32_t* cu_seqlens, int n_seqs, int64_t T_tot, int conv_dim, int K,
                      const void* conv_state_in, void* conv_state_out, int state_len, int silu, void* y,
                      void* stream) {
  const char* fn = "gdn_causal_conv1d";
  if (!valid_dtype(dtype)) return fail(GDN_ERR_INVALID_ARGUMENT, "%s: dtype %d is not f32/bf16", fn, dtype);
  if (n_seqs <= 0 || T_tot < 0 || conv_dim <= 0 || K <= 0)
    return fail(GDN_ERR_INVALID_ARGUMENT, "%s: need n_seqs >= 1, T_tot >= 0, conv_dim > 0, K > 0", fn);
  if (state_len < K - 1) return fail(GDN_ERR_INVALID_ARGUMENT, "%s: state_len (%d) < K - 1", fn, state_len);
  if (K != 4) return fail(GDN_ERR_UNSUPPORTED, "%s: only K = 4 is built (got %d)", fn, K);
  if (conv_dim % 8) return fail(GDN_ERR_UNSUPPORTED, "%s: conv_dim must be a multiple of 8", fn);
  if (T_tot > INT32_MAX) return fail(GDN_ERR_UNSUPPORTED, "%s: T_tot above 2^31-1", fn);
  if (!cu_seqlens && n_seqs != 1) return fail(GDN_ERR_INVALID_ARGUMENT, "%s: cu_seqlens is required when n_seqs > 1", fn);
  if (!weight) return fail(GDN_ERR_INVALID_ARGUMENT, "%s: weight is required", fn);
  if (x_tok_stride == 0) x_tok_stride = conv_dim;
  if (x_tok_stride < conv_dim) return fail(GDN_ERR_INVALID_ARGUMENT, "%s: x token stride smaller than conv_dim", fn);
  if (T_tot > 0) {
    if (!x || !y) return fail(GDN_ERR_INVALID_ARGUMENT, "%s: x and y are required", fn);
    if (x_tok_stride % 8) return fail(GDN_ERR_UNSUPPORTED, "%s: x token stride must be a multiple of 8", fn);
    if (!aligned(x, 16) || !aligned(y, 16)) return fail(GDN_ERR_UNSUPPORTED, "%s: x and y must be 16-byte aligned", fn);
  }
  // grid x: 64 tokens per thread, 256 threads per workgroup; the state-out pass one thread per (seq, channel)
  if (!grid_fits((T_tot + 63) / 64, 256) || !grid_fits((static_cast<int64_t>(n_seqs) * conv_dim + 255) / 256, 256))
    return fail(GDN_ERR_UNSUPPORTED, "%s: too many tokens or (seq, channel) units for one launch", fn);
  if (conv_state_in && conv_state_out) {
    const size_t bytes = static_cast<size_t>(n_seqs) * conv_dim * state_len * dsize(dtype);
    const char* a0 = static_cast<const char*>(conv_state_in);
    const char* b0 = static_cast<const char*>(conv_state_out);
    if (a0 < b0 + bytes && b0 < a0 + bytes)
      return fail(GDN_ERR_INVALID_ARGUMENT, "%s: conv_state_out must not overlap conv_state_in", fn);
  }
  return launched(gdn::launch_causal_conv1d(x, dtype == GDN_BF16, x_tok_stride, weight, bias, cu_seqlens, n_seqs,
                                            T_tot, conv_dim, conv_state_in, conv_state_out, state_len, silu != 0, y,
                                            static_cast<hipStream_t>(stream)),
                  fn);
}

int gdn_causal_conv1d_update(const void* x, int dtype, void* conv_state, int state_len, const float* weight,
                             const float* bias, int n_seqs, int conv_dim, int K, int silu, void* y, void* stream) {
  const char* fn = "gdn_causal_conv1d_update";
  if (!valid_dtype(dtype)) return fail(GDN_ERR_INVALID_ARGUMENT, "%s: dtype %d is not f32/bf16", fn, dtype);
  if (n_seqs < 0 || conv_dim <= 0 || K <= 0)
    return fail(GDN_ERR_INVALID_ARGUMENT, "%s: need n_seqs >= 0, conv_dim > 0, K > 0", fn);
  if (state_len < K - 1) return fail(GDN_ERR_INVALID_ARGUMENT, "%s: state_len (%d) < K - 1", fn, state_len);
  if (K != 4) return fail(GDN_ERR_UNSUPPORTED, "%s: only K = 4 is built (got %d)", fn, K);
  if (!weight) return fail(GDN_ERR_INVALID_ARGUMENT, "%s: weight is required", fn);
  if (n_seqs == 0) return ok();
  if (!x || !conv_state || !y) return fail(GDN_ERR_INVALID_ARGUMENT, "%s: x, conv_state and y are required", fn);
  if (!grid_fits((static_cast<int64_t>(n_seqs) * conv_dim + 255) / 256, 256))
    return fail(GDN_ERR_UNSUPPORTED, "%s: too many (seq, channel) units for one launch", fn);
  return launched(gdn::launch_causal_conv1d_update(x, dtype == GDN_BF16, conv_state, state_len, weight, bias, n_seqs,
                                                   conv_dim, silu != 0, y, static_cast<hipStream_t>(stream)),
                  fn);
}

int gdn_gated_rmsnorm(const void* x, int x_dtype, const void* z, int z_dtype, const float* weight, int64_t rows,
                      int D, float eps, void* y, int y_dtype, void* stream) {
  const char* fn = "gdn_gated_rmsnorm";
  if (!valid_dtype(x_dtype) || !valid_dtype(z_dtype) || !valid_dtype(y_dtype))
    return fail(GDN_ERR_INVALID_ARGUMENT, "%s: dtypes must be f32/bf16", fn);
  if (rows < 0 || D <= 0) return fail(GDN_ERR_INVALID_ARGUMENT, "%s: need rows >= 0 and D > 0", fn);
  if (!(eps >= 0.0f)) return fail(GDN_ERR_INVALID_ARGUMENT, "%s: eps must be >= 0", fn);
  if (D % 4 || D > 4096) return fail(GDN_ERR_UNSUPPORTED, "%s: D must be a multiple of 4 and <= 4096", fn);
  if (!weight) return fail(GDN_ERR_INVALID_ARGUMENT, "%s: weight is required", fn);
  if (rows == 0) return ok();
  if (!x || !z || !y) return fail(GDN_ERR_INVALID_ARGUMENT, "%s: x, z and y are required", fn);
  if (!grid_fits((rows + 7) / 8, 256)) return fail(GDN_ERR_UNSUPPORTED, "%s: too many rows for one launch", fn);
  return launched(gdn::launch_gated_rmsnorm(x, x_dtype == GDN_BF16, z, z_dtype == GDN_BF16, weight, rows, D, eps, y,
                                            y_dtype == GDN_BF16, static_cast<hipStream_t>(stream)),
                  fn);
}

}  // extern "C"
