// gdn_internal.hpp -- launchers shared between the C-ABI layer and the kernel files.
// All arguments have been validated by the caller (gdn_api.cpp).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gdn {

hipError_t launch_gating(const void* a, const void* b, int bf16, const float* A_log,
                         const float* dt_bias, int64_t T, int nv, float* g, float* beta,
                         hipStream_t s);

hipError_t launch_gated_rmsnorm(const void* x, int x_bf16, const void* z, int z_bf16,
                                const float* w, int64_t rows, int D, float eps, void* y,
                                int y_bf16, hipStream_t s);

hipError_t launch_causal_conv1d(const void* x, int bf16, int64_t x_stride, const float* w,
                                const float* bias, const int32_t* cu, int n_seqs, int64_t T,
                                int C, const void* st_in, void* st_out, int state_len, int silu,
                                void* y, hipStream_t s);

// Only the conv_state_out part of launch_causal_conv1d: the last state_len
// inputs of every sequence (for callers that apply the conv elsewhere).
hipError_t launch_conv_state_out(const void* x, int bf16, int64_t x_stride, const int32_t* cu, int n_seqs,
                                 int64_t T, int C, const void* st_in, void* st_out, int state_len, hipStream_t s);

hipError_t launch_causal_conv1d_update(const void* x, int bf16, void* state, int state_len,
                                       const float* w, const float* bias, int n_seqs, int C,
                                       int silu, void* y, hipStream_t s);

hipError_t launch_recurrent(const void* q, const void* k, const void* v, int bf16,
                            int64_t qs, int64_t ks, int64_t vs, const float* g, const float* beta,
                            const int32_t* cu, int n_seqs, int64_t T, int nk, int nv, float scale, int l2,
                            float* state, void* o, int o_bf16, hipStream_t s);

// Fused decode step (conv update + SiLU, gating, recurrent rule); nv / nk must
// be 1, 2 or 4.
hipError_t launch_decode_fused(const void* x, int bf16, int64_t x_stride, void* conv_state, int state_len,
                               const float* conv_w, const float* conv_b, const void* a, const void* b,
                               const float* A_log, const float* dt_bias, const int32_t* cu, int n_seqs,
                               int64_t T_tot, int nk, int nv, float scale, int l2, float* state,
                               const int32_t* slots, int n_slots, float* snap, void* o, int o_bf16,
                               hipStream_t s);

// Chunked path. The workspace holds, per chunk and value head, the packed
// 64x64 tile [T strictly lower | P turned by 180 degrees on and above the
// diagonal] and the per-token scalars, and for bf16 inputs per chunk and key
// head the K and Q operand tiles; see k_chunk.hip.
size_t chunk_workspace_bytes(int64_t T, int n_seqs, int nk, int nv, int bf16);
// Gating inputs: gm = 0: ga, gb are g and beta (fp32); gm = 1 / 2: ga, gb are
// the raw a and b (bf16 / fp32), gated inside the prep kernel with A_log, dt_bias.
hipError_t launch_chunk_fwd(const void* q, const void* k, const void* v, int bf16,
                            int64_t qs, int64_t ks, int64_t vs, const void* ga, const void* gb, int gm,
                            const float* A_log, const float* dt_bias, const int32_t* cu, int n_seqs,
                            int64_t T, int nk, int nv, float scale, int l2, const float* S0, float* ST,
                            void* o, int o_bf16, void* ws, hipStream_t s);

// Bytes of the device-resident scratch array that replaces the workspace in
// the allocation-free entry point (one array per GPU, held by the library).
constexpr size_t kNoallocScratchBytes = size_t(256) << 20;
// launch_chunk_fwd with the library's scratch array as the workspace; the
// caller has checked that the workspace fits it. No allocation.
hipError_t launch_chunk_fwd_noalloc(const void* q, const void* k, const void* v, int bf16,
                                    int64_t qs, int64_t ks, int64_t vs, const void* ga, const void* gb, int gm,
                                    const float* A_log, const float* dt_bias, const int32_t* cu, int n_seqs,
                                    int64_t T, int nk, int nv, float scale, int l2, const float* S0, float* ST,
                                    void* o, int o_bf16, hipStream_t s);

// Gated RMSNorm applied to the chunked path's output: y = o rms(o)^-1 (1 + w)
// z sigmoid(z) per (token, value head) row of 128; z bf16 [T, nv, 128] dense.
struct NormEpi {
  const uint16_t* z;
  const float* w;
  float eps;
};

// The chunked path with the causal conv1d (4 taps) + SiLU folded in, bf16 x
// [T, (2 nk + nv) 128] with token stride xs; gating inputs as for gm = 1 / 2.
// The conv state out is not written here (launch_conv_state_out). With ne,
// o (fp32) receives the normalized output: inside the state kernel when its
// wide form runs with every workgroup resident, else by the norm kernel in
// place afterwards.
hipError_t launch_chunk_fwd_conv(const void* x, int64_t xs, const float* conv_w, const float* conv_b,
                                 const void* conv_st, int state_len, const void* a, const void* b, int gm,
                                 const float* A_log, const float* dt_bias, const int32_t* cu, int n_seqs, int64_t T,
                                 int nk, int nv, float scale, int l2, const float* S0, float* ST, void* o, int o_bf16,
                                 void* ws, const NormEpi* ne, hipStream_t s);

}  // namespace gdn
