/*
 * gdn.h -- C ABI of libgdn.so: the Gated DeltaNet core for AMD MI355X (gfx950).
 *
 * The operations are those of a Gated DeltaNet token mixer as published in
 * "Qwen3.5 Dense Model Architecture" (blog), section "Linear Attention"
 * (mechanism list, minimal forward example, cache table) and in "Qwen3.5
 * Simulation Support Design Document" (msmodeling RFC), sections 1.1, 2.2
 * (decomposed op flow: causal conv / conv update, gating, chunk and recurrent
 * gated delta rule, gated RMSNorm), 2.3 (chunk vs recurrent path selection)
 * and 2.4 (conv body vs conv state update).
 *
 * General conventions (all entry points):
 *   - Every tensor pointer is a DEVICE pointer unless stated otherwise. The
 *     caller allocates and owns every buffer, including workspaces; the
 *     library never allocates, frees or synchronises on these paths.
 *   - Every call is asynchronous on `stream` (a hipStream_t; NULL = the
 *     default stream). Return value GDN_OK only means the work was enqueued.
 *   - Arguments are validated on the host before any HIP call; a non-OK
 *     return enqueues nothing and leaves outputs untouched. gdn_last_error()
 *     then describes the failure (thread-local string).
 *   - Data-dependent preconditions that the host cannot see (cu_seqlens
 *     monotone, starting at 0 and ending at T_tot; finite inputs; g within
 *     [-1e4, 0]) are the caller's responsibility; violating them gives
 *     unspecified output, never an out-of-bounds access of any buffer whose
 *     documented size is respected.
 *   - Layouts are row-major with the last index contiguous. A "token stride"
 *     is the distance in elements between consecutive tokens (0 = dense),
 *     which lets q/k/v be zero-copy views into a packed [T, conv_dim] tensor.
 *   - dtype codes: GDN_F32 = 0, GDN_BF16 = 1. Parameters (A_log, dt_bias,
 *     conv weight/bias, norm weight) are always fp32. Recurrent states are
 *     always fp32; conv states use the activation dtype.
 *   - Results are deterministic: the kernels use no atomics.
 */
#ifndef GDN_H
#define GDN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GDN_ABI_VERSION 1

enum gdn_status {
  GDN_OK = 0,
  GDN_ERR_INVALID_ARGUMENT = 1, /* null required pointer, bad size, nv % nk != 0, ...   */
  GDN_ERR_UNSUPPORTED = 2,      /* valid but not implemented (e.g. dk != 128, K != 4)  */
  GDN_ERR_WORKSPACE_TOO_SMALL = 3,
  GDN_ERR_LAUNCH = 4            /* a HIP launch or runtime call failed                */
};

enum gdn_dtype { GDN_F32 = 0, GDN_BF16 = 1 };

int gdn_abi_version(void);
const char* gdn_status_string(int status);
/* Detail of the last non-OK return on the calling thread ("" if none). */
const char* gdn_last_error(void);

/*
 * Gating ("Qwen3.5 Dense Model Architecture", Linear Attention, the beta and g
 * lines of the minimal example; computed in fp32 as the page notes, to keep
 * A_log from overflowing in low precision):
 *   beta[t,h] = sigmoid(b[t,h])
 *   g[t,h]    = -exp(A_log[h]) * softplus(a[t,h] + dt_bias[h])
 * a, b : [T_tot, nv] of ab_dtype, dense.  A_log, dt_bias : [nv] fp32.
 * g, beta : [T_tot, nv] fp32 outputs.  T_tot = 0 is a no-op.
 */
int gdn_gating(const void* a, const void* b, int ab_dtype,
               const float* A_log, const float* dt_bias,
               int64_t T_tot, int nv, float* g, float* beta, void* stream);

/*
 * Chunked gated delta rule, the prefill path ("Qwen3.5 Simulation Support
 * Design Document", 2.2 op 4 and Appendix B: the sequence is split into
 * chunks of 64 for intra-chunk attention plus an inter-chunk recurrence;
 * "Qwen3.5 Dense Model Architecture", Linear Attention: prefill calls the
 * chunk kernel and writes the final state back to the cache).
 *
 * Per packed sequence n (tokens [cu[n], cu[n+1])) and value head h, with key
 * head hk = h / (nv / nk) (repeat_interleave), the result equals the token
 * recurrence
 *   qh = q[t,hk] / sqrt(|q|^2 + 1e-6) * scale,  kh = k[t,hk] / sqrt(|k|^2 + 1e-6)
 *   S <- exp(g[t,h]) S ;  S <- S + beta[t,h] kh (v[t,h] - S^T kh)^T ;  o[t,h] = S^T qh
 * (the L2 norms are skipped when qk_l2norm == 0), evaluated chunk-parallel.
 *
 *   q, k   : [T_tot, nk, dk] of in_dtype, token stride q_tok_stride / k_tok_stride
 *   v      : [T_tot, nv, dv] of in_dtype, token stride v_tok_stride
 *            (heads are contiguous inside a token in all three)
 *   g, beta: [T_tot, nv] fp32 dense (gdn_gating output; g must lie in [-1e4, 0])
 *   cu_seqlens : device int32 [n_seqs + 1], or NULL for one sequence of T_tot
 *   scale  : <= 0 selects dk^-1/2
 *   initial_state : [n_seqs, nv, dk, dv] fp32 or NULL (zero state)
 *   final_state   : same shape, or NULL (not written); may alias initial_state
 *   o      : [T_tot, nv, dv], o_dtype (fp32 recommended; bf16 rounds once)
 *   workspace : device buffer of at least gdn_chunk_fwd_workspace_size(...) bytes,
 *            256-byte aligned; its contents on entry are ignored.
 * Supported: dk = dv = 128; in_dtype f32 or bf16; nv % nk == 0; token strides
 * up to 2^24 elements.
 * For bf16 inputs the library picks one of two forms of its state kernel from
 * the launch shape (one 16-column slice per workgroup, or two when there are
 * more slices than the device has CUs); both give the same
 * bits. The environment variable GDN_STATE_FORM=narrow or =wide, read at each
 * call, forces one (for tests and measurement). This applies to every chunk
 * entry point below.
 * Segment-parallel prefill: one sequence (n_seqs == 1) with bf16 inputs and
 * at most eight value heads has few independent recurrences (8 per value
 * head), so gdn_chunk_fwd and gdn_chunk_fwd_gated split it into segments of
 * whole chunks: eight (of at least four chunks) up to four value heads, four
 * from five to eight heads when the sequence has at least 256 chunks. Each segment's final state is affine in its
 * incoming state, S_out = M S_in + D: a first pass forms every segment's D
 * (from a zero state) and M (from the identity with v = 0), a small kernel
 * chains the incoming states in segment order, and a second pass reruns every
 * segment from its incoming state, writing o and the final state. The split
 * depends on the shape only, so results do not depend on the device; they
 * differ from the unsplit call by rounding only. gdn_prefill_fused splits the
 * same way (the conv inputs before a segment's first token are then x rows;
 * the conv state only precedes the first segment). GDN_SEGMENTS=<P> in the
 * environment (read at each call) forces P segments, 1 = unsplit. The
 * workspace size includes room for up to 16 segments whenever the shape
 * allows the split.
 */
size_t gdn_chunk_fwd_workspace_size(int64_t T_tot, int n_seqs, int nk, int nv,
                                    int dk, int dv, int in_dtype);
int gdn_chunk_fwd(const void* q, const void* k, const void* v, int in_dtype,
                  int64_t q_tok_stride, int64_t k_tok_stride, int64_t v_tok_stride,
                  const float* g, const float* beta,
                  const int32_t* cu_seqlens, int n_seqs, int64_t T_tot,
                  int nk, int nv, int dk, int dv, float scale, int qk_l2norm,
                  const float* initial_state, float* final_state,
                  void* o, int o_dtype,
                  void* workspace, size_t workspace_bytes, void* stream);

/*
 * gdn_chunk_fwd with the gating folded in: takes the raw a and b ([T_tot, nv]
 * of ab_dtype, dense) with A_log and dt_bias ([nv] fp32) where gdn_chunk_fwd
 * takes g and beta, and computes g and beta as gdn_gating does, inside the
 * chunk preparation ("Qwen3.5 Dense Model Architecture", Linear Attention:
 * the beta and g lines of the minimal example feed the chunk rule directly;
 * "Qwen3.5 Simulation Support Design Document", 2.2 ops 3 and 4). One launch
 * fewer and no g/beta round trip; the results are bit for bit those of
 * gdn_gating followed by gdn_chunk_fwd. All other arguments, the workspace
 * size and the supported shapes are those of gdn_chunk_fwd.
 */
int gdn_chunk_fwd_gated(const void* q, const void* k, const void* v, int in_dtype,
                        int64_t q_tok_stride, int64_t k_tok_stride, int64_t v_tok_stride,
                        const void* a, const void* b, int ab_dtype,
                        const float* A_log, const float* dt_bias,
                        const int32_t* cu_seqlens, int n_seqs, int64_t T_tot,
                        int nk, int nv, int dk, int dv, float scale, int qk_l2norm,
                        const float* initial_state, float* final_state,
                        void* o, int o_dtype,
                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * gdn_chunk_fwd_gated without a caller workspace, for callers that cannot
 * allocate device memory around the call: code being captured into a device
 * graph, tight serving loops, harnesses that forbid allocation. The library
 * holds one scratch array of gdn_chunk_fwd_noalloc_max_bytes() bytes per GPU
 * it runs on (a device-resident static, kept until the process ends) and
 * uses it in place of the workspace; this entry point itself allocates and
 * frees nothing. All arguments, results and supported shapes are those of
 * gdn_chunk_fwd_gated (same kernels, same bits), minus the workspace.
 * Errors: GDN_ERR_WORKSPACE_TOO_SMALL when
 * gdn_chunk_fwd_workspace_size(T_tot, n_seqs, nk, nv, dk, dv, in_dtype)
 * exceeds gdn_chunk_fwd_noalloc_max_bytes() (then nothing is enqueued; use
 * gdn_chunk_fwd_gated with a workspace); otherwise as gdn_chunk_fwd_gated.
 * Every call on one GPU shares that GPU's scratch array, and its contents on
 * entry are ignored (nothing in it needs to start at zero): calls that overlap
 * in time on one GPU (different streams, or different host threads without
 * ordering) race on it and give unspecified results.
 */
size_t gdn_chunk_fwd_noalloc_max_bytes(void);
int gdn_chunk_fwd_gated_noalloc(const void* q, const void* k, const void* v, int in_dtype,
                                int64_t q_tok_stride, int64_t k_tok_stride, int64_t v_tok_stride,
                                const void* a, const void* b, int ab_dtype,
                                const float* A_log, const float* dt_bias,
                                const int32_t* cu_seqlens, int n_seqs, int64_t T_tot,
                                int nk, int nv, int dk, int dv, float scale, int qk_l2norm,
                                const float* initial_state, float* final_state,
                                void* o, int o_dtype, void* stream);

/*
 * The prefill core of one layer with the causal conv folded into the chunk
 * kernels ("Qwen3.5 Dense Model Architecture", Linear Attention, minimal
 * example: the packed q|k|v projection goes through the causal conv1d and
 * SiLU, is split into q, k, v, and feeds the chunk rule with the beta and g of
 * the gating; "Qwen3.5 Simulation Support Design Document", 2.2 ops 1-4).
 * The prep kernel applies the conv to the key and query rows of each chunk
 * and the state kernel to the value rows it stages, each from a 3-token halo,
 * so the conv output never goes to memory. The results (o, final_state,
 * conv_state_out) are bit for bit those of gdn_causal_conv1d (silu = 1,
 * output in the dtype of x), gdn_gating and gdn_chunk_fwd run one after the
 * other, q, k, v being the views of the conv output at channel offsets 0,
 * nk*dk and 2*nk*dk.
 *   x          : [T_tot, conv_dim] bf16, channels dense, token stride
 *                x_tok_stride (0 = conv_dim); conv_dim = 2*nk*dk + nv*dv;
 *                16-byte aligned, stride a multiple of 8
 *   conv_weight: [conv_dim, K] fp32;  conv_bias : [conv_dim] fp32 or NULL
 *   conv_state_in : [n_seqs, conv_dim, state_len] bf16 or NULL (zero history):
 *                its last K-1 entries precede each sequence's first token
 *   conv_state_out: same shape or NULL (not written): the last state_len
 *                inputs of each sequence; must not overlap conv_state_in
 *   a, b, A_log, dt_bias : as gdn_chunk_fwd_gated
 *   cu_seqlens, scale, qk_l2norm, initial_state, final_state, o, workspace:
 *                as gdn_chunk_fwd, with the workspace size of
 *                gdn_chunk_fwd_workspace_size(T_tot, n_seqs, nk, nv, dk, dv, GDN_BF16)
 * Supported: dtype bf16, K = 4, dk = dv = 128, nv % nk == 0, x_tok_stride up to 2^24.
 */
int gdn_prefill_fused(const void* x, int dtype, int64_t x_tok_stride,
                      const float* conv_weight, const float* conv_bias, int K,
                      const void* conv_state_in, void* conv_state_out, int state_len,
                      const void* a, const void* b, int ab_dtype,
                      const float* A_log, const float* dt_bias,
                      const int32_t* cu_seqlens, int n_seqs, int64_t T_tot,
                      int nk, int nv, int dk, int dv, float scale, int qk_l2norm,
                      const float* initial_state, float* final_state,
                      void* o, int o_dtype,
                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * gdn_prefill_fused followed by the layer's gated RMSNorm of its output, in
 * one call ("Qwen3.5 Dense Model Architecture", Linear Attention, minimal
 * example: the core output goes straight into the gated norm with z;
 * "Qwen3.5 Simulation Support Design Document" 2.2, the decomposed op flow):
 *   y[t,h,:] = o[t,h,:] (mean(o[t,h,:]^2) + eps)^-1/2 (1 + norm_weight) z[t,h,:] sigmoid(z[t,h,:])
 * where o is what gdn_prefill_fused would write (fp32).
 *   z          : [T_tot, nv, dv] bf16, dense, 16-byte aligned
 *   norm_weight: [dv] fp32;  eps >= 0
 *   y          : [T_tot, nv, dv] fp32 output (o is not written anywhere)
 * Every other argument is as for gdn_prefill_fused (same workspace size).
 * When the launch runs the wide form of the state kernel and all of its
 * workgroups fit the device at once, the norm runs inside the state kernel: o
 * never leaves the CU, and the four workgroups that hold a row's 128 columns
 * exchange their partial sums of squares through a small ring in the
 * workspace (a cooperative launch; each wait for a partner is bounded, and a
 * row whose partners never arrive would come out NaN rather than hang).
 * Otherwise (the four-wave form, a segment-parallel split, or a cooperative
 * launch the runtime refuses) o is written to y and
 * normalized there by a second launch. The two routes differ by the order of
 * the sum of squares only. Calls on one stream are ordered; concurrent calls
 * on different streams need different workspaces, as for every call here.
 */
int gdn_prefill_fused_norm(const void* x, int dtype, int64_t x_tok_stride,
                           const float* conv_weight, const float* conv_bias, int K,
                           const void* conv_state_in, void* conv_state_out, int state_len,
                           const void* a, const void* b, int ab_dtype,
                           const float* A_log, const float* dt_bias,
                           const int32_t* cu_seqlens, int n_seqs, int64_t T_tot,
                           int nk, int nv, int dk, int dv, float scale, int qk_l2norm,
                           const float* initial_state, float* final_state,
                           const void* z, int z_dtype, const float* norm_weight, float eps,
                           float* y,
                           void* workspace, size_t workspace_bytes, void* stream);

/*
 * Recurrent gated delta rule, the decode path ("Qwen3.5 Simulation Support
 * Design Document", 2.2 op 5 and 2.3: decode batches, including multi-token
 * MTP decode, take the token-by-token path; "Qwen3.5 Dense Model
 * Architecture", cache table: decode updates the recurrent state in place).
 * Same recurrence and argument meaning as gdn_chunk_fwd, except:
 *   cu_seqlens : device int32 [n_seqs + 1], or NULL for exactly one token per
 *                sequence (then T_tot must equal n_seqs)
 *   state      : [n_seqs, nv, dk, dv] fp32, read and then overwritten in place
 *                with the state after each sequence's last token.
 * Supported: dk = dv = 128; in_dtype f32 or bf16; token strides up to 2^24 elements.
 */
int gdn_recurrent_fwd(const void* q, const void* k, const void* v, int in_dtype,
                      int64_t q_tok_stride, int64_t k_tok_stride, int64_t v_tok_stride,
                      const float* g, const float* beta,
                      const int32_t* cu_seqlens, int n_seqs, int64_t T_tot,
                      int nk, int nv, int dk, int dv, float scale, int qk_l2norm,
                      float* state, void* o, int o_dtype, void* stream);

/*
 * One fused decode step of the layer core: conv update with SiLU over the
 * packed q|k|v channels, gating, and the recurrent gated delta rule with
 * L2-normalised q and k, in a single launch ("Qwen3.5 Dense Model
 * Architecture", Linear Attention, decode branch of the minimal example and
 * its cache table: conv state and recurrent state are updated in place;
 * "Qwen3.5 Simulation Support Design Document", 2.2 ops 1, 3 and 5 and 2.3:
 * single-token and 1 + num_mtp_tokens (MTP) decode batches take the
 * recurrent path; "Qwen3.5 / Qwen3.6 Inference Path on vLLM Ascend", step
 * execution and graph capture: decode steps run as captured device graphs).
 *
 * The result is that of gdn_causal_conv1d_update (gdn_causal_conv1d with
 * conv_state_in/out for several tokens per sequence), gdn_gating and
 * gdn_recurrent_fwd run one after the other, with q, k, v the views of the
 * conv output at channel offsets 0, nk*dk and 2*nk*dk, and the conv output
 * rounded to the activation dtype in between as a stored tensor would be.
 * For one token per sequence the fused step reproduces those three launches
 * bit for bit.
 *   x          : [T_tot, conv_dim] of dtype, channels dense, token stride
 *                x_tok_stride (0 = conv_dim); conv_dim = 2*nk*dk + nv*dv
 *   conv_state : [n_slots, conv_dim, state_len] of dtype pool, updated in place
 *                to the last state_len entries of [conv_state, x of the sequence]
 *   conv_weight: [conv_dim, K] fp32;  conv_bias : [conv_dim] fp32 or NULL
 *   a, b       : [T_tot, nv] of dtype, dense;  A_log, dt_bias : [nv] fp32
 *   cu_seqlens : device int32 [n_seqs + 1] (tokens of each sequence, 0 allowed),
 *                or NULL for exactly one token per sequence (T_tot == n_seqs)
 *   scale      : <= 0 selects dk^-1/2
 *   state      : [n_slots, nv, dk, dv] fp32 pool, updated in place
 *   state_indices : device int32 [n_seqs] or NULL. Sequence n uses slot
 *                state_indices[n] of both pools (state and conv_state, whose
 *                first dimension is then n_slots); a slot < 0 or >= n_slots
 *                marks padding: that sequence is skipped, its o rows are not
 *                written. NULL means slot n (and n_slots must equal n_seqs).
 *                Non-negative slots must be distinct.
 *   state_snapshots : [T_tot, nv, dk, dv] fp32 or NULL: when given, the state
 *                after every token is also written there (row t = the state
 *                after token t), so a caller can roll back to the state after
 *                any accepted draft token.
 *   o          : [T_tot, nv, dv] of o_dtype
 * Supported: dk = dv = 128, K = 4, nv / nk in {1, 2, 4}, dtype f32 or bf16.
 * Calls that share conv_state or state rows must not overlap in time.
 */
int gdn_decode_step_fused(const void* x, int dtype, int64_t x_tok_stride,
                          void* conv_state, int state_len,
                          const float* conv_weight, const float* conv_bias, int K,
                          const void* a, const void* b,
                          const float* A_log, const float* dt_bias,
                          const int32_t* cu_seqlens, int n_seqs, int64_t T_tot,
                          int nk, int nv, int dk, int dv, float scale, int qk_l2norm,
                          float* state, const int32_t* state_indices, int n_slots,
                          float* state_snapshots, void* o, int o_dtype, void* stream);

/*
 * Causal depthwise conv1d with optional SiLU over packed sequences, the
 * prefill conv body ("Qwen3.5 Simulation Support Design Document", 2.4;
 * "Qwen3.5 Dense Model Architecture", Linear Attention: depthwise Conv1d of
 * kernel size linear_conv_kernel_dim over the packed QKV, then SiLU; a cached
 * conv state is prepended when present):
 *   y[t,c] = act(bias[c] + sum_{j<K} w[c,j] * x[t-(K-1)+j, c])
 * where inputs before a sequence's first token come from the last K-1 entries
 * of conv_state_in[n,c,:] (zeros when conv_state_in is NULL).
 *   x, y          : [T_tot, conv_dim] of dtype; x token stride x_tok_stride
 *                   (0 = dense); y is dense
 *   weight        : [conv_dim, K] fp32;  bias : [conv_dim] fp32 or NULL
 *   conv_state_in : [n_seqs, conv_dim, state_len] of dtype, or NULL
 *   conv_state_out: same shape or NULL: the last state_len entries of
 *                   concat(conv_state_in[n,c,:] or zeros, x[seq n, c]).
 *                   Must not overlap conv_state_in.
 * Supported: K = 4, state_len >= K - 1, conv_dim % 8 == 0, dtype f32 or bf16.
 */
int gdn_causal_conv1d(const void* x, int dtype, int64_t x_tok_stride,
                      const float* weight, const float* bias,
                      const int32_t* cu_seqlens, int n_seqs, int64_t T_tot,
                      int conv_dim, int K,
                      const void* conv_state_in, void* conv_state_out, int state_len,
                      int silu, void* y, void* stream);

/*
 * One decode step of the causal conv ("Qwen3.5 Simulation Support Design
 * Document", 2.4 state update; "Qwen3.5 Dense Model Architecture", decode
 * branch of the minimal example): window = [conv_state[n,c,-(K-1):], x[n,c]],
 *   y[n,c] = act(bias[c] + sum_j w[c,j] window[j]),
 * then conv_state[n,c,:] <- [conv_state[n,c,1:], x[n,c]] in place.
 *   x, y : [n_seqs, conv_dim] of dtype, dense.
 *   conv_state : [n_seqs, conv_dim, state_len] of dtype, updated in place.
 * Supported: K = 4, state_len >= K - 1, dtype f32 or bf16.
 */
int gdn_causal_conv1d_update(const void* x, int dtype, void* conv_state, int state_len,
                             const float* weight, const float* bias,
                             int n_seqs, int conv_dim, int K, int silu,
                             void* y, void* stream);

/*
 * Gated RMSNorm epilogue ("Qwen3.5 Simulation Support Design Document", 1.1
 * and Appendix B: RMSNorm whose output is scaled by 1 + weight, with the
 * SiLU(z) gate of 2.2 op 6; "Qwen3.5 Dense Model Architecture", minimal
 * example: norm(core_output, z) over rows of Dv):
 *   y[r,:] = x[r,:] * (mean(x[r,:]^2) + eps)^(-1/2) * (1 + weight) * z[r,:] * sigmoid(z[r,:])
 *   x : [rows, D] of x_dtype;  z : [rows, D] of z_dtype;  weight : [D] fp32;
 *   y : [rows, D] of y_dtype. All dense.
 * Supported: D % 4 == 0 and D <= 4096.
 */
int gdn_gated_rmsnorm(const void* x, int x_dtype, const void* z, int z_dtype,
                      const float* weight, int64_t rows, int D, float eps,
                      void* y, int y_dtype, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* GDN_H */
