"""Python binding of libgdn.so -- the Gated DeltaNet core for AMD MI355X (gfx950).

A thin ctypes layer: every function has the name of the C entry point it
calls (see include/gdn.h) and only marshals arguments -- device pointers,
strides, dtype codes and the current HIP stream. All arithmetic runs in the
HIP kernels of libgdn.so; PyTorch only provides device memory and streams.
There is no fallback: if the library is missing, every call raises.

Build the library with ``python -m gated_deltanet_gdn_amd.build``.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "GdnError", "lib", "F32", "BF16",
    "gdn_abi_version", "gdn_status_string", "gdn_last_error",
    "gdn_gating", "gdn_chunk_fwd_workspace_size", "gdn_chunk_fwd", "gdn_chunk_fwd_gated", "gdn_recurrent_fwd",
    "gdn_causal_conv1d", "gdn_causal_conv1d_update", "gdn_gated_rmsnorm", "gdn_decode_step_fused",
    "gdn_prefill_fused", "gdn_chunk_fwd_noalloc_max_bytes", "gdn_chunk_fwd_gated_noalloc", "gdn_prefill_fused_norm",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libgdn.so")
F32, BF16 = 0, 1
_DT = {torch.float32: F32, torch.bfloat16: BF16}
_TORCH_DT = {F32: torch.float32, BF16: torch.bfloat16}
_lib = None


class GdnError(RuntimeError):
    def __init__(self, fn, status, detail):
        super().__init__(f"{fn} failed with status {status}: {detail}")
        self.status = status


def lib():
    """Load libgdn.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python -m gated_deltanet_gdn_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, f32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    sig = {
        "gdn_abi_version": (i32, []),
        "gdn_status_string": (ctypes.c_char_p, [i32]),
        "gdn_last_error": (ctypes.c_char_p, []),
        "gdn_gating": (i32, [vp, vp, i32, vp, vp, i64, i32, vp, vp, vp]),
        "gdn_chunk_fwd_workspace_size": (sz, [i64, i32, i32, i32, i32, i32, i32]),
        "gdn_chunk_fwd": (i32, [vp, vp, vp, i32, i64, i64, i64, vp, vp, vp, i32, i64, i32, i32, i32, i32,
                                f32, i32, vp, vp, vp, i32, vp, sz, vp]),
        "gdn_chunk_fwd_gated": (i32, [vp, vp, vp, i32, i64, i64, i64, vp, vp, i32, vp, vp, vp, i32, i64, i32, i32,
                                      i32, i32, f32, i32, vp, vp, vp, i32, vp, sz, vp]),
        "gdn_recurrent_fwd": (i32, [vp, vp, vp, i32, i64, i64, i64, vp, vp, vp, i32, i64, i32, i32, i32, i32,
                                    f32, i32, vp, vp, i32, vp]),
        "gdn_causal_conv1d": (i32, [vp, i32, i64, vp, vp, vp, i32, i64, i32, i32, vp, vp, i32, i32, vp, vp]),
        "gdn_causal_conv1d_update": (i32, [vp, i32, vp, i32, vp, vp, i32, i32, i32, i32, vp, vp]),
        "gdn_gated_rmsnorm": (i32, [vp, i32, vp, i32, vp, i64, i32, f32, vp, i32, vp]),
        "gdn_chunk_fwd_noalloc_max_bytes": (sz, []),
        "gdn_chunk_fwd_gated_noalloc": (i32, [vp, vp, vp, i32, i64, i64, i64, vp, vp, i32, vp, vp, vp, i32, i64, i32,
                                              i32, i32, i32, f32, i32, vp, vp, vp, i32, vp]),
        "gdn_prefill_fused": (i32, [vp, i32, i64, vp, vp, i32, vp, vp, i32, vp, vp, i32, vp, vp, vp, i32, i64,
                                    i32, i32, i32, i32, f32, i32, vp, vp, vp, i32, vp, sz, vp]),
        "gdn_prefill_fused_norm": (i32, [vp, i32, i64, vp, vp, i32, vp, vp, i32, vp, vp, i32, vp, vp, vp, i32, i64,
                                         i32, i32, i32, i32, f32, i32, vp, vp, vp, i32, vp, f32, vp, vp, sz, vp]),
        "gdn_decode_step_fused": (i32, [vp, i32, i64, vp, i32, vp, vp, i32, vp, vp, vp, vp, vp, i32, i64, i32, i32,
                                        i32, i32, f32, i32, vp, vp, i32, vp, vp, i32, vp]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype, fn.argtypes = res, args
    _lib = L
    return L


def gdn_abi_version() -> int:
    return lib().gdn_abi_version()


def gdn_status_string(status: int) -> str:
    return lib().gdn_status_string(status).decode()


def gdn_last_error() -> str:
    return lib().gdn_last_error().decode()


# ------------------------------------------------------------------ marshalling helpers

def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _check(fn, status):
    if status != 0:
        raise GdnError(fn, gdn_status_string(status), gdn_last_error())


def _dt(t, name):
    if t.dtype not in _DT:
        raise TypeError(f"{name}: dtype {t.dtype} is not float32/bfloat16")
    return _DT[t.dtype]


def _tok_view(t, name):
    """[T, H, D] with heads and features dense; the token stride may be anything."""
    if t.dim() != 3 or t.stride(2) != 1 or t.stride(1) != t.shape[2]:
        raise ValueError(f"{name}: expected a [T, H, D] view with dense heads (strides (*, D, 1))")
    return t.stride(0)


def _need(t, name, dtype=None, contiguous=True):
    if t is None:
        raise ValueError(f"{name} is required")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _cu(cu_seqlens, T):
    if cu_seqlens is None:
        return None, 1
    _need(cu_seqlens, "cu_seqlens", torch.int32)
    return cu_seqlens, cu_seqlens.numel() - 1


# ------------------------------------------------------------------ entry points

def gdn_gating(a, b, A_log, dt_bias, g=None, beta=None, stream=None):
    """beta = sigmoid(b), g = -exp(A_log) softplus(a + dt_bias); a, b: [T, nv]. Returns (g, beta)."""
    _need(a, "a"); _need(b, "b", a.dtype)
    _need(A_log, "A_log", torch.float32); _need(dt_bias, "dt_bias", torch.float32)
    T, nv = a.shape
    g = torch.empty((T, nv), device=a.device, dtype=torch.float32) if g is None else g
    beta = torch.empty((T, nv), device=a.device, dtype=torch.float32) if beta is None else beta
    _check("gdn_gating", lib().gdn_gating(_ptr(a), _ptr(b), _dt(a, "a"), _ptr(A_log), _ptr(dt_bias), T, nv,
                                          _ptr(g), _ptr(beta), _stream(stream)))
    return g, beta


def gdn_chunk_fwd_workspace_size(T_tot, n_seqs, nk, nv, dk=128, dv=128, in_dtype=BF16) -> int:
    return lib().gdn_chunk_fwd_workspace_size(T_tot, n_seqs, nk, nv, dk, dv, in_dtype)


def gdn_chunk_fwd(q, k, v, g, beta, cu_seqlens=None, initial_state=None, output_final_state=True,
                  final_state=None, o=None, o_dtype=torch.float32, scale=None, qk_l2norm=True,
                  workspace=None, stream=None):
    """Chunked gated delta rule. q, k: [T, nk, dk]; v: [T, nv, dv] (token-strided views allowed).

    Returns (o [T, nv, dv], final_state [n, nv, dk, dv] or None). ``final_state`` may be the
    ``initial_state`` tensor itself (in-place update).
    """
    for t, nm in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, nm, contiguous=False)
    qs, ks, vs = _tok_view(q, "q"), _tok_view(k, "k"), _tok_view(v, "v")
    _need(g, "g", torch.float32); _need(beta, "beta", torch.float32)
    T, nk, dk = q.shape
    nv, dv = v.shape[1], v.shape[2]
    cu, n = _cu(cu_seqlens, T)
    if initial_state is not None:
        _need(initial_state, "initial_state", torch.float32)
    if final_state is None and output_final_state:
        final_state = torch.empty((n, nv, dk, dv), device=q.device, dtype=torch.float32)
    if o is None:
        o = torch.empty((T, nv, dv), device=q.device, dtype=o_dtype)
    need = gdn_chunk_fwd_workspace_size(T, n, nk, nv, dk, dv, _dt(q, "q"))
    if workspace is None:
        workspace = torch.empty(max(need, 1), device=q.device, dtype=torch.uint8)
    st = lib().gdn_chunk_fwd(_ptr(q), _ptr(k), _ptr(v), _dt(q, "q"), qs, ks, vs, _ptr(g), _ptr(beta), _ptr(cu), n,
                             T, nk, nv, dk, dv, float(scale or 0.0), int(bool(qk_l2norm)),
                             _ptr(initial_state), _ptr(final_state), _ptr(o), _dt(o, "o"),
                             _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream))
    _check("gdn_chunk_fwd", st)
    return o, final_state


def gdn_chunk_fwd_gated(q, k, v, a, b, A_log, dt_bias, cu_seqlens=None, initial_state=None,
                        output_final_state=True, final_state=None, o=None, o_dtype=torch.float32, scale=None,
                        qk_l2norm=True, workspace=None, stream=None):
    """gdn_chunk_fwd with the gating folded in: a, b [T, nv] (raw) and A_log, dt_bias [nv] fp32 in place
    of g and beta. Returns (o, final_state) like gdn_chunk_fwd."""
    for t, nm in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, nm, contiguous=False)
    qs, ks, vs = _tok_view(q, "q"), _tok_view(k, "k"), _tok_view(v, "v")
    _need(a, "a"); _need(b, "b", a.dtype)
    _need(A_log, "A_log", torch.float32); _need(dt_bias, "dt_bias", torch.float32)
    T, nk, dk = q.shape
    nv, dv = v.shape[1], v.shape[2]
    cu, n = _cu(cu_seqlens, T)
    if initial_state is not None:
        _need(initial_state, "initial_state", torch.float32)
    if final_state is None and output_final_state:
        final_state = torch.empty((n, nv, dk, dv), device=q.device, dtype=torch.float32)
    if o is None:
        o = torch.empty((T, nv, dv), device=q.device, dtype=o_dtype)
    need = gdn_chunk_fwd_workspace_size(T, n, nk, nv, dk, dv, _dt(q, "q"))
    if workspace is None:
        workspace = torch.empty(max(need, 1), device=q.device, dtype=torch.uint8)
    st = lib().gdn_chunk_fwd_gated(_ptr(q), _ptr(k), _ptr(v), _dt(q, "q"), qs, ks, vs, _ptr(a), _ptr(b),
                                   _dt(a, "a"), _ptr(A_log), _ptr(dt_bias), _ptr(cu), n, T, nk, nv, dk, dv,
                                   float(scale or 0.0), int(bool(qk_l2norm)), _ptr(initial_state),
                                   _ptr(final_state), _ptr(o), _dt(o, "o"), _ptr(workspace),
                                   workspace.numel() * workspace.element_size(), _stream(stream))
    _check("gdn_chunk_fwd_gated", st)
    return o, final_state


def gdn_chunk_fwd_noalloc_max_bytes() -> int:
    return lib().gdn_chunk_fwd_noalloc_max_bytes()


def gdn_chunk_fwd_gated_noalloc(q, k, v, a, b, A_log, dt_bias, cu_seqlens=None, initial_state=None,
                                output_final_state=True, final_state=None, o=None, o_dtype=torch.float32,
                                scale=None, qk_l2norm=True, stream=None):
    """gdn_chunk_fwd_gated with the library's per-device scratch array as its workspace (the C call
    allocates nothing; outputs not passed in are allocated here by torch). Calls that overlap in time
    on one GPU share that array and race. Returns (o, final_state)."""
    for t, nm in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, nm, contiguous=False)
    qs, ks, vs = _tok_view(q, "q"), _tok_view(k, "k"), _tok_view(v, "v")
    _need(a, "a"); _need(b, "b", a.dtype)
    _need(A_log, "A_log", torch.float32); _need(dt_bias, "dt_bias", torch.float32)
    T, nk, dk = q.shape
    nv, dv = v.shape[1], v.shape[2]
    cu, n = _cu(cu_seqlens, T)
    if initial_state is not None:
        _need(initial_state, "initial_state", torch.float32)
    if final_state is None and output_final_state:
        final_state = torch.empty((n, nv, dk, dv), device=q.device, dtype=torch.float32)
    if o is None:
        o = torch.empty((T, nv, dv), device=q.device, dtype=o_dtype)
    st = lib().gdn_chunk_fwd_gated_noalloc(_ptr(q), _ptr(k), _ptr(v), _dt(q, "q"), qs, ks, vs, _ptr(a), _ptr(b),
                                           _dt(a, "a"), _ptr(A_log), _ptr(dt_bias), _ptr(cu), n, T, nk, nv, dk, dv,
                                           float(scale or 0.0), int(bool(qk_l2norm)), _ptr(initial_state),
                                           _ptr(final_state), _ptr(o), _dt(o, "o"), _stream(stream))
    _check("gdn_chunk_fwd_gated_noalloc", st)
    return o, final_state


def gdn_prefill_fused(x, conv_weight, a, b, A_log, dt_bias, nk, nv, conv_bias=None, cu_seqlens=None,
                      conv_state_in=None, conv_state_out=None, state_len=None, output_conv_state=True,
                      initial_state=None, output_final_state=True, final_state=None, o=None,
                      o_dtype=torch.float32, scale=None, qk_l2norm=True, workspace=None, stream=None):
    """Causal conv1d + SiLU, gating and the chunked rule in one call on x [T, conv_dim] (bf16, packed q | k | v;
    a token-strided view is allowed). Returns (o, final_state, conv_state_out)."""
    _need(x, "x", contiguous=False)
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x: expected a [T, conv_dim] view with dense channels")
    _need(conv_weight, "conv_weight", torch.float32)
    _need(a, "a"); _need(b, "b", a.dtype)
    _need(A_log, "A_log", torch.float32); _need(dt_bias, "dt_bias", torch.float32)
    T, C = x.shape
    K = conv_weight.shape[1]
    dk = dv = 128
    cu, n = _cu(cu_seqlens, T)
    if state_len is None:
        state_len = conv_state_in.shape[2] if conv_state_in is not None else K - 1
    if conv_state_in is not None:
        _need(conv_state_in, "conv_state_in", x.dtype)
    if conv_state_out is None and output_conv_state:
        conv_state_out = torch.empty((n, C, state_len), device=x.device, dtype=x.dtype)
    if initial_state is not None:
        _need(initial_state, "initial_state", torch.float32)
    if final_state is None and output_final_state:
        final_state = torch.empty((n, nv, dk, dv), device=x.device, dtype=torch.float32)
    if o is None:
        o = torch.empty((T, nv, dv), device=x.device, dtype=o_dtype)
    need = gdn_chunk_fwd_workspace_size(T, n, nk, nv, dk, dv, _dt(x, "x"))
    if workspace is None:
        workspace = torch.empty(max(need, 1), device=x.device, dtype=torch.uint8)
    st = lib().gdn_prefill_fused(_ptr(x), _dt(x, "x"), x.stride(0), _ptr(conv_weight), _ptr(conv_bias), K,
                                 _ptr(conv_state_in), _ptr(conv_state_out), state_len, _ptr(a), _ptr(b),
                                 _dt(a, "a"), _ptr(A_log), _ptr(dt_bias), _ptr(cu), n, T, nk, nv, dk, dv,
                                 float(scale or 0.0), int(bool(qk_l2norm)), _ptr(initial_state), _ptr(final_state),
                                 _ptr(o), _dt(o, "o"), _ptr(workspace), workspace.numel() * workspace.element_size(),
                                 _stream(stream))
    _check("gdn_prefill_fused", st)
    return o, final_state, conv_state_out


def gdn_prefill_fused_norm(x, conv_weight, a, b, A_log, dt_bias, nk, nv, z, norm_weight, eps=1e-6,
                           conv_bias=None, cu_seqlens=None, conv_state_in=None, conv_state_out=None, state_len=None,
                           output_conv_state=True, initial_state=None, output_final_state=True, final_state=None,
                           y=None, scale=None, qk_l2norm=True, workspace=None, stream=None):
    """gdn_prefill_fused followed by the gated RMSNorm of its output, in one call: y [T, nv, 128] fp32 =
    o rms(o)^-1 (1 + norm_weight) z sigmoid(z), with z [T, nv, 128] bf16 dense. Returns (y, final_state,
    conv_state_out)."""
    _need(x, "x", contiguous=False)
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x: expected a [T, conv_dim] view with dense channels")
    _need(conv_weight, "conv_weight", torch.float32)
    _need(a, "a"); _need(b, "b", a.dtype)
    _need(A_log, "A_log", torch.float32); _need(dt_bias, "dt_bias", torch.float32)
    _need(z, "z"); _need(norm_weight, "norm_weight", torch.float32)
    T, C = x.shape
    K = conv_weight.shape[1]
    dk = dv = 128
    cu, n = _cu(cu_seqlens, T)
    if state_len is None:
        state_len = conv_state_in.shape[2] if conv_state_in is not None else K - 1
    if conv_state_in is not None:
        _need(conv_state_in, "conv_state_in", x.dtype)
    if conv_state_out is None and output_conv_state:
        conv_state_out = torch.empty((n, C, state_len), device=x.device, dtype=x.dtype)
    if initial_state is not None:
        _need(initial_state, "initial_state", torch.float32)
    if final_state is None and output_final_state:
        final_state = torch.empty((n, nv, dk, dv), device=x.device, dtype=torch.float32)
    if y is None:
        y = torch.empty((T, nv, dv), device=x.device, dtype=torch.float32)
    need = gdn_chunk_fwd_workspace_size(T, n, nk, nv, dk, dv, _dt(x, "x"))
    if workspace is None:
        workspace = torch.empty(max(need, 1), device=x.device, dtype=torch.uint8)
    st = lib().gdn_prefill_fused_norm(_ptr(x), _dt(x, "x"), x.stride(0), _ptr(conv_weight), _ptr(conv_bias), K,
                                      _ptr(conv_state_in), _ptr(conv_state_out), state_len, _ptr(a), _ptr(b),
                                      _dt(a, "a"), _ptr(A_log), _ptr(dt_bias), _ptr(cu), n, T, nk, nv, dk, dv,
                                      float(scale or 0.0), int(bool(qk_l2norm)), _ptr(initial_state),
                                      _ptr(final_state), _ptr(z), _dt(z, "z"), _ptr(norm_weight), float(eps),
                                      _ptr(y), _ptr(workspace), workspace.numel() * workspace.element_size(),
                                      _stream(stream))
    _check("gdn_prefill_fused_norm", st)
    return y, final_state, conv_state_out


def gdn_recurrent_fwd(q, k, v, g, beta, state, cu_seqlens=None, o=None, o_dtype=torch.float32, scale=None,
                      qk_l2norm=True, stream=None):
    """Recurrent gated delta rule; ``state`` [n, nv, dk, dv] fp32 is updated in place. Returns o."""
    for t, nm in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, nm, contiguous=False)
    qs, ks, vs = _tok_view(q, "q"), _tok_view(k, "k"), _tok_view(v, "v")
    _need(g, "g", torch.float32); _need(beta, "beta", torch.float32)
    _need(state, "state", torch.float32)
    T, nk, dk = q.shape
    nv, dv = v.shape[1], v.shape[2]
    cu, n = _cu(cu_seqlens, T)
    if cu is None:
        n = state.shape[0]
    if o is None:
        o = torch.empty((T, nv, dv), device=q.device, dtype=o_dtype)
    st = lib().gdn_recurrent_fwd(_ptr(q), _ptr(k), _ptr(v), _dt(q, "q"), qs, ks, vs, _ptr(g), _ptr(beta), _ptr(cu), n,
                                 T, nk, nv, dk, dv, float(scale or 0.0), int(bool(qk_l2norm)), _ptr(state), _ptr(o),
                                 _dt(o, "o"), _stream(stream))
    _check("gdn_recurrent_fwd", st)
    return o


def gdn_causal_conv1d(x, weight, bias=None, cu_seqlens=None, conv_state_in=None, conv_state_out=None,
                      state_len=None, silu=True, y=None, output_final_state=True, stream=None):
    """Causal depthwise conv1d (+SiLU). x: [T, C] (token-strided view allowed); weight: [C, K] fp32.

    Returns (y [T, C], conv_state_out [n, C, state_len] or None).
    """
    _need(x, "x", contiguous=False)
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x: expected a [T, C] view with dense channels")
    _need(weight, "weight", torch.float32)
    T, C = x.shape
    K = weight.shape[1]
    cu, n = _cu(cu_seqlens, T)
    if state_len is None:
        state_len = conv_state_in.shape[2] if conv_state_in is not None else K - 1
    if conv_state_in is not None:
        _need(conv_state_in, "conv_state_in", x.dtype)
    if conv_state_out is None and output_final_state:
        conv_state_out = torch.empty((n, C, state_len), device=x.device, dtype=x.dtype)
    if y is None:
        y = torch.empty((T, C), device=x.device, dtype=x.dtype)
    st = lib().gdn_causal_conv1d(_ptr(x), _dt(x, "x"), x.stride(0), _ptr(weight), _ptr(bias), _ptr(cu), n, T, C, K,
                                 _ptr(conv_state_in), _ptr(conv_state_out), state_len, int(bool(silu)), _ptr(y),
                                 _stream(stream))
    _check("gdn_causal_conv1d", st)
    return y, conv_state_out


def gdn_causal_conv1d_update(x, conv_state, weight, bias=None, silu=True, y=None, stream=None):
    """One decode step; conv_state [n, C, state_len] is updated in place. Returns y [n, C]."""
    _need(x, "x"); _need(conv_state, "conv_state", x.dtype); _need(weight, "weight", torch.float32)
    n, C = x.shape
    K = weight.shape[1]
    if y is None:
        y = torch.empty_like(x)
    st = lib().gdn_causal_conv1d_update(_ptr(x), _dt(x, "x"), _ptr(conv_state), conv_state.shape[2], _ptr(weight),
                                        _ptr(bias), n, C, K, int(bool(silu)), _ptr(y), _stream(stream))
    _check("gdn_causal_conv1d_update", st)
    return y


def gdn_gated_rmsnorm(x, z, weight, eps=1e-6, y=None, y_dtype=torch.float32, stream=None):
    """y = x rsqrt(mean(x^2) + eps) (1 + weight) silu(z) over the last dim."""
    _need(x, "x"); _need(z, "z"); _need(weight, "weight", torch.float32)
    D = x.shape[-1]
    rows = x.numel() // D
    if y is None:
        y = torch.empty(x.shape, device=x.device, dtype=y_dtype)
    st = lib().gdn_gated_rmsnorm(_ptr(x), _dt(x, "x"), _ptr(z), _dt(z, "z"), _ptr(weight), rows, D, float(eps),
                                 _ptr(y), _dt(y, "y"), _stream(stream))
    _check("gdn_gated_rmsnorm", st)
    return y


def gdn_decode_step_fused(x, conv_state, conv_weight, a, b, A_log, dt_bias, state, nk, cu_seqlens=None,
                          conv_bias=None, state_indices=None, state_snapshots=None, o=None, o_dtype=torch.float32,
                          scale=None, qk_l2norm=True, stream=None):
    """Conv update + SiLU, gating and the recurrent rule in one launch.

    x: [T, conv_dim] (token-strided view allowed) with conv_dim = 2*nk*128 + nv*128 packed q|k|v;
    conv_state [slots, conv_dim, state_len] and state [slots, nv, 128, 128] are updated in place;
    a, b: [T, nv]. state_indices (int32 [n]) maps sequence n to its slot (negative = padding, skipped);
    without it sequence n uses slot n. state_snapshots ([T, nv, 128, 128] fp32) receives the state
    after every token. Returns o [T, nv, 128].
    """
    _need(x, "x", contiguous=False)
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x: expected a [T, C] view with dense channels")
    _need(conv_state, "conv_state", x.dtype); _need(conv_weight, "conv_weight", torch.float32)
    _need(a, "a", x.dtype); _need(b, "b", x.dtype)
    _need(A_log, "A_log", torch.float32); _need(dt_bias, "dt_bias", torch.float32)
    _need(state, "state", torch.float32)
    T = x.shape[0]
    n_slots, nv, dk, dv = state.shape
    if conv_state.shape[0] != n_slots:
        raise ValueError("conv_state and state must hold the same number of slots")
    cu, n = _cu(cu_seqlens, T)
    if state_indices is not None:
        _need(state_indices, "state_indices", torch.int32)
        if cu is not None and state_indices.numel() != n:
            raise ValueError(f"state_indices has {state_indices.numel()} entries, cu_seqlens {n} sequences")
        n = state_indices.numel()
    elif cu is None:
        n = n_slots
    elif n != n_slots:
        raise ValueError(f"cu_seqlens describes {n} sequences, state holds {n_slots} slots")
    if state_snapshots is not None:
        _need(state_snapshots, "state_snapshots", torch.float32)
    if o is None:
        o = torch.empty((T, nv, dv), device=x.device, dtype=o_dtype)
    st = lib().gdn_decode_step_fused(_ptr(x), _dt(x, "x"), x.stride(0), _ptr(conv_state), conv_state.shape[2],
                                     _ptr(conv_weight), _ptr(conv_bias), conv_weight.shape[1], _ptr(a), _ptr(b),
                                     _ptr(A_log), _ptr(dt_bias), _ptr(cu), n, T, nk, nv, dk, dv, float(scale or 0.0),
                                     int(bool(qk_l2norm)), _ptr(state), _ptr(state_indices), n_slots,
                                     _ptr(state_snapshots), _ptr(o), _dt(o, "o"), _stream(stream))
    _check("gdn_decode_step_fused", st)
    return o
