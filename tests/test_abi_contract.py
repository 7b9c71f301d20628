"""C-ABI contract of libgdn.so, checked without a GPU.

Every argument error is detected on the host before any HIP call, so these
tests pass arbitrary non-null "device" addresses and expect the documented
status. No compute entry point is called with valid arguments here.
"""
import ctypes
import os
import re

import pytest

import gated_deltanet_gdn_amd as gdn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdn.h")

OK, INVALID, UNSUPPORTED, WS_SMALL, LAUNCH = 0, 1, 2, 3, 4
P = ctypes.c_void_p(0x100000)      # a fake, 256-byte aligned "device" address (never dereferenced)
P2 = ctypes.c_void_p(0x200000)
MIS = ctypes.c_void_p(0x100002)    # misaligned
NULL = None


def declared_functions():
    src = open(HEADER).read()
    return sorted(set(re.findall(r"\b(gdn_[a-z0-9_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def L():
    return gdn.lib()


def test_library_exports_every_declared_symbol(L):
    names = declared_functions()
    assert "gdn_chunk_fwd" in names and len(names) >= 10
    for n in names:
        assert hasattr(L, n), f"libgdn.so does not export {n}"


def test_version_and_status_strings(L):
    assert gdn.gdn_abi_version() == 1
    assert gdn.gdn_status_string(OK) == "GDN_OK"
    assert gdn.gdn_status_string(INVALID) == "GDN_ERR_INVALID_ARGUMENT"
    assert gdn.gdn_status_string(UNSUPPORTED) == "GDN_ERR_UNSUPPORTED"
    assert gdn.gdn_status_string(WS_SMALL) == "GDN_ERR_WORKSPACE_TOO_SMALL"
    assert gdn.gdn_status_string(LAUNCH) == "GDN_ERR_LAUNCH"
    assert gdn.gdn_status_string(99) == "GDN_ERR_UNKNOWN"


def _chunk(L, **kw):
    a = dict(q=P, k=P, v=P, in_dtype=1, qs=0, ks=0, vs=0, g=P, beta=P, cu=NULL, n=1, T=256, nk=1, nv=2, dk=128,
             dv=128, scale=0.0, l2=1, s0=NULL, st=NULL, o=P, o_dtype=0, ws=P2, ws_bytes=1 << 40, stream=NULL)
    a.update(kw)
    return L.gdn_chunk_fwd(a["q"], a["k"], a["v"], a["in_dtype"], a["qs"], a["ks"], a["vs"], a["g"], a["beta"],
                           a["cu"], a["n"], a["T"], a["nk"], a["nv"], a["dk"], a["dv"], a["scale"], a["l2"],
                           a["s0"], a["st"], a["o"], a["o_dtype"], a["ws"], a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(nk=3, nv=4), INVALID),            # nv % nk != 0 (the pages' head-divisibility error)
    (dict(nk=0), INVALID),
    (dict(vs=(1 << 24) + 8), UNSUPPORTED),   # chunk rows use 32-bit buffer offsets
    (dict(n=0), INVALID),
    (dict(T=-1), INVALID),
    (dict(in_dtype=7), INVALID),
    (dict(o_dtype=5), INVALID),
    (dict(q=NULL), INVALID),
    (dict(beta=NULL), INVALID),
    (dict(o=NULL), INVALID),
    (dict(n=2), INVALID),                   # several sequences need cu_seqlens
    (dict(qs=100), INVALID),                # token stride smaller than a row (nk*dk = 128)
    (dict(ws=NULL), INVALID),
    (dict(ws=MIS), INVALID),
    (dict(ws_bytes=16), WS_SMALL),
    (dict(dk=64), UNSUPPORTED),
    (dict(dv=256), UNSUPPORTED),
    (dict(qs=132), UNSUPPORTED),            # not a multiple of 8 elements
    (dict(q=MIS), UNSUPPORTED),
    (dict(T=1 << 32), UNSUPPORTED),
])
def test_chunk_fwd_argument_errors(L, kw, status):
    assert _chunk(L, **kw) == status
    assert gdn.gdn_last_error().startswith("gdn_chunk_fwd")


def test_workspace_size_is_monotone_and_positive(L):
    s1 = gdn.gdn_chunk_fwd_workspace_size(8192, 1, 16, 32)
    s2 = gdn.gdn_chunk_fwd_workspace_size(8192 + 64, 1, 16, 32)
    s3 = gdn.gdn_chunk_fwd_workspace_size(8192, 8, 16, 32)
    assert 0 < s1 < s2 and s1 < s3
    assert s1 % 256 == 0
    # per chunk and value head: a 64x64 fp32 tile, 64 float4 scalars, one float
    assert s1 >= (8192 // 64) * 32 * (64 * 64 * 4 + 64 * 16 + 4)
    assert gdn.gdn_chunk_fwd_workspace_size(-1, 1, 16, 32) == 0


def test_workspace_reserves_segment_states_for_one_sequence_with_few_heads(L):
    """One sequence with bf16 inputs and at most eight value heads may run as up to 16 segments: the workspace
    then also holds 3 x 16 fp32 states per value head (local states, transitions, incoming states)."""
    state = 128 * 128 * 4
    for nk, nv in [(1, 1), (1, 2), (2, 4), (2, 8)]:
        one = gdn.gdn_chunk_fwd_workspace_size(8192, 1, nk, nv)
        two = gdn.gdn_chunk_fwd_workspace_size(8192, 2, nk, nv)
        assert one >= two + 3 * 16 * nv * state - 512 * 1024   # two sequences hold one more chunk slot
    # not for fp32 inputs, several sequences or more heads
    wide = gdn.gdn_chunk_fwd_workspace_size(8192, 1, 4, 16)
    assert wide < gdn.gdn_chunk_fwd_workspace_size(8192, 2, 4, 16) + 3 * 16 * 16 * state
    f32 = gdn.gdn_chunk_fwd_workspace_size(8192, 1, 1, 2, in_dtype=gdn.F32)
    assert f32 < gdn.gdn_chunk_fwd_workspace_size(8192, 2, 1, 2, in_dtype=gdn.F32) + 3 * 16 * 2 * state


def _rec(L, **kw):
    a = dict(q=P, k=P, v=P, in_dtype=1, qs=0, ks=0, vs=0, g=P, beta=P, cu=NULL, n=4, T=4, nk=2, nv=4, dk=128,
             dv=128, scale=0.0, l2=1, state=P2, o=P, o_dtype=0, stream=NULL)
    a.update(kw)
    return L.gdn_recurrent_fwd(a["q"], a["k"], a["v"], a["in_dtype"], a["qs"], a["ks"], a["vs"], a["g"], a["beta"],
                               a["cu"], a["n"], a["T"], a["nk"], a["nv"], a["dk"], a["dv"], a["scale"], a["l2"],
                               a["state"], a["o"], a["o_dtype"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(nk=3), INVALID),
    (dict(state=NULL), INVALID),
    (dict(T=5), INVALID),                   # one token per sequence without cu_seqlens
    (dict(v=NULL), INVALID),
    (dict(dk=96), UNSUPPORTED),
    (dict(state=MIS), UNSUPPORTED),
])
def test_recurrent_fwd_argument_errors(L, kw, status):
    assert _rec(L, **kw) == status


def _conv(L, **kw):
    a = dict(x=P, dtype=1, xs=0, w=P, b=NULL, cu=NULL, n=1, T=10, C=64, K=4, si=NULL, so=NULL, sl=3, silu=1, y=P2,
             stream=NULL)
    a.update(kw)
    return L.gdn_causal_conv1d(a["x"], a["dtype"], a["xs"], a["w"], a["b"], a["cu"], a["n"], a["T"], a["C"], a["K"],
                               a["si"], a["so"], a["sl"], a["silu"], a["y"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(sl=2), INVALID),                  # state_len < K - 1
    (dict(K=0), INVALID),
    (dict(n=2), INVALID),                   # missing cu_seqlens
    (dict(w=NULL), INVALID),
    (dict(x=NULL), INVALID),
    (dict(xs=32), INVALID),                 # stride < conv_dim
    (dict(si=P, so=ctypes.c_void_p(0x100000 + 64)), INVALID),   # overlapping states
    (dict(K=3, sl=3), UNSUPPORTED),
    (dict(C=60), UNSUPPORTED),
    (dict(xs=68), UNSUPPORTED),
    (dict(dtype=3), INVALID),
])
def test_causal_conv1d_argument_errors(L, kw, status):
    assert _conv(L, **kw) == status


@pytest.mark.parametrize("args,status", [
    ((P, 1, P2, 2, P, NULL, 4, 64, 4, 1, P, NULL), INVALID),      # state_len 2 < 3
    ((P, 1, P2, 3, NULL, NULL, 4, 64, 4, 1, P, NULL), INVALID),   # no weight
    ((NULL, 1, P2, 3, P, NULL, 4, 64, 4, 1, P, NULL), INVALID),   # no x
    ((P, 1, P2, 3, P, NULL, 4, 64, 2, 1, P, NULL), UNSUPPORTED),  # K = 2
    ((P, 1, P2, 3, P, NULL, 0, 64, 4, 1, P, NULL), OK),           # zero sequences: no-op, no HIP call
])
def test_conv_update_argument_errors(L, args, status):
    assert L.gdn_causal_conv1d_update(*args) == status


@pytest.mark.parametrize("args,status", [
    ((P, 0, P, 1, P, 10, 130, 1e-6, P2, 0, NULL), UNSUPPORTED),   # D % 4
    ((P, 0, P, 1, P, 10, 8192, 1e-6, P2, 0, NULL), UNSUPPORTED),  # D too large
    ((P, 0, P, 1, NULL, 10, 128, 1e-6, P2, 0, NULL), INVALID),
    ((P, 0, P, 1, P, 10, 128, -1.0, P2, 0, NULL), INVALID),
    ((P, 2, P, 1, P, 10, 128, 1e-6, P2, 0, NULL), INVALID),
    ((P, 0, P, 1, P, 0, 128, 1e-6, P2, 0, NULL), OK),            # zero rows: no-op
])
def test_gated_rmsnorm_argument_errors(L, args, status):
    assert L.gdn_gated_rmsnorm(*args) == status


@pytest.mark.parametrize("args,status", [
    ((P, P, 1, P, P, 10, 0, P, P, NULL), INVALID),      # nv = 0
    ((P, P, 1, NULL, P, 10, 4, P, P, NULL), INVALID),   # no A_log
    ((P, NULL, 1, P, P, 10, 4, P, P, NULL), INVALID),
    ((P, P, 9, P, P, 10, 4, P, P, NULL), INVALID),
    ((NULL, NULL, 1, P, P, 0, 4, NULL, NULL, NULL), OK),  # T = 0: no-op
])
def test_gating_argument_errors(L, args, status):
    assert L.gdn_gating(*args) == status


def test_python_binding_requires_device_tensors():
    import torch
    x = torch.zeros(4, 2)
    with pytest.raises(ValueError):
        gdn.gdn_gating(x, x, torch.zeros(2), torch.zeros(2))


def _fused(L, **kw):
    a = dict(x=P, dtype=1, xs=0, cst=P, sl=3, w=P, bias=NULL, K=4, a=P, b=P, alog=P, dtb=P, cu=NULL, n=4, T=4,
             nk=2, nv=4, dk=128, dv=128, scale=0.0, l2=1, state=P2, idx=NULL, n_slots=4, snap=NULL, o=P, o_dtype=0,
             stream=NULL)
    a.update(kw)
    return L.gdn_decode_step_fused(a["x"], a["dtype"], a["xs"], a["cst"], a["sl"], a["w"], a["bias"], a["K"], a["a"],
                                   a["b"], a["alog"], a["dtb"], a["cu"], a["n"], a["T"], a["nk"], a["nv"], a["dk"],
                                   a["dv"], a["scale"], a["l2"], a["state"], a["idx"], a["n_slots"], a["snap"], a["o"],
                                   a["o_dtype"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(nk=3, nv=4), INVALID),            # nv % nk != 0
    (dict(dtype=3), INVALID),
    (dict(o_dtype=2), INVALID),
    (dict(n=0), INVALID),
    (dict(T=5), INVALID),                   # one token per sequence without cu_seqlens
    (dict(sl=2), INVALID),                  # state_len < K - 1
    (dict(cst=NULL), INVALID),
    (dict(w=NULL), INVALID),
    (dict(state=NULL), INVALID),
    (dict(alog=NULL), INVALID),
    (dict(x=NULL), INVALID),
    (dict(o=NULL), INVALID),
    (dict(xs=1000), INVALID),               # token stride below conv_dim = (2*2 + 4) * 128
    (dict(nk=1, nv=8), UNSUPPORTED),        # eight value heads per key head
    (dict(nk=2, nv=6), UNSUPPORTED),        # three value heads per key head
    (dict(dk=64), UNSUPPORTED),
    (dict(K=3, sl=2), UNSUPPORTED),
    (dict(state=MIS), UNSUPPORTED),
    (dict(n_slots=5), INVALID),             # without state_indices the pool has one slot per sequence
    (dict(idx=P, n_slots=0), INVALID),
    (dict(snap=MIS), UNSUPPORTED),
])
def test_decode_step_fused_argument_errors(L, kw, status):
    assert _fused(L, **kw) == status
    assert gdn.gdn_last_error() != ""


def test_decode_step_fused_empty_batch_needs_no_inputs(L):
    # no tokens: x, a, b and o may be NULL; the call is still a valid (state-preserving) launch
    # request, so only argument checks run here -- with T = 0 and cu_seqlens NULL it must fail
    assert _fused(L, T=0, x=NULL, a=NULL, b=NULL, o=NULL) == INVALID


def _gated(L, **kw):
    a = dict(q=P, k=P, v=P, in_dtype=1, qs=0, ks=0, vs=0, a=P, b=P, ab_dtype=1, alog=P, dtb=P, cu=NULL, n=1, T=256,
             nk=1, nv=2, dk=128, dv=128, scale=0.0, l2=1, s0=NULL, st=NULL, o=P, o_dtype=0, ws=P2, ws_bytes=1 << 40,
             stream=NULL)
    a.update(kw)
    return L.gdn_chunk_fwd_gated(a["q"], a["k"], a["v"], a["in_dtype"], a["qs"], a["ks"], a["vs"], a["a"], a["b"],
                                 a["ab_dtype"], a["alog"], a["dtb"], a["cu"], a["n"], a["T"], a["nk"], a["nv"],
                                 a["dk"], a["dv"], a["scale"], a["l2"], a["s0"], a["st"], a["o"], a["o_dtype"],
                                 a["ws"], a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(ab_dtype=4), INVALID),
    (dict(a=NULL), INVALID),
    (dict(b=NULL), INVALID),
    (dict(alog=NULL), INVALID),
    (dict(dtb=NULL), INVALID),
    (dict(nk=3, nv=4), INVALID),
    (dict(n=2), INVALID),
    (dict(ws=NULL), INVALID),
    (dict(ws_bytes=16), WS_SMALL),
    (dict(dk=64), UNSUPPORTED),
])
def test_chunk_fwd_gated_argument_errors(L, kw, status):
    assert _gated(L, **kw) == status
    assert gdn.gdn_last_error() != ""


def _prefill(L, **kw):
    a = dict(x=P, dtype=1, xs=0, cw=P, cb=NULL, K=4, csi=NULL, cso=NULL, sl=3, a=P, b=P, ab_dtype=1, alog=P, dtb=P,
             cu=NULL, n=1, T=256, nk=1, nv=2, dk=128, dv=128, scale=0.0, l2=1, s0=NULL, st=NULL, o=P, o_dtype=0,
             ws=P2, ws_bytes=1 << 40, stream=NULL)
    a.update(kw)
    return L.gdn_prefill_fused(a["x"], a["dtype"], a["xs"], a["cw"], a["cb"], a["K"], a["csi"], a["cso"], a["sl"],
                               a["a"], a["b"], a["ab_dtype"], a["alog"], a["dtb"], a["cu"], a["n"], a["T"], a["nk"],
                               a["nv"], a["dk"], a["dv"], a["scale"], a["l2"], a["s0"], a["st"], a["o"],
                               a["o_dtype"], a["ws"], a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=0), UNSUPPORTED),          # fp32 x is not built for the fused prefill
    (dict(dtype=5), INVALID),
    (dict(ab_dtype=4), INVALID),
    (dict(K=3, sl=2), UNSUPPORTED),
    (dict(sl=2), INVALID),                 # state_len < K - 1
    (dict(xs=100), INVALID),               # stride below conv_dim = 512
    (dict(xs=516), UNSUPPORTED),           # stride not a multiple of 8
    (dict(x=MIS), UNSUPPORTED),
    (dict(x=NULL), INVALID),
    (dict(cw=NULL), INVALID),
    (dict(a=NULL), INVALID),
    (dict(alog=NULL), INVALID),
    (dict(dtb=NULL), INVALID),
    (dict(nk=3, nv=4), INVALID),
    (dict(n=2), INVALID),                  # several sequences need cu_seqlens
    (dict(ws=NULL), INVALID),
    (dict(ws_bytes=16), WS_SMALL),
    (dict(dk=64, dv=64), UNSUPPORTED),
    (dict(csi=P, cso=ctypes.c_void_p(0x100000 + 256)), INVALID),   # overlapping conv states
])
def test_prefill_fused_argument_errors(L, kw, status):
    assert _prefill(L, **kw) == status
    assert gdn.gdn_last_error() != ""


def _prefill_norm(L, **kw):
    a = dict(x=P, dtype=1, xs=0, cw=P, cb=NULL, K=4, csi=NULL, cso=NULL, sl=3, a=P, b=P, ab_dtype=1, alog=P, dtb=P,
             cu=NULL, n=1, T=256, nk=1, nv=2, dk=128, dv=128, scale=0.0, l2=1, s0=NULL, st=NULL, z=P, z_dtype=1,
             nw=P, eps=1e-6, y=P, ws=P2, ws_bytes=1 << 40, stream=NULL)
    a.update(kw)
    return L.gdn_prefill_fused_norm(a["x"], a["dtype"], a["xs"], a["cw"], a["cb"], a["K"], a["csi"], a["cso"],
                                    a["sl"], a["a"], a["b"], a["ab_dtype"], a["alog"], a["dtb"], a["cu"], a["n"],
                                    a["T"], a["nk"], a["nv"], a["dk"], a["dv"], a["scale"], a["l2"], a["s0"],
                                    a["st"], a["z"], a["z_dtype"], a["nw"], a["eps"], a["y"], a["ws"],
                                    a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(z_dtype=0), UNSUPPORTED),        # only bf16 z is built
    (dict(z_dtype=7), INVALID),
    (dict(z=NULL), INVALID),
    (dict(z=MIS), UNSUPPORTED),
    (dict(nw=NULL), INVALID),
    (dict(eps=-1.0), INVALID),
    (dict(eps=float("nan")), INVALID),
    (dict(y=NULL), INVALID),
    (dict(dtype=0), UNSUPPORTED),          # the fused prefill's own checks apply as well
    (dict(ws_bytes=16), WS_SMALL),
    (dict(nk=3, nv=4), INVALID),
])
def test_prefill_fused_norm_argument_errors(L, kw, status):
    assert _prefill_norm(L, **kw) == status
    assert gdn.gdn_last_error() != ""


def _declared_arg_counts():
    """Number of parameters of every function declared in gdn.h (comments stripped)."""
    src = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    out = {}
    for name, args in re.findall(r"\b(gdn_[a-z0-9_]+)\s*\(([^)]*)\)\s*;", src, flags=re.S):
        args = args.strip()
        out[name] = 0 if args in ("", "void") else len(args.split(","))
    return out


def test_binding_signatures_match_the_header(L):
    """The ctypes binding declares the same number of arguments as the C header, for every entry point."""
    decl = _declared_arg_counts()
    assert len(decl) >= 10
    for name, n in decl.items():
        fn = getattr(L, name)
        assert fn.argtypes is not None, f"{name}: no argtypes in the binding"
        assert len(fn.argtypes) == n, f"{name}: header has {n} arguments, binding {len(fn.argtypes)}"


def _noalloc(L, **kw):
    a = dict(q=P, k=P, v=P, in_dtype=1, qs=0, ks=0, vs=0, a=P, b=P, ab_dtype=1, alog=P, dtb=P, cu=NULL, n=1, T=256,
             nk=1, nv=2, dk=128, dv=128, scale=0.0, l2=1, s0=NULL, st=NULL, o=P, o_dtype=0, stream=NULL)
    a.update(kw)
    return L.gdn_chunk_fwd_gated_noalloc(a["q"], a["k"], a["v"], a["in_dtype"], a["qs"], a["ks"], a["vs"], a["a"],
                                         a["b"], a["ab_dtype"], a["alog"], a["dtb"], a["cu"], a["n"], a["T"],
                                         a["nk"], a["nv"], a["dk"], a["dv"], a["scale"], a["l2"], a["s0"], a["st"],
                                         a["o"], a["o_dtype"], a["stream"])


def test_noalloc_scratch_limit_is_stated(L):
    assert gdn.gdn_chunk_fwd_noalloc_max_bytes() == 256 << 20
    # the prefill T=8192 (16 -> 32 heads) workload fits it; T=65536 does not
    assert gdn.gdn_chunk_fwd_workspace_size(8192, 1, 16, 32) <= gdn.gdn_chunk_fwd_noalloc_max_bytes()
    assert gdn.gdn_chunk_fwd_workspace_size(65536, 1, 16, 32) > gdn.gdn_chunk_fwd_noalloc_max_bytes()


@pytest.mark.parametrize("kw,status", [
    (dict(T=65536, nk=16, nv=32), WS_SMALL),   # workspace above the scratch array: rejected before any HIP call
    (dict(ab_dtype=4), INVALID),
    (dict(a=NULL), INVALID),
    (dict(alog=NULL), INVALID),
    (dict(nk=3, nv=4), INVALID),
    (dict(n=2), INVALID),                      # several sequences need cu_seqlens
    (dict(dk=64), UNSUPPORTED),
    (dict(q=MIS), UNSUPPORTED),
])
def test_chunk_fwd_gated_noalloc_argument_errors(L, kw, status):
    assert _noalloc(L, **kw) == status
    err = gdn.gdn_last_error()
    assert err.startswith("gdn_chunk_fwd_gated_noalloc")
    if status == WS_SMALL:
        assert "scratch" in err and str(256 << 20) in err


def test_launches_beyond_2_32_work_items_are_rejected_on_the_host(L):
    """One dispatch holds at most 2^32 - 1 work-items: every entry point rejects larger grids with
    UNSUPPORTED before enqueuing anything (no HIP call is reached with these arguments)."""
    n = 1 << 21   # 2^21 sequences x 8 value heads x 256 threads = 2^32 work-items
    assert _rec(L, n=n, T=n, nk=8, nv=8) == UNSUPPORTED
    assert _fused(L, n=n, T=n, nk=8, nv=8, n_slots=n) == UNSUPPORTED
    # chunk state kernel: 8 column slices x 256 threads per (sequence, value head)
    assert _chunk(L, cu=P, n=1 << 19, T=1 << 19, nk=4, nv=8) == UNSUPPORTED
    assert _noalloc(L, cu=P, n=1 << 19, T=1 << 19, nk=4, nv=8) in (UNSUPPORTED, WS_SMALL)
    # gated RMSNorm: 8 rows per 256-thread workgroup
    assert L.gdn_gated_rmsnorm(P, 0, P, 1, P, 1 << 30, 128, ctypes.c_float(1e-6), P2, 0, NULL) == UNSUPPORTED
    # gating: one thread per (token, head) in the worst case
    assert L.gdn_gating(P, P, 1, P, P, 1 << 30, 8, P2, P2, NULL) == UNSUPPORTED
    # conv update: one thread per (sequence, channel)
    assert L.gdn_causal_conv1d_update(P, 1, P, 3, P, NULL, 1 << 20, 1 << 12, 4, 1, P2, NULL) == UNSUPPORTED
