"""The allocation-free chunk entry point against the one with a caller workspace.

gdn_chunk_fwd_gated_noalloc runs the same kernels as gdn_chunk_fwd_gated with
the library's per-device scratch array in place of the workspace, so its
outputs must equal that entry point's bit for bit. Four calls in a row go
through the C ABI on the same GPU, each smaller than the one before (the
prefill T=8192 workload, then one GPU's share of it under an 8-way head
split, which runs segment-parallel, then a varlen batch with initial
states, then a small fp32 call), so each call reuses the scratch the
previous one left behind; each is compared with a fresh
gdn_chunk_fwd_gated call.
"""
import pytest
import torch

import gated_deltanet_gdn_amd as gdn
import workloads as W
from gpu_common import dev

pytestmark = pytest.mark.gpu


def _inputs(name, seed=None):
    wl = W.WORKLOADS[name]
    x = W.chunk_inputs(wl)
    d = {k: (v.to(dev()) if isinstance(v, torch.Tensor) else v) for k, v in x.items()}
    return wl, d


def _small_varlen(dtype):
    g = torch.Generator().manual_seed(1234)
    lens = [300, 1, 64, 129]
    T = sum(lens)
    nk, nv = 2, 4
    cu = torch.tensor([0] + list(torch.tensor(lens).cumsum(0)), dtype=torch.int32)
    q = torch.randn(T, nk, 128, generator=g).to(dtype)
    k = torch.randn(T, nk, 128, generator=g).to(dtype)
    v = torch.randn(T, nv, 128, generator=g).to(dtype)
    a = torch.randn(T, nv, generator=g).to(dtype)
    b = torch.randn(T, nv, generator=g).to(dtype)
    A_log = torch.log(torch.empty(nv).uniform_(1, 16, generator=g))
    dt_bias = 0.1 * torch.randn(nv, generator=g)
    S0 = 0.02 * torch.randn(len(lens), nv, 128, 128, generator=g)
    d = dict(q=q, k=k, v=v, a=a, b=b, A_log=A_log, dt_bias=dt_bias, S0=S0, cu_seqlens=cu)
    return {kk: vv.to(dev()) for kk, vv in d.items()}


def _both(d, cu=None, S0=None):
    o_ref, st_ref = gdn.gdn_chunk_fwd_gated(d["q"], d["k"], d["v"], d["a"], d["b"], d["A_log"], d["dt_bias"],
                                            cu_seqlens=cu, initial_state=S0)
    o, st = gdn.gdn_chunk_fwd_gated_noalloc(d["q"], d["k"], d["v"], d["a"], d["b"], d["A_log"], d["dt_bias"],
                                            cu_seqlens=cu, initial_state=S0)
    torch.cuda.synchronize()
    return o, st, o_ref, st_ref


def test_noalloc_equals_workspace_entry_point_on_calls_of_shrinking_size():
    print("[case] noalloc: prefill_chunk_t8k", flush=True)
    wl, d = _inputs("prefill_chunk_t8k")
    need = gdn.gdn_chunk_fwd_workspace_size(wl.T, 1, wl.nk, wl.nv)
    assert need <= gdn.gdn_chunk_fwd_noalloc_max_bytes()
    o, st, o_ref, st_ref = _both(d)
    assert torch.isfinite(o).all()
    assert torch.equal(o, o_ref) and torch.equal(st, st_ref), "T=8192: no-alloc call differs"
    del d, o, st, o_ref, st_ref

    print("[case] noalloc: prefill_head_share_t8k (segment-parallel), with an initial state", flush=True)
    wl, d = _inputs("prefill_head_share_t8k")
    S0 = 0.05 * torch.randn(1, wl.nv, 128, 128, device=dev(), generator=torch.Generator(dev()).manual_seed(9))
    o, st, o_ref, st_ref = _both(d, None, S0)
    assert torch.isfinite(o).all()
    assert torch.equal(o, o_ref) and torch.equal(st, st_ref), "segment-parallel call: no-alloc call differs"
    del d, o, st, o_ref, st_ref

    print("[case] noalloc: varlen 4 sequences, bf16, initial states", flush=True)
    d = _small_varlen(torch.bfloat16)
    o, st, o_ref, st_ref = _both(d, d["cu_seqlens"], d["S0"])
    assert torch.equal(o, o_ref) and torch.equal(st, st_ref), "varlen bf16: no-alloc call differs"

    print("[case] noalloc: varlen 4 sequences, fp32", flush=True)
    d = _small_varlen(torch.float32)
    o, st, o_ref, st_ref = _both(d, d["cu_seqlens"], d["S0"])
    assert torch.equal(o, o_ref) and torch.equal(st, st_ref), "varlen fp32: no-alloc call differs"


def test_noalloc_rejects_calls_beyond_the_scratch_array():
    print("[case] noalloc: oversized call is rejected", flush=True)
    T, nk, nv = 65536, 16, 32
    assert gdn.gdn_chunk_fwd_workspace_size(T, 1, nk, nv) > gdn.gdn_chunk_fwd_noalloc_max_bytes()
    q = torch.zeros(T, nk, 128, device=dev(), dtype=torch.bfloat16)
    v = torch.zeros(T, nv, 128, device=dev(), dtype=torch.bfloat16)
    a = torch.zeros(T, nv, device=dev(), dtype=torch.bfloat16)
    p = torch.zeros(nv, device=dev())
    with pytest.raises(gdn.GdnError, match="scratch"):
        gdn.gdn_chunk_fwd_gated_noalloc(q, q, v, a, a, p, p)
