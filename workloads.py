"""Seeded synthetic workloads for the Gated DeltaNet core.

This module only draws random inputs; it holds none of the method's
arithmetic. It is the one module that both the GPU-path tests/bench and the
CPU oracle's callers share.

Recipe (distributions chosen to match the published layer's inputs: conv +
SiLU output for q/k/v is O(1), a/b are raw projection outputs, A_log = log of
a decay rate in [1, 16], dt_bias a small bias):
  * every tensor has its own torch.Generator stream seeded with
    ``1000 * config_seed + tensor_index`` (tensor index order: lengths, q, k,
    v, a, b, A_log, dt_bias, S0, x, conv_state, conv_w, z, norm_w);
  * draws are fp32, then rounded to bf16 (round-to-nearest-even, torch's own
    conversion) where the workload is bf16; consumers read the rounded values;
  * q, k, v, a, b, x, z ~ N(0, 1); A_log = log U[1, 16]; dt_bias ~ N(0, 0.1);
    initial recurrent state ~ N(0, 0.02) where nonzero; conv weight ~
    U(-1/2, 1/2) (the nn.Conv1d default bound 1/sqrt(K) at K = 4); norm weight
    ~ N(0, 0.1); the decode conv state ~ N(0, 1);
  * varlen lengths ~ U{512 .. 16384} (inclusive), from numpy PCG64.
N(m, s) means standard deviation s.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch

IDX = dict(lengths=0, q=1, k=2, v=3, a=4, b=5, A_log=6, dt_bias=7, S0=8, x=9,
           conv_state=10, conv_w=11, z=12, norm_w=13)


@dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    kind: str                  # "chunk", "decode", "fused"
    dtype: str                 # "f32" or "bf16"  (q/k/v/a/b/x/z dtype)
    T: int = 0                 # total tokens (single sequence) -- 0 for varlen/decode
    n_seqs: int = 1
    nk: int = 16
    nv: int = 32
    dk: int = 128
    dv: int = 128
    chunk: int = 64
    s0_std: float = 0.0        # 0 => zero initial state
    len_range: tuple = ()      # varlen (lo, hi) inclusive
    conv_k: int = 4
    state_len: int = 3
    extra: dict = field(default_factory=dict)

    @property
    def conv_dim(self):
        return 2 * self.nk * self.dk + self.nv * self.dv


WORKLOADS = {
    "tiny_chunk_f32": Workload("tiny_chunk_f32", 1, "chunk", "f32", T=256, nk=1, nv=2),
    "prefill_chunk_t8k": Workload("prefill_chunk_t8k", 2, "chunk", "bf16", T=8192, nk=16, nv=32),
    "varlen_prefill_8seq": Workload("varlen_prefill_8seq", 3, "chunk", "bf16", n_seqs=8,
                                    nk=16, nv=32, s0_std=0.02, len_range=(512, 16384)),
    "decode_256seq": Workload("decode_256seq", 4, "decode", "bf16", n_seqs=256, nk=16, nv=32,
                              s0_std=0.02),
    "long_fused_t256k": Workload("long_fused_t256k", 5, "fused", "bf16", T=262144, nk=16, nv=64),
    # one GPU's share of prefill_chunk_t8k when its 16 key heads are split over 8 GPUs: few column
    # slices, the shape the segment-parallel prefill is for
    "prefill_head_share_t8k": Workload("prefill_head_share_t8k", 7, "chunk", "bf16", T=8192, nk=2, nv=4),
    # decode with multi-token prediction: each sequence carries 1 + 3 draft tokens
    "decode_mtp_256x4": Workload("decode_mtp_256x4", 6, "decode", "bf16", n_seqs=256, nk=16, nv=32,
                                 s0_std=0.02, extra=dict(tokens_per_seq=4)),
}

TORCH_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16}


def _gen(seed, idx, device):
    g = torch.Generator(device=device)
    g.manual_seed(1000 * seed + idx)
    return g


def randn(shape, seed, idx, dtype="f32", std=1.0, device="cpu"):
    g = _gen(seed, idx, device)
    x = torch.randn(shape, generator=g, dtype=torch.float32, device=device)
    if std != 1.0:
        x.mul_(std)
    return x.to(TORCH_DTYPE[dtype])


def uniform(shape, seed, idx, lo, hi, device="cpu"):
    g = _gen(seed, idx, device)
    x = torch.rand(shape, generator=g, dtype=torch.float32, device=device)
    return x.mul_(hi - lo).add_(lo)


def a_log(nv, seed, device="cpu"):
    # A_log = log U[1, 16]
    return torch.log(uniform((nv,), seed, IDX["A_log"], 1.0, 16.0, device))


def varlen_lengths(wl: Workload):
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([wl.seed, IDX["lengths"]])))
    lo, hi = wl.len_range
    return rng.integers(lo, hi + 1, size=wl.n_seqs).astype(np.int64)


def cu_from_lengths(lengths):
    cu = np.zeros(len(lengths) + 1, dtype=np.int64)
    cu[1:] = np.cumsum(lengths)
    return cu


def chunk_inputs(wl: Workload, device="cpu", T=None, lengths=None, s0_std=None):
    """q, k, v, a, b, A_log, dt_bias, cu_seqlens (int32), S0 for a chunk workload.

    ``T`` / ``lengths`` override the workload's token layout (used for reduced
    parity cases); everything else keeps the workload's recipe.
    """
    if lengths is None:
        lengths = varlen_lengths(wl) if wl.len_range else np.array([T or wl.T], dtype=np.int64)
    lengths = np.asarray(lengths, dtype=np.int64)
    cu = cu_from_lengths(lengths)
    T_tot = int(cu[-1])
    n = len(lengths)
    s, dt = wl.seed, wl.dtype
    out = dict(
        q=randn((T_tot, wl.nk, wl.dk), s, IDX["q"], dt, device=device),
        k=randn((T_tot, wl.nk, wl.dk), s, IDX["k"], dt, device=device),
        v=randn((T_tot, wl.nv, wl.dv), s, IDX["v"], dt, device=device),
        a=randn((T_tot, wl.nv), s, IDX["a"], dt, device=device),
        b=randn((T_tot, wl.nv), s, IDX["b"], dt, device=device),
        A_log=a_log(wl.nv, s, device),
        dt_bias=randn((wl.nv,), s, IDX["dt_bias"], "f32", std=0.1, device=device),
        cu_seqlens=torch.tensor(cu, dtype=torch.int32, device=device),
        lengths=lengths,
    )
    std = wl.s0_std if s0_std is None else s0_std
    out["S0"] = (randn((n, wl.nv, wl.dk, wl.dv), s, IDX["S0"], "f32", std=std, device=device)
                 if std > 0 else None)
    return out


def decode_inputs(wl: Workload, device="cpu", n_seqs=None):
    """Inputs of one decode step: conv update on packed QKV, gating, recurrent update."""
    n = n_seqs or wl.n_seqs
    s, dt = wl.seed, wl.dtype
    C = wl.conv_dim
    return dict(
        x=randn((n, C), s, IDX["x"], dt, device=device),
        conv_state=randn((n, C, wl.state_len), s, IDX["conv_state"], dt, device=device),
        conv_w=uniform((C, wl.conv_k), s, IDX["conv_w"], -0.5, 0.5, device),
        a=randn((n, wl.nv), s, IDX["a"], dt, device=device),
        b=randn((n, wl.nv), s, IDX["b"], dt, device=device),
        A_log=a_log(wl.nv, s, device),
        dt_bias=randn((wl.nv,), s, IDX["dt_bias"], "f32", std=0.1, device=device),
        state=randn((n, wl.nv, wl.dk, wl.dv), s, IDX["S0"], "f32", std=wl.s0_std, device=device),
    )


def decode_mtp_inputs(wl: Workload, lengths, device="cpu"):
    """Inputs of a decode step with lengths[n] tokens for sequence n (1 + draft tokens):
    packed x [sum, conv_dim], a, b [sum, nv], per-sequence conv and recurrent states, cu_seqlens."""
    n, T = len(lengths), int(sum(lengths))
    s, dt = wl.seed, wl.dtype
    C = wl.conv_dim
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lengths)]), dtype=torch.int32)
    return dict(
        x=randn((T, C), s, IDX["x"], dt, device=device),
        conv_state=randn((n, C, wl.state_len), s, IDX["conv_state"], dt, device=device),
        conv_w=uniform((C, wl.conv_k), s, IDX["conv_w"], -0.5, 0.5, device),
        a=randn((T, wl.nv), s, IDX["a"], dt, device=device),
        b=randn((T, wl.nv), s, IDX["b"], dt, device=device),
        A_log=a_log(wl.nv, s, device),
        dt_bias=randn((wl.nv,), s, IDX["dt_bias"], "f32", std=0.1, device=device),
        state=randn((n, wl.nv, wl.dk, wl.dv), s, IDX["S0"], "f32", std=wl.s0_std, device=device),
        cu_seqlens=cu.to(device),
    )


def fused_inputs(wl: Workload, device="cpu", T=None):
    """Inputs of the long prefill pipeline: conv+SiLU -> gating -> chunk -> gated RMSNorm."""
    T = T or wl.T
    s, dt = wl.seed, wl.dtype
    C = wl.conv_dim
    return dict(
        x=randn((T, C), s, IDX["x"], dt, device=device),
        conv_w=uniform((C, wl.conv_k), s, IDX["conv_w"], -0.5, 0.5, device),
        a=randn((T, wl.nv), s, IDX["a"], dt, device=device),
        b=randn((T, wl.nv), s, IDX["b"], dt, device=device),
        A_log=a_log(wl.nv, s, device),
        dt_bias=randn((wl.nv,), s, IDX["dt_bias"], "f32", std=0.1, device=device),
        z=randn((T, wl.nv, wl.dv), s, IDX["z"], dt, device=device),
        norm_w=randn((wl.dv,), s, IDX["norm_w"], "f32", std=0.1, device=device),
    )
