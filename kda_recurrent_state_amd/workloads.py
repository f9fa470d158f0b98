"""Seeded synthetic workloads for the KDA / Gated DeltaNet state layer.

This module only draws inputs: it holds none of the layer's arithmetic and is
shared by the tests (which feed the same tensors to the oracle and to the GPU
path) and by the benchmark.  Shapes follow the hybrid-model layers the pages
describe (three linear layers per attention layer, key/value width 128, long
contexts and large decode batches); the pages' own serving benchmark data is
not used, these synthetic tensors stand in for it.

Distributions (N(mu, s) means mean mu and standard deviation s):
  q, v ~ N(0, 1); k ~ N(0, 1) then L2-normalised per (token, head) in fp32,
  all three then rounded to the working dtype (bf16 round-to-nearest-even);
  beta = sigmoid(N(0, 1)); log_a = -softplus(N(0, s_a)), optionally clipped to
  [clip, 0], one value per key channel (KDA) or per (token, head) (GDN);
  S0 ~ N(0, s_0) in fp32, or absent (zero state).
Draw order, from one torch generator seeded with ``seed``: q, k, v, log_a, beta,
S0.  Variable lengths are drawn first, from numpy's default_rng(seed).
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    name: str
    kind: str  # "prefill" or "decode"
    n_seqs: int
    heads: int
    dk: int
    dv: int
    dtype: torch.dtype
    scalar_decay: bool
    seqlen: int = 0  # fixed length per sequence (prefill)
    len_range: tuple = ()  # (lo, hi) inclusive, variable lengths (prefill)
    la_std: float = 1.0
    la_clip: float | None = None
    s0_std: float = 0.0  # 0 -> no initial state (zeros)
    steps: int = 1  # decode: chained steps
    chunk: int = 64
    note: str = field(default="", compare=False)


WORKLOADS = {
    "kda_t64_d16_fp32": Workload(
        "kda_t64_d16_fp32", "prefill", 1, 1, 16, 16, torch.float32, False, seqlen=64,
        note="KDA recurrence, B=1, H=1, T=64, dk=dv=16, fp32, S0=0"),
    "gdn_h16_t4096_d128_bf16": Workload(
        "gdn_h16_t4096_d128_bf16", "prefill", 1, 16, 128, 128, torch.bfloat16, True,
        seqlen=4096, note="Gated DeltaNet chunked prefill, B=1, H=16, T=4096, C=64, S0=0"),
    "kda_b2_h32_t32768_d128_bf16": Workload(
        "kda_b2_h32_t32768_d128_bf16", "prefill", 2, 32, 128, 128, torch.bfloat16, False,
        seqlen=32768, la_std=2.0, la_clip=-8.0, s0_std=0.02,
        note="KDA chunked prefill, B=2, H=32, T=32768, log_a clipped to [-8,0], S0~N(0,0.02)"),
    "kda_decode_b256_h32_d128": Workload(
        "kda_decode_b256_h32_d128", "decode", 256, 32, 128, 128, torch.bfloat16, False,
        s0_std=0.05, steps=100,
        note="KDA decode step, 256 sequences x H=32, fp32 state S~N(0,0.05), 100 chained steps"),
    "kda_varlen_64seq_h32_d128": Workload(
        "kda_varlen_64seq_h32_d128", "prefill", 64, 32, 128, 128, torch.bfloat16, False,
        len_range=(512, 16384), la_std=2.0, la_clip=-8.0, s0_std=0.02,
        note="KDA packed varlen prefill, 64 sequences, lengths U[512,16384], H=32"),
}


def scaled(w: Workload, **changes) -> Workload:
    """The same distributions at other sizes (tests use this for small cases)."""
    return replace(w, **changes)


def _lengths(w: Workload, seed: int) -> np.ndarray:
    if w.len_range:
        lo, hi = w.len_range
        return np.random.default_rng(seed).integers(lo, hi + 1, size=w.n_seqs)
    return np.full(w.n_seqs, w.seqlen, dtype=np.int64)


def generate_raw(w: Workload, seed: int, device="cpu", lengths=None, k_scale: float = 3.0):
    """The same batch before the input prologue: k unnormalised (scaled by
    k_scale), log_a as the pre-activation x of log a = -softplus(x) and beta as
    logits, for calls with an input prologue.  Other tensors as generate()."""
    out = generate(w, seed, device, lengths)
    g = torch.Generator(device=device)
    g.manual_seed(seed + 7919)
    f32 = torch.float32
    k = torch.randn(out["k"].shape, generator=g, device=device, dtype=f32) * k_scale
    la = torch.randn(out["log_a"].shape, generator=g, device=device, dtype=f32) * w.la_std
    beta = torch.randn(out["beta"].shape, generator=g, device=device, dtype=f32)
    out.update(k=k.to(w.dtype), log_a=la.contiguous(), beta=beta.contiguous())
    return out


def generate(w: Workload, seed: int, device="cpu", lengths=None):
    """Draw one batch.  Prefill returns q/k/v [T,H,d], log_a [T,H,dk] or [T,H],
    beta [T,H], S0 [N,H,dk,dv] or None, cu_seqlens int32 [N+1] (all on device).
    Decode returns the same per-token tensors with a leading step axis
    ([steps, N, H, d], one token per sequence per step) and S [N,H,dk,dv]."""
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    f32 = torch.float32
    if w.kind == "decode":
        lead = (w.steps, w.n_seqs, w.heads)
        lens = None
    else:
        lens = np.asarray(lengths if lengths is not None else _lengths(w, seed), dtype=np.int64)
        lead = (int(lens.sum()), w.heads)

    def normal(shape, std=1.0):
        x = torch.randn(shape, generator=g, device=device, dtype=f32)
        return x * std if std != 1.0 else x

    q = normal(lead + (w.dk,))
    k = normal(lead + (w.dk,))
    k = k / torch.linalg.vector_norm(k, dim=-1, keepdim=True)
    v = normal(lead + (w.dv,))
    la = -torch.nn.functional.softplus(normal(lead if w.scalar_decay else lead + (w.dk,), w.la_std))
    if w.la_clip is not None:
        la = la.clamp(min=w.la_clip, max=0.0)
    beta = torch.sigmoid(normal(lead))
    state_shape = (w.n_seqs, w.heads, w.dk, w.dv)
    S0 = normal(state_shape, w.s0_std) if w.s0_std > 0 else None
    out = dict(q=q.to(w.dtype), k=k.to(w.dtype), v=v.to(w.dtype),
               log_a=la.contiguous(), beta=beta.contiguous())
    if w.kind == "decode":
        out["S"] = S0 if S0 is not None else torch.zeros(state_shape, device=device, dtype=f32)
    else:
        cu = np.zeros(w.n_seqs + 1, dtype=np.int64)
        cu[1:] = np.cumsum(lens)
        out["S0"] = S0
        out["cu_seqlens"] = torch.tensor(cu, dtype=torch.int32, device=device)
        out["lengths"] = lens
    return out
