"""Helpers shared by the GPU parity tests: error metric and oracle calls.

Error metric: err(x, r) = max|x - r| / max|r| over one output tensor (o or the
final state), in fp64, against the oracle fed the very same (already rounded)
inputs; the absolute error when r is all zero.  Bars: 1e-4 for fp32 inputs,
2e-2 for bf16 inputs (fp32 state).
"""
from __future__ import annotations

import sys

import numpy as np
import torch

from oracle import kda_oracle

TOL = {torch.float32: 1e-4, torch.bfloat16: 2e-2}


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def np64(t):
    return t.detach().to("cpu", torch.float64).numpy() if isinstance(t, torch.Tensor) else np.asarray(t, np.float64)


def max_rel_err(x, r):
    x, r = np64(x), np64(r)
    assert x.shape == r.shape, (x.shape, r.shape)
    if x.size == 0:
        return 0.0
    assert np.all(np.isfinite(x)), "non-finite values in GPU output"
    den = float(np.max(np.abs(r)))
    num = float(np.max(np.abs(x - r)))
    return num / den if den > 0 else num


def oracle_all(inp, order=0):
    """Oracle over the whole packed batch (all sequences and heads)."""
    return kda_oracle(inp["q"], inp["k"], inp["v"], inp["log_a"], inp["beta"], S0=inp.get("S0"),
                      cu_seqlens=inp["cu_seqlens"].cpu().numpy(), order=order)


def oracle_unit(inp, n, h, order=0):
    """Oracle for one (sequence n, head h) of a packed batch: (o [L, dv], S_T [dk, dv])."""
    cu = inp["cu_seqlens"].cpu().numpy()
    s, e = int(cu[n]), int(cu[n + 1])
    sl = lambda t: t[s:e, h:h + 1]
    S0 = inp.get("S0")
    S0u = None if S0 is None else S0[n:n + 1, h:h + 1]
    o, ST = kda_oracle(sl(inp["q"]), sl(inp["k"]), sl(inp["v"]), sl(inp["log_a"]), sl(inp["beta"]),
                       S0=S0u, order=order)
    return o[:, 0], ST[0, 0]


def decode_as_sequence(inp):
    """A chain of decode steps is one token per step of each sequence: repack the
    [steps, N, H, ...] tensors as N sequences of `steps` tokens for the oracle."""
    steps, N, H = inp["q"].shape[:3]
    tr = lambda t: t.transpose(0, 1).reshape((N * steps,) + tuple(t.shape[2:]))
    cu = np.arange(0, N * steps + 1, steps)
    out = dict(q=tr(inp["q"]), k=tr(inp["k"]), v=tr(inp["v"]), log_a=tr(inp["log_a"]),
               beta=tr(inp["beta"]), S0=inp["S"], cu_seqlens=torch.tensor(cu, dtype=torch.int32))
    return out, steps, N


def oracle_snapshots(inp, every, n, h=None):
    """Oracle states of sequence n after each whole `every` tokens: [R_n, H, dk, dv]
    (or [R_n, dk, dv] for one head h).  The recurrence is run piece by piece,
    each piece of `every` tokens starting from the fp64 state the previous one
    ended with, which is the token-by-token recurrence itself cut at those points."""
    cu = inp["cu_seqlens"].cpu().numpy()
    s, e = int(cu[n]), int(cu[n + 1])
    hs = slice(None) if h is None else slice(h, h + 1)
    S0 = inp.get("S0")
    S = None if S0 is None else np64(S0[n:n + 1, hs])
    out = []
    for p in range((e - s) // every):
        a, b = s + p * every, s + (p + 1) * every
        sl = lambda t: t[a:b, hs]
        _, S = kda_oracle(sl(inp["q"]), sl(inp["k"]), sl(inp["v"]), sl(inp["log_a"]), sl(inp["beta"]), S0=S)
        out.append(S[0] if h is None else S[0, 0])
    q = inp["q"]
    shape = ((q.shape[1],) if h is None else ()) + (q.shape[2], inp["v"].shape[2])
    return np.stack(out) if out else np.zeros((0,) + shape)
