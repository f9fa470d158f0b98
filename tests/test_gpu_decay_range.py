"""Decay range on the GPU: steep per-token decays (log a far below the workloads'
clip at -8) in the middle of multi-chunk sequences, on every prefill method,
against the fp64 oracle.

The KDA row of the table on page "The argument, in one page" ("Everything, in one
table") singles out the per-channel decay's numerical range.  The chunk kernels
split decay factors around 16-token references while every token of a chunk has
log2 a >= -12 and switch a chunk with a steeper token to one exponential per
term, so the bar here is the ordinary one: 1e-4 for fp32 inputs, 2e-2 for bf16.
"""
import numpy as np
import pytest
import torch

import kda_recurrent_state_amd as kda
from kda_recurrent_state_amd.workloads import WORKLOADS, generate, generate_raw, scaled
from tests.parity import TOL, decode_as_sequence, log, max_rel_err, oracle_all

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
SINGLE, TWO = kda.METHOD_SINGLE, kda.METHOD_TWO_PASS
STEEP = [-9.0, -10.5, -12.0, -25.0, -80.0]
LENGTHS = [150, 47]     # sequence 0 spans five 32-token chunks
STRETCH = (40, 76)      # tokens of sequence 0 with the steep decay: crosses chunk ends at 64


def host(inp):
    return {k: (v.cpu() if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}


def steep_batch(dtype, dk, dv, steep, scalar=False, seed=0, stretch=STRETCH, lengths=LENGTHS):
    """Seeded batch with log a = `steep` on tokens stretch of sequence 0: on every
    channel for a scalar gate, else on two channels in three (the rest keep their
    ordinary decays and carry the state across the stretch)."""
    base = "kda_t64_d16_fp32" if dtype == torch.float32 else "kda_b2_h32_t32768_d128_bf16"
    w = scaled(WORKLOADS[base], n_seqs=len(lengths), heads=2, dk=dk, dv=dv, scalar_decay=scalar, s0_std=0.05)
    inp = generate(w, seed=seed, device=DEV, lengths=lengths)
    la = inp["log_a"].clone()
    a, b = stretch
    if scalar:
        la[a:b] = steep
    else:
        ch = torch.arange(dk, device=DEV) % 3 != 0
        la[a:b, :, ch] = steep
    inp["log_a"] = la.contiguous()
    return inp


def run(inp, **kw):
    o, ST = kda.chunk_fwd(inp["q"], inp["k"], inp["v"], inp["log_a"], inp["beta"], S0=inp["S0"],
                          cu_seqlens=inp["cu_seqlens"], **kw)
    torch.cuda.synchronize()
    return o, ST


def check(inp, o, ST, tol, order=0, what=""):
    assert torch.isfinite(o.float()).all() and torch.isfinite(ST).all(), "non-finite output"
    ro, rS = oracle_all(host(inp), order=order)
    eo, es = max_rel_err(o, ro), max_rel_err(ST, rS)
    log(f"  {what} err o {eo:.2e} S {es:.2e}")
    assert eo <= tol, f"o error {eo}"
    assert es <= tol, f"S_T error {es}"


@pytest.mark.parametrize("order", [0, 1])
@pytest.mark.parametrize("steep", STEEP)
@pytest.mark.parametrize("method", [SINGLE, TWO])
@pytest.mark.parametrize("dk", [64, 128])
def test_steep_bf16(dk, method, steep, order):
    log(f"steep bf16 dk={dk} method={method} log_a={steep} order={order}")
    inp = steep_batch(torch.bfloat16, dk, dk, steep, seed=dk + 3)
    o, ST = run(inp, method=method, order=order)
    check(inp, o, ST, TOL[torch.bfloat16], order, "bf16")


@pytest.mark.parametrize("order", [0, 1])
@pytest.mark.parametrize("steep", STEEP)
@pytest.mark.parametrize("dk", [32, 64, 128])
def test_steep_fp32(dk, steep, order):
    """fp32 inputs run the single-pass kernel (the two-pass one is bf16 only)."""
    log(f"steep fp32 dk={dk} log_a={steep} order={order}")
    inp = steep_batch(torch.float32, dk, dk, steep, seed=dk + 5)
    o, ST = run(inp, order=order)
    check(inp, o, ST, TOL[torch.float32], order, "fp32")


@pytest.mark.parametrize("steep", [-10.5, -80.0])
def test_steep_fp32_chunk64(steep):
    """C = 64 (compiled for fp32 at dk = dv = 16): four 16-token blocks per chunk."""
    log(f"steep fp32 C=64 log_a={steep}")
    inp = steep_batch(torch.float32, 16, 16, steep, seed=7)
    o, ST = run(inp, chunk_size=64)
    check(inp, o, ST, TOL[torch.float32], 0, "fp32 C=64")


@pytest.mark.parametrize("steep", [-12.0, -80.0])
@pytest.mark.parametrize("dtype,dk,method", [(torch.bfloat16, 128, TWO), (torch.bfloat16, 64, TWO),
                                             (torch.bfloat16, 128, SINGLE), (torch.float32, 32, SINGLE)])
def test_steep_scalar_gate(dtype, dk, method, steep):
    log(f"steep scalar gate {dtype} dk={dk} method={method} log_a={steep}")
    inp = steep_batch(dtype, dk, dk, steep, scalar=True, seed=dk + 9)
    o, ST = run(inp, method=method)
    check(inp, o, ST, TOL[dtype], 0, "scalar gate")


@pytest.mark.parametrize("method", [SINGLE, TWO])
def test_isolated_steep_tokens(method):
    """Single steep tokens scattered over the sequence (one at a chunk's first
    token, one at its last, one mid-block), each with a different decay."""
    log(f"isolated steep tokens method={method}")
    inp = steep_batch(torch.bfloat16, 128, 128, -9.0, seed=31, stretch=(0, 0))
    la = inp["log_a"].clone()
    for t, v in [(32, -40.0), (63, -15.0), (100, -200.0), (101, -13.0), (170, -60.0)]:
        la[t, :, ::2] = v
    inp["log_a"] = la.contiguous()
    o, ST = run(inp, method=method)
    check(inp, o, ST, 2e-2, 0, "isolated")


@pytest.mark.parametrize("method", [SINGLE, TWO])
def test_steep_everywhere(method):
    """Every token steep (all chunks take the exact path): log a ~ U[-30, -8]."""
    log(f"steep everywhere method={method}")
    inp = steep_batch(torch.bfloat16, 128, 128, -9.0, seed=37, stretch=(0, 0), lengths=[200, 33, 64])
    g = torch.Generator(device=DEV)
    g.manual_seed(37)
    inp["log_a"] = (-8.0 - 22.0 * torch.rand(inp["log_a"].shape, generator=g, device=DEV)).contiguous()
    o, ST = run(inp, method=method)
    check(inp, o, ST, 2e-2, 0, "all steep")


@pytest.mark.parametrize("method", [SINGLE, TWO])
def test_steep_two_pass_segments_and_snapshots(method):
    """Steep chunks with the smallest two-pass workspace (every chunk its own
    segment, so the marks are made and cleared once per segment) and with state
    snapshots; both agree with the oracle and with the plain call."""
    log(f"steep with segments and snapshots method={method}")
    inp = steep_batch(torch.bfloat16, 128, 128, -25.0, seed=41)
    o, ST = run(inp, method=method)
    check(inp, o, ST, 2e-2, 0, "plain")
    if method == TWO:
        least = kda.chunk_workspace_size(inp["q"], inp["v"], num_seqs=2, method=TWO, max_seqlen=150, minimum=True)
        ws = torch.empty(least, dtype=torch.uint8, device=DEV)
        o2, S2 = run(inp, method=TWO, workspace=ws, max_seqlen=150)
        assert torch.equal(o2, o) and torch.equal(S2, ST)
    o3, S3, snaps = kda.chunk_fwd_snapshots(inp["q"], inp["k"], inp["v"], inp["log_a"], inp["beta"],
                                            S0=inp["S0"], cu_seqlens=inp["cu_seqlens"], snapshot_every=32,
                                            method=method)
    torch.cuda.synchronize()
    assert torch.equal(o3, o) and torch.equal(S3, ST)
    assert snaps.shape[0] == 150 // 32 + 47 // 32


def test_steep_chunked_matches_recurrent():
    """The decode kernel takes a = exp(log a) per token and has no range limit;
    the chunked prefill agrees with a chain of decode steps through the stretch."""
    log("steep chunked vs recurrent")
    inp = steep_batch(torch.bfloat16, 128, 128, -25.0, seed=43, lengths=[100])
    o, ST = run(inp)
    S = inp["S0"].clone()
    outs = []
    for t in range(100):
        ot, S = kda.decode_step(inp["q"][t:t + 1], inp["k"][t:t + 1], inp["v"][t:t + 1],
                                inp["log_a"][t:t + 1], inp["beta"][t:t + 1], S)
        outs.append(ot)
    torch.cuda.synchronize()
    assert max_rel_err(torch.cat(outs), o) <= 2e-2
    assert max_rel_err(S, ST) <= 2e-2
    check(inp, o, ST, 2e-2, 0, "prefill")


@pytest.mark.parametrize("dk", [64, 128])
def test_prologue_unclipped_large_logits(dk):
    """The prologue's -softplus without a clip on large pre-activations (a ~ e^-200):
    finite, and equal to the oracle's fp64 prologue, on the two-pass method."""
    from oracle import kda_oracle
    log(f"prologue unclipped large logits dk={dk}")
    w = scaled(WORKLOADS["kda_varlen_64seq_h32_d128"], n_seqs=2, heads=2, dk=dk, dv=dk)
    inp = generate_raw(w, seed=47 + dk, device=DEV, lengths=[140, 60])
    x = inp["log_a"].clone()
    x[30:90] = x[30:90].abs() * 60.0 + 20.0   # softplus(x) from 20 to a few hundred
    inp["log_a"] = x.contiguous()
    pro = dict(normalize_k=True, beta_logits=True, log_a_raw=True, log_a_min=None)
    o, ST = kda.chunk_fwd(inp["q"], inp["k"], inp["v"], inp["log_a"], inp["beta"], S0=inp["S0"],
                          cu_seqlens=inp["cu_seqlens"], prologue=pro, method=TWO)
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all() and torch.isfinite(ST).all()
    h = host(inp)
    ro, rS = kda_oracle(h["q"], h["k"], h["v"], h["log_a"], h["beta"], S0=h["S0"],
                        cu_seqlens=h["cu_seqlens"].numpy(), pro=pro)
    eo, es = max_rel_err(o, ro), max_rel_err(ST, rS)
    log(f"  err o {eo:.2e} S {es:.2e}")
    assert eo <= 2e-2 and es <= 2e-2


def test_decode_steep():
    """Decode chains with log a down to -80 against the oracle."""
    log("decode steep")
    w = scaled(WORKLOADS["kda_decode_b256_h32_d128"], n_seqs=4, heads=2, steps=12)
    inp = generate(w, seed=53, device=DEV)
    la = inp["log_a"].clone()
    la[3:7, :, :, ::2] = -80.0
    la[8, :, :, 1::2] = -12.0
    inp["log_a"] = la.contiguous()
    S = inp["S"].clone()
    outs = []
    for t in range(12):
        ot, S = kda.decode_step(inp["q"][t], inp["k"][t], inp["v"][t], inp["log_a"][t], inp["beta"][t], S)
        outs.append(ot)
    torch.cuda.synchronize()
    seq, steps, N = decode_as_sequence(host(inp))
    ro, rS = oracle_all(seq)
    got = torch.stack(outs).transpose(0, 1).reshape(N * steps, *outs[0].shape[1:])
    eo, es = max_rel_err(got, ro), max_rel_err(S, rS)
    log(f"  err o {eo:.2e} S {es:.2e}")
    assert eo <= 2e-2 and es <= 2e-2
