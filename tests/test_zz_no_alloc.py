"""The allocation-free prefill entry point (kda_chunk_fwd_noalloc) on the GPU:
two calls in a row, the second on a smaller input, each against kda_chunk_fwd
(the entry point with a caller-owned workspace) on the same inputs."""
import pytest
import torch

import kda_recurrent_state_amd as kda
from kda_recurrent_state_amd.workloads import WORKLOADS, generate, scaled
from tests.parity import TOL, log, max_rel_err

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def both(inp, **kw):
    args = (inp["q"], inp["k"], inp["v"], inp["log_a"], inp["beta"])
    ref = kda.chunk_fwd(*args, S0=inp["S0"], cu_seqlens=inp["cu_seqlens"], **kw)
    got = kda.chunk_fwd_noalloc(*args, S0=inp["S0"], cu_seqlens=inp["cu_seqlens"], **kw)
    torch.cuda.synchronize()
    return ref, got


def compare(ref, got, what):
    eo = max_rel_err(got[0], ref[0])
    es = 0.0 if ref[1] is None else max_rel_err(got[1], ref[1])
    same = torch.equal(got[0], ref[0]) and (ref[1] is None or torch.equal(got[1], ref[1]))
    log(f"  {what}: err o {eo:.2e} S {es:.2e} bit-identical {same}")
    assert eo <= TOL[torch.bfloat16] and es <= TOL[torch.bfloat16]


def test_noalloc_two_calls_second_smaller():
    # 1st: 2 x 16 heads x 8192 tokens at d = 128 needs several segments of the
    # 128 MiB scratch (32 units x 37,376 bytes per chunk: 112 chunks per segment)
    log("noalloc call 1: 2 x 16 heads x 8192 tokens, d = 128")
    w = scaled(WORKLOADS["kda_b2_h32_t32768_d128_bf16"], seqlen=8192, heads=16)
    big = generate(w, seed=61, device=DEV)
    compare(*both(big), "call 1")
    # 2nd, smaller and ragged, with a steep stretch (marked chunks re-formed in the scratch)
    log("noalloc call 2: ragged [300, 7, 161] x 2 heads, steep stretch")
    w2 = scaled(WORKLOADS["kda_varlen_64seq_h32_d128"], n_seqs=3, heads=2)
    small = generate(w2, seed=62, device=DEV, lengths=[300, 7, 161])
    la = small["log_a"].clone()
    la[100:140, :, ::2] = -30.0
    small["log_a"] = la.contiguous()
    compare(*both(small), "call 2")
    # 3rd: without S_T the running states live in the scratch too
    log("noalloc call 3: no final state")
    compare(*both(small, final_state=False), "call 3")


def test_noalloc_dk64_and_single_pass_shapes():
    log("noalloc dk = 64 (two-pass) and fp32 (single-pass, no scratch)")
    w = scaled(WORKLOADS["kda_varlen_64seq_h32_d128"], n_seqs=2, heads=3, dk=64, dv=64)
    inp = generate(w, seed=63, device=DEV, lengths=[500, 77])
    compare(*both(inp), "dk 64")
    w32 = scaled(WORKLOADS["kda_t64_d16_fp32"], n_seqs=2, heads=2, dk=32, dv=32)
    inp32 = generate(w32, seed=64, device=DEV, lengths=[90, 33])
    ref, got = both(inp32)
    assert torch.equal(ref[0], got[0]) and torch.equal(ref[1], got[1])


def test_noalloc_many_sequences_longest_first():
    """300 packed sequences: more state-pass workgroups than compute units, so
    the scratch also holds the longest-first order in front of the blocks; the
    results equal those of kda_chunk_fwd, with and without S_T."""
    import numpy as np
    log("noalloc 300 sequences longest first")
    rng = np.random.default_rng(65)
    lengths = rng.integers(0, 150, 300)
    lengths[5] = 600
    w = scaled(WORKLOADS["kda_varlen_64seq_h32_d128"], n_seqs=300, heads=1)
    inp = generate(w, seed=65, device=DEV, lengths=lengths.tolist())
    ref, got = both(inp)
    compare(ref, got, "300 sequences")
    assert torch.equal(ref[0], got[0]) and torch.equal(ref[1], got[1])
    compare(*both(inp, final_state=False), "300 sequences, no final state")


@pytest.mark.parametrize("packed", [False, True])
def test_noalloc_graph_replays(packed):
    """The call the entry point is for: captured in a HIP graph and replayed three
    times with eager work between, each replay bit-identical to the eager call."""
    log(f"noalloc under graph capture, packed={packed}")
    if packed:
        w = scaled(WORKLOADS["kda_varlen_64seq_h32_d128"], n_seqs=3, heads=4)
        x = generate(w, seed=66, device=DEV, lengths=[700, 33, 1290])
    else:
        w = scaled(WORKLOADS["kda_b2_h32_t32768_d128_bf16"], seqlen=2048, heads=4)
        x = generate(w, seed=66, device=DEV)
    T = x["q"].shape[0]
    args = (x["q"], x["k"], x["v"], x["log_a"], x["beta"])
    # max_seqlen given: the binding would otherwise read it from cu_seqlens on the host
    maxlen = int(max(x["lengths"])) if "lengths" in x else w.seqlen
    kw = dict(S0=x["S0"], cu_seqlens=x["cu_seqlens"], num_seqs=w.n_seqs, max_seqlen=maxlen)
    o_ref = torch.empty((T, w.heads, w.dv), dtype=w.dtype, device=DEV)
    S_ref = torch.empty((w.n_seqs, w.heads, w.dk, w.dv), dtype=torch.float32, device=DEV)
    kda.chunk_fwd_noalloc(*args, out=o_ref, final_state=S_ref, **kw)  # eager, also the first-call set-up
    torch.cuda.synchronize()
    o = torch.zeros_like(o_ref)
    S = torch.zeros_like(S_ref)
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            kda.chunk_fwd_noalloc(*args, out=o, final_state=S, **kw)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    junk = torch.randn(1 << 20, device=DEV)
    for r in range(3):
        o.fill_(7.0)
        S.fill_(-3.0)
        junk.mul_(1.0001)  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        same = torch.equal(o, o_ref) and torch.equal(S, S_ref)
        log(f"  replay {r}: bit-identical {same}")
        assert same, f"replay {r} differs from the eager call"
