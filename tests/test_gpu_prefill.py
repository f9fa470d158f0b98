"""Chunked prefill on the GPU against the fp64 oracle, plus self-consistency."""
import numpy as np
import pytest
import torch

import kda_recurrent_state_amd as kda
from kda_recurrent_state_amd.workloads import WORKLOADS, generate, scaled
from tests.parity import TOL, log, max_rel_err, np64, oracle_all

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def gpu_prefill(inp, **kw):
    o, ST = kda.chunk_fwd(inp["q"], inp["k"], inp["v"], inp["log_a"], inp["beta"], S0=inp["S0"],
                          cu_seqlens=inp["cu_seqlens"], **kw)
    torch.cuda.synchronize()
    return o, ST


def check_all(inp, o, ST, tol, what=""):
    ro, rS = oracle_all({k: (v.cpu() if isinstance(v, torch.Tensor) else v) for k, v in inp.items()})
    eo, es = max_rel_err(o, ro), max_rel_err(ST, rS)
    log(f"  {what} err o {eo:.2e} S {es:.2e}")
    assert eo <= tol, f"o error {eo}"
    assert es <= tol, f"S_T error {es}"
    return eo, es


def test_prefill_kda_t64_d16_fp32():
    """B=1, H=1, T=64, dk=dv=16, fp32 inputs, zero initial state: 1e-4."""
    log("prefill C1: KDA T=64 d=16 fp32")
    inp = generate(WORKLOADS["kda_t64_d16_fp32"], seed=0, device=DEV)
    o, ST = gpu_prefill(inp)
    check_all(inp, o, ST, 1e-4, "C1")


@pytest.mark.parametrize("dk,dv", [(16, 16), (32, 32), (64, 64), (32, 16), (64, 32), (128, 128), (128, 16)])
@pytest.mark.parametrize("scalar", [False, True])
def test_prefill_fp32_varlen(dk, dv, scalar):
    log(f"prefill fp32 varlen dk={dk} dv={dv} scalar={scalar}")
    w = scaled(WORKLOADS["kda_varlen_64seq_h32_d128"], n_seqs=4, heads=2, dk=dk, dv=dv, dtype=torch.float32,
               scalar_decay=scalar)
    inp = generate(w, seed=dk * 3 + dv + scalar, device=DEV, lengths=[37, 0, 96, 5])
    o, ST = gpu_prefill(inp)
    check_all(inp, o, ST, 1e-4)


SINGLE, TWO = kda.METHOD_SINGLE, kda.METHOD_TWO_PASS


def documented_unsupported(dtype, dk, dv, method=0, split=0):
    """Shapes the header documents as not compiled: the two-pass method is bf16
    with dk 64 or 128 only, and every dv slice (dv / split) is 16, 32 or 64."""
    if method == TWO and not (dtype == torch.bfloat16 and dk in (64, 128)):
        return True
    return split > 0 and dv // split not in (16, 32, 64)


def run_method(inp, method, unsupported=False, **kw):
    """Prefill with an explicit method.  For a shape documented as not compiled
    the call must refuse with KDA_ERR_UNSUPPORTED (returns None)."""
    if unsupported:
        with pytest.raises(kda.KdaError) as e:
            gpu_prefill(inp, method=method, **kw)
        assert e.value.status == 2, e.value
        log(f"  refused as documented: {e.value}")
        return None
    return gpu_prefill(inp, method=method, **kw)


@pytest.mark.parametrize("method", [SINGLE, TWO])
@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 64), (32, 32), (128, 64), (64, 128), (128, 32)])
@pytest.mark.parametrize("scalar", [False, True])
def test_prefill_bf16_varlen(dk, dv, scalar, method):
    log(f"prefill bf16 varlen dk={dk} dv={dv} scalar={scalar} method={method}")
    w = scaled(WORKLOADS["kda_varlen_64seq_h32_d128"], n_seqs=4, heads=3, dk=dk, dv=dv, scalar_decay=scalar)
    inp = generate(w, seed=dk + dv + scalar, device=DEV, lengths=[45, 0, 170, 96])
    res = run_method(inp, method, documented_unsupported(torch.bfloat16, dk, dv, method))
    if res is not None:
        check_all(inp, *res, 2e-2)


@pytest.mark.parametrize("dk,dv", [(64, 64), (128, 128)])
def test_two_pass_segments(dk, dv):
    """The two-pass method with the smallest workspace (one chunk per segment),
    a middle one, and the preferred one agree with the oracle and each other;
    without S_T the running state lives in the workspace."""
    chunk = 32
    log(f"two-pass segments dk={dk} dv={dv}")
    w = scaled(WORKLOADS["kda_varlen_64seq_h32_d128"], n_seqs=3, heads=2, dk=dk, dv=dv)
    inp = generate(w, seed=21 + dk, device=DEV, lengths=[300, 7, 161])
    q, v = inp["q"], inp["v"]
    least = kda.chunk_workspace_size(q, v, num_seqs=3, chunk_size=chunk, method=TWO, max_seqlen=300,
                                     minimum=True)
    pref = kda.chunk_workspace_size(q, v, num_seqs=3, chunk_size=chunk, method=TWO, max_seqlen=300)
    assert 0 < least <= pref
    ref = None
    for nbytes in sorted({least, least + (pref - least) // 2, pref}):
        ws = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
        o, ST = run_method(inp, TWO, chunk_size=chunk, workspace=ws, max_seqlen=300)
        check_all(inp, o, ST, 2e-2, f"workspace {nbytes}")
        o2, none = run_method(inp, TWO, chunk_size=chunk, workspace=ws, max_seqlen=300, final_state=False)
        assert none is None and torch.equal(o2, o)
        if ref is None:
            ref = (o, ST)
        else:
            assert torch.equal(o, ref[0]) and torch.equal(ST, ref[1])  # segmenting is exact


@pytest.mark.parametrize("n_seqs", [300, 304])
def test_prefill_many_sequences_longest_first(n_seqs):
    """More state-pass workgroups than compute units: the state pass takes the
    sequences longest first (300 units: rank order; 304: ranks dealt over the
    eight XCDs).  Lengths repeat, include empty sequences and one long one, so
    ties and empty units are ranked too; the preferred and the smallest
    workspace (a segment per chunk) both match the oracle."""
    log(f"prefill {n_seqs} sequences longest first")
    rng = np.random.default_rng(n_seqs)
    lengths = rng.integers(0, 120, n_seqs)
    lengths[rng.integers(0, n_seqs, 20)] = 0
    lengths[7] = 900
    lengths[rng.integers(0, n_seqs, 30)] = 64
    w = scaled(WORKLOADS["kda_varlen_64seq_h32_d128"], n_seqs=n_seqs, heads=1)
    inp = generate(w, seed=40 + n_seqs, device=DEV, lengths=lengths.tolist())
    q, v = inp["q"], inp["v"]
    least = kda.chunk_workspace_size(q, v, num_seqs=n_seqs, method=TWO, max_seqlen=900, minimum=True)
    ref = None
    for ws in (None, torch.empty(least, dtype=torch.uint8, device=DEV)):
        o, ST = run_method(inp, TWO, workspace=ws, max_seqlen=900)
        if ref is None:
            check_all(inp, o, ST, 2e-2, "preferred workspace")
            ref = (o, ST)
        else:
            assert torch.equal(o, ref[0]) and torch.equal(ST, ref[1])  # segmenting is exact


@pytest.mark.parametrize("n_seqs", [2500, 4097])
def test_prefill_thousands_of_short_sequences(n_seqs):
    """2500 sequences: the rank kernel reads the lengths in three LDS tiles of
    1024 and the last of its 10 workgroups is partly idle; 4097 sequences are
    past the ranked maximum and run in index order.  Short lengths with many
    ties and empty sequences; every unit against the oracle."""
    log(f"prefill {n_seqs} short sequences")
    rng = np.random.default_rng(n_seqs)
    lengths = rng.integers(0, 24, n_seqs)
    lengths[rng.integers(0, n_seqs, n_seqs // 10)] = 0
    lengths[n_seqs // 2] = 200
    w = scaled(WORKLOADS["kda_varlen_64seq_h32_d128"], n_seqs=n_seqs, heads=1)
    inp = generate(w, seed=50 + n_seqs, device=DEV, lengths=lengths.tolist())
    o, ST = run_method(inp, TWO, max_seqlen=200)
    check_all(inp, o, ST, 2e-2, f"{n_seqs} sequences")


def test_two_pass_matches_single_pass():
    log("two-pass vs single-pass, d=128")
    w = scaled(WORKLOADS["kda_b2_h32_t32768_d128_bf16"], seqlen=1000, heads=2)
    inp = generate(w, seed=22, device=DEV)
    o1, S1 = run_method(inp, SINGLE)
    o2, S2 = run_method(inp, TWO)
    check_all(inp, o2, S2, 2e-2, "two-pass")
    assert max_rel_err(o2, o1) <= 2e-2 and max_rel_err(S2, S1) <= 2e-2


@pytest.mark.parametrize("method", [SINGLE, TWO])
@pytest.mark.parametrize("split", [1, 2, 4, 8])
def test_prefill_dv_split_invariance(split, method):
    """Splitting dv over workgroups changes nothing beyond rounding."""
    log(f"prefill dv_split={split} method={method}")
    w = scaled(WORKLOADS["kda_b2_h32_t32768_d128_bf16"], seqlen=200, heads=2, dk=64, dv=64)
    inp = generate(w, seed=5, device=DEV)
    res = run_method(inp, method, documented_unsupported(torch.bfloat16, 64, 64, method, split), dv_split=split)
    if res is not None:
        check_all(inp, *res, 2e-2, f"split {split}")


def test_prefill_chunk64_matches_chunk32():
    log("prefill chunk 64 vs 32")
    w = scaled(WORKLOADS["kda_b2_h32_t32768_d128_bf16"], seqlen=300, heads=2, dk=32, dv=32)
    inp = generate(w, seed=6, device=DEV)
    o32, S32 = gpu_prefill(inp, chunk_size=32)
    o64, S64 = gpu_prefill(inp, chunk_size=64)
    check_all(inp, o64, S64, 2e-2, "C=64")
    assert max_rel_err(o64, o32) <= 2e-2 and max_rel_err(S64, S32) <= 2e-2


def test_prefill_continuation_and_alias():
    """Split a sequence at a point that is not a chunk multiple, feed S_T back as
    S0 (written in place over S0), compare with one pass."""
    log("prefill continuation")
    w = scaled(WORKLOADS["kda_b2_h32_t32768_d128_bf16"], n_seqs=1, seqlen=333, heads=2)
    inp = generate(w, seed=7, device=DEV)
    o, ST = gpu_prefill(inp)
    cut = 77
    part = lambda t, a, b: t[a:b].contiguous()
    S = inp["S0"].clone()
    o1, _ = kda.chunk_fwd(part(inp["q"], 0, cut), part(inp["k"], 0, cut), part(inp["v"], 0, cut),
                          part(inp["log_a"], 0, cut), part(inp["beta"], 0, cut), S0=S, final_state=S)
    o2, _ = kda.chunk_fwd(part(inp["q"], cut, 333), part(inp["k"], cut, 333), part(inp["v"], cut, 333),
                          part(inp["log_a"], cut, 333), part(inp["beta"], cut, 333), S0=S, final_state=S)
    torch.cuda.synchronize()
    assert max_rel_err(torch.cat([o1, o2]), o) <= 2e-2
    assert max_rel_err(S, ST) <= 2e-2
    check_all(inp, o, ST, 2e-2, "one pass")


@pytest.mark.parametrize("method", [SINGLE, TWO])
def test_prefill_deterministic(method):
    log(f"prefill determinism method={method}")
    w = scaled(WORKLOADS["kda_b2_h32_t32768_d128_bf16"], seqlen=256, heads=4)
    inp = generate(w, seed=8, device=DEV)
    a = run_method(inp, method)
    b = run_method(inp, method)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


@pytest.mark.parametrize("method", [SINGLE, TWO])
def test_prefill_empty_and_no_state(method):
    """All sequences empty: S_T = S0; S0 = None means zeros."""
    log(f"prefill empty sequences method={method}")
    w = scaled(WORKLOADS["kda_varlen_64seq_h32_d128"], n_seqs=3, heads=2)
    inp = generate(w, seed=9, device=DEV, lengths=[0, 0, 0])
    o, ST = run_method(inp, method)
    assert torch.equal(ST, inp["S0"])
    inp2 = generate(w, seed=10, device=DEV, lengths=[20, 0, 64])
    inp2["S0"] = None
    o2, ST2 = run_method(inp2, method)
    check_all(inp2, o2, ST2, 2e-2, "S0=None")


def test_chunked_matches_recurrent():
    """Prefill and a chain of single-token decode steps agree on the GPU."""
    log("chunked vs recurrent")
    w = scaled(WORKLOADS["kda_b2_h32_t32768_d128_bf16"], n_seqs=1, seqlen=70, heads=3)
    inp = generate(w, seed=11, device=DEV)
    o, ST = gpu_prefill(inp)
    S = inp["S0"].clone()
    outs = []
    for t in range(70):
        ot, S = kda.decode_step(inp["q"][t:t + 1], inp["k"][t:t + 1], inp["v"][t:t + 1],
                                inp["log_a"][t:t + 1], inp["beta"][t:t + 1], S)
        outs.append(ot)
    torch.cuda.synchronize()
    assert max_rel_err(torch.cat(outs), o) <= 2e-2
    assert max_rel_err(S, ST) <= 2e-2


# ---- full sizes, in the launch configuration the benchmark times ------------------------
def test_prefill_gdn_h16_t4096_full():
    """Gated DeltaNet, H=16, T=4096, dk=dv=128: every head checked."""
    log("prefill C2 full: GDN H=16 T=4096")
    inp = generate(WORKLOADS["gdn_h16_t4096_d128_bf16"], seed=2, device=DEV)
    o, ST = gpu_prefill(inp)
    check_all(inp, o, ST, 2e-2, "C2")


@pytest.mark.timeout(300)
@pytest.mark.parametrize("method", [SINGLE, TWO])
def test_prefill_kda_b2_h32_t32768_full(method):
    """B=2, H=32, T=32768, log_a clipped at -8: every output and final state of
    the whole batch against the oracle (the two-pass run is the benchmark's
    launch)."""
    log(f"prefill C3 full: KDA B=2 H=32 T=32768 method={method}")
    inp = generate(WORKLOADS["kda_b2_h32_t32768_d128_bf16"], seed=3, device=DEV)
    o, ST = run_method(inp, method)
    check_all(inp, o, ST, 2e-2, "C3 all 64 units")


@pytest.mark.timeout(400)
def test_prefill_varlen_64seq_full():
    """64 packed sequences, lengths U[512, 16384], H=32: all 2048 (sequence, head)
    units against the oracle, run over groups of 8 sequences to bound host memory
    (the oracle works in fp64)."""
    log("prefill C5 full: varlen 64 sequences, all units")
    inp = generate(WORKLOADS["kda_varlen_64seq_h32_d128"], seed=5, device=DEV)
    o, ST = gpu_prefill(inp)
    cu = inp["cu_seqlens"].cpu().numpy().astype(np.int64)
    worst_o = worst_s = 0.0
    G = 8
    for g0 in range(0, 64, G):
        a, b = int(cu[g0]), int(cu[g0 + G])
        part = {key: inp[key][a:b].cpu() for key in ("q", "k", "v", "log_a", "beta")}
        part["S0"] = inp["S0"][g0:g0 + G].cpu()
        part["cu_seqlens"] = torch.tensor(cu[g0:g0 + G + 1] - a, dtype=torch.int32)
        ro, rS = oracle_all(part)
        worst_o = max(worst_o, max_rel_err(o[a:b], ro))
        worst_s = max(worst_s, max_rel_err(ST[g0:g0 + G], rS))
        log(f"  sequences {g0}-{g0 + G - 1}: worst so far o {worst_o:.2e} S {worst_s:.2e}")
    assert worst_o <= 2e-2 and worst_s <= 2e-2
