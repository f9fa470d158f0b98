"""Chunk-boundary state snapshots of the prefill (kda_chunk_fwd_snapshots):
the state after every L tokens of each sequence, against the fp64 oracle run
up to those points, and bit-identical to S_T of the prefix alone."""
import numpy as np
import pytest
import torch

import kda_recurrent_state_amd as kda
from kda_recurrent_state_amd.workloads import WORKLOADS, generate, scaled
from tests.parity import log, max_rel_err, oracle_snapshots

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
SINGLE, TWO = kda.METHOD_SINGLE, kda.METHOD_TWO_PASS


def snap_call(inp, every, **kw):
    try:
        r = kda.chunk_fwd_snapshots(inp["q"], inp["k"], inp["v"], inp["log_a"], inp["beta"], S0=inp["S0"],
                                    cu_seqlens=inp["cu_seqlens"], snapshot_every=every, **kw)
    except kda.KdaError as e:
        if e.status == 2:
            raise AssertionError(f"snapshots refused for a shape that is compiled: {e}")
        raise
    torch.cuda.synchronize()
    return r


def rows_of(inp, every):
    """First snapshot row of each sequence, and the total (from the lengths)."""
    lens = np.diff(inp["cu_seqlens"].cpu().numpy().astype(np.int64))
    per = lens // every
    return np.concatenate([[0], np.cumsum(per)]), int(per.sum())


def check_snapshots(inp, snaps, every, tol, what=""):
    first, total = rows_of(inp, every)
    assert snaps.shape[0] == total
    worst = 0.0
    host = {k: (v.cpu() if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    for n in range(len(first) - 1):
        ref = oracle_snapshots(host, every, n)
        got = snaps[first[n]:first[n + 1]]
        assert got.shape[0] == ref.shape[0]
        if ref.shape[0]:
            worst = max(worst, max_rel_err(got, ref))
    log(f"  {what} snapshots {total} rows, err {worst:.2e}")
    assert worst <= tol
    return worst


@pytest.mark.parametrize("method", [SINGLE, TWO])
@pytest.mark.parametrize("dk,dv,scalar", [(128, 128, False), (64, 64, True), (128, 32, False), (64, 128, False)])
def test_snapshots_bf16_varlen(dk, dv, scalar, method):
    """Ragged sequences (shorter than L, exact multiples, one chunk past, empty)."""
    log(f"snapshots bf16 dk={dk} dv={dv} scalar={scalar} method={method}")
    w = scaled(WORKLOADS["kda_varlen_64seq_h32_d128"], n_seqs=5, heads=2, dk=dk, dv=dv, scalar_decay=scalar)
    inp = generate(w, seed=40 + dk + dv + scalar, device=DEV, lengths=[300, 7, 128, 0, 161])
    o, ST, snaps = snap_call(inp, 64, method=method)
    check_snapshots(inp, snaps, 64, 2e-2, f"method {method}")
    # the prefill's own outputs are those of the plain call
    o2, S2 = kda.chunk_fwd(inp["q"], inp["k"], inp["v"], inp["log_a"], inp["beta"], S0=inp["S0"],
                           cu_seqlens=inp["cu_seqlens"], method=method)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(ST, S2)
    # the last row of a sequence whose length L divides is its S_T
    first, _ = rows_of(inp, 64)
    assert torch.equal(snaps[first[3] - 1], ST[2])


def test_snapshots_longest_first():
    """300 sequences (more state-pass workgroups than compute units, so the
    walk takes them longest first): each sequence's rows still land at its own
    place in the packed snapshot buffer."""
    log("snapshots, 300 sequences longest first")
    rng = np.random.default_rng(7)
    lengths = rng.integers(0, 200, 300)
    lengths[rng.integers(0, 300, 30)] = 64
    lengths[11] = 0
    w = scaled(WORKLOADS["kda_varlen_64seq_h32_d128"], n_seqs=300, heads=1)
    inp = generate(w, seed=71, device=DEV, lengths=lengths.tolist())
    o, ST, snaps = snap_call(inp, 64, method=TWO)
    check_snapshots(inp, snaps, 64, 2e-2, "300 sequences")


@pytest.mark.parametrize("dk,dv", [(32, 32), (64, 32), (128, 32)])
def test_snapshots_fp32(dk, dv):
    log(f"snapshots fp32 dk={dk} dv={dv}")
    w = scaled(WORKLOADS["kda_varlen_64seq_h32_d128"], n_seqs=3, heads=2, dk=dk, dv=dv, dtype=torch.float32)
    inp = generate(w, seed=50 + dk, device=DEV, lengths=[200, 64, 31])
    _, _, snaps = snap_call(inp, 32)
    check_snapshots(inp, snaps, 32, 1e-4, "fp32")


@pytest.mark.parametrize("method", [SINGLE, TWO])
def test_snapshot_equals_prefix_state(method):
    """Row s is bit-identical to S_T of a call on the first (s + 1) L tokens
    alone (same method, chunk size and dv split)."""
    log(f"snapshots vs prefix S_T method={method}")
    w = scaled(WORKLOADS["kda_b2_h32_t32768_d128_bf16"], n_seqs=1, seqlen=416, heads=3)
    inp = generate(w, seed=60, device=DEV)
    every = 96
    _, _, snaps = snap_call(inp, every, method=method, dv_split=4)
    assert snaps.shape[0] == 416 // every
    for s in range(snaps.shape[0]):
        t = (s + 1) * every
        cu = torch.tensor([0, t], dtype=torch.int32, device=DEV)
        sl = lambda x: x[:t].contiguous()
        _, ST = kda.chunk_fwd(sl(inp["q"]), sl(inp["k"]), sl(inp["v"]), sl(inp["log_a"]), sl(inp["beta"]),
                              S0=inp["S0"], cu_seqlens=cu, method=method, dv_split=4)
        torch.cuda.synchronize()
        assert torch.equal(snaps[s], ST[0]), f"row {s}"


def test_snapshots_across_segments_and_equal_lengths():
    """Two-pass with the smallest workspace (a segment per chunk) gives the same
    rows as the preferred one; equal lengths without cu_seqlens give the same
    rows as cu_seqlens."""
    log("snapshots across workspace segments")
    w = scaled(WORKLOADS["kda_b2_h32_t32768_d128_bf16"], n_seqs=2, seqlen=320, heads=2)
    inp = generate(w, seed=61, device=DEV)
    q, v = inp["q"], inp["v"]
    least = kda.chunk_workspace_size(q, v, num_seqs=2, method=TWO, max_seqlen=320, minimum=True)
    ws = torch.empty(least, dtype=torch.uint8, device=DEV)
    _, _, a = snap_call(inp, 64, method=TWO, workspace=ws, max_seqlen=320)
    _, _, b = snap_call(inp, 64, method=TWO)
    assert torch.equal(a, b)
    check_snapshots(inp, a, 64, 2e-2, "segments")
    _, _, c = kda.chunk_fwd_snapshots(inp["q"], inp["k"], inp["v"], inp["log_a"], inp["beta"], S0=inp["S0"],
                                      num_seqs=2, snapshot_every=64, method=TWO)
    torch.cuda.synchronize()
    assert torch.equal(c, b)


@pytest.mark.parametrize("method", [SINGLE, TWO])
def test_snapshot_rows_limit(method):
    """A buffer of fewer rows than the lengths give: the rows it holds are
    written, nothing past them."""
    log(f"snapshot rows limit method={method}")
    w = scaled(WORKLOADS["kda_varlen_64seq_h32_d128"], n_seqs=3, heads=2, dk=64, dv=64)
    inp = generate(w, seed=62, device=DEV, lengths=[256, 100, 200])
    _, _, full = snap_call(inp, 32, method=method)
    R = full.shape[0]
    assert R == 8 + 3 + 6
    buf = torch.full((R + 4,) + tuple(full.shape[1:]), float("nan"), device=DEV)
    part = buf[:10]
    snap_call(inp, 32, method=method, snapshots=part)
    assert torch.equal(buf[:10], full[:10])
    assert torch.isnan(buf[10:]).all()


@pytest.mark.parametrize("method", [SINGLE, TWO])
def test_snapshots_kda_b2_h32_t32768_sampled(method):
    """B=2, H=32, T=32768 with a snapshot every 8192 tokens: rows of 3 heads
    checked against the oracle."""
    log(f"snapshots full size method={method}")
    inp = generate(WORKLOADS["kda_b2_h32_t32768_d128_bf16"], seed=3, device=DEV)
    every = 8192
    o, ST, snaps = snap_call(inp, every, method=method)
    assert snaps.shape[0] == 2 * 4
    host = {k: (v.cpu() if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    worst = 0.0
    for n, h in [(0, 5), (1, 30)]:
        ref = oracle_snapshots(host, every, n, h)
        worst = max(worst, max_rel_err(snaps[4 * n:4 * n + 4, h], ref))
    log(f"  sampled snapshot err {worst:.2e}")
    assert worst <= 2e-2
