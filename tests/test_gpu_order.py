"""The decay-first ordering, S <- (I - b k^T k) Diag(a) S + b k^T v, on the GPU
(prefill, both methods, snapshots, and decode) against the fp64 oracle run with
the same ordering; with a scalar decay both orderings are one map."""
import numpy as np
import pytest
import torch

import kda_recurrent_state_amd as kda
from kda_recurrent_state_amd.workloads import WORKLOADS, generate, scaled
from tests.parity import TOL, decode_as_sequence, log, max_rel_err, np64, oracle_all, oracle_unit

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
SINGLE, TWO = kda.METHOD_SINGLE, kda.METHOD_TWO_PASS
D1 = kda.ORDER_DECAY_FIRST


def host(inp):
    return {k: (v.cpu() if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}


def prefill(inp, unsupported=False, **kw):
    """Prefill; for a shape documented as not compiled (the two-pass method is bf16
    with dk 64 or 128 only) the call must refuse with KDA_ERR_UNSUPPORTED (None)."""
    call = lambda: kda.chunk_fwd(inp["q"], inp["k"], inp["v"], inp["log_a"], inp["beta"], S0=inp["S0"],
                                 cu_seqlens=inp["cu_seqlens"], **kw)
    if unsupported:
        with pytest.raises(kda.KdaError) as e:
            call()
        assert e.value.status == 2, e.value
        log(f"  refused as documented: {e.value}")
        return None
    o, ST = call()
    torch.cuda.synchronize()
    return o, ST


def check(inp, o, ST, tol, what=""):
    ro, rS = oracle_all(host(inp), order=1)
    eo, es = max_rel_err(o, ro), max_rel_err(ST, rS)
    log(f"  {what} err o {eo:.2e} S {es:.2e}")
    assert eo <= tol and es <= tol


@pytest.mark.parametrize("method", [SINGLE, TWO])
@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 64), (128, 32), (64, 128), (32, 32)])
def test_decay_first_prefill_bf16(dk, dv, method):
    log(f"decay-first prefill bf16 dk={dk} dv={dv} method={method}")
    w = scaled(WORKLOADS["kda_varlen_64seq_h32_d128"], n_seqs=4, heads=3, dk=dk, dv=dv)
    inp = generate(w, seed=70 + dk + dv, device=DEV, lengths=[45, 0, 170, 96])
    res = prefill(inp, unsupported=(method == TWO and dk not in (64, 128)), method=method, order=D1)
    if res is not None:
        check(inp, *res, 2e-2, f"method {method}")


@pytest.mark.parametrize("dk,dv", [(16, 16), (32, 32), (64, 32), (128, 64)])
def test_decay_first_prefill_fp32(dk, dv):
    log(f"decay-first prefill fp32 dk={dk} dv={dv}")
    w = scaled(WORKLOADS["kda_varlen_64seq_h32_d128"], n_seqs=4, heads=2, dk=dk, dv=dv, dtype=torch.float32)
    inp = generate(w, seed=80 + dk + dv, device=DEV, lengths=[37, 0, 96, 5])
    o, ST = prefill(inp, order=D1)
    check(inp, o, ST, 1e-4, "fp32")


def test_orders_differ_with_channel_decay_and_agree_with_scalar_decay():
    log("decay-first vs erase-first")
    w = scaled(WORKLOADS["kda_varlen_64seq_h32_d128"], n_seqs=2, heads=2, dk=64, dv=64)
    inp = generate(w, seed=90, device=DEV, lengths=[100, 64])
    o0, S0 = prefill(inp)
    o1, S1 = prefill(inp, order=D1)
    # the per-channel decay tells them apart by more than the bf16 parity bar, so
    # a kernel running the other order fails the parity tests above
    assert max_rel_err(o1, o0) > 2e-2
    ws = scaled(w, scalar_decay=True)
    inp = generate(ws, seed=91, device=DEV, lengths=[100, 64])
    for method in (SINGLE, TWO):
        o0, S0 = prefill(inp, method=method)
        o1, S1 = prefill(inp, method=method, order=D1)
        assert torch.equal(o0, o1) and torch.equal(S0, S1)
    check(inp, o1, S1, 2e-2, "scalar decay")


def test_decay_first_two_pass_segments_and_snapshots():
    """Decay-first blocks are smaller; the smallest workspace (a segment per
    chunk) gives the preferred workspace's results exactly, and snapshots match
    the oracle."""
    log("decay-first segments and snapshots")
    w = scaled(WORKLOADS["kda_b2_h32_t32768_d128_bf16"], n_seqs=2, seqlen=320, heads=2)
    inp = generate(w, seed=92, device=DEV)
    q, v = inp["q"], inp["v"]
    least = kda.chunk_workspace_size(q, v, num_seqs=2, method=TWO, max_seqlen=320, minimum=True, order=D1)
    least0 = kda.chunk_workspace_size(q, v, num_seqs=2, method=TWO, max_seqlen=320, minimum=True)
    assert least < least0
    ws = torch.empty(least, dtype=torch.uint8, device=DEV)
    o_a, S_a = prefill(inp, method=TWO, order=D1, workspace=ws, max_seqlen=320)
    o_b, S_b = prefill(inp, method=TWO, order=D1)
    assert torch.equal(o_a, o_b) and torch.equal(S_a, S_b)
    check(inp, o_b, S_b, 2e-2, "segments")
    _, _, snaps = kda.chunk_fwd_snapshots(inp["q"], inp["k"], inp["v"], inp["log_a"], inp["beta"], S0=inp["S0"],
                                          cu_seqlens=inp["cu_seqlens"], snapshot_every=128, method=TWO, order=D1)
    torch.cuda.synchronize()
    assert snaps.shape[0] == 4
    hi = host(inp)
    for n in range(2):
        for s in range(2):
            t = (s + 1) * 128
            sub = dict(hi)
            for key in ("q", "k", "v", "log_a", "beta"):
                sub[key] = hi[key][320 * n:320 * n + t]
            sub["S0"] = hi["S0"][n:n + 1]
            sub["cu_seqlens"] = torch.tensor([0, t], dtype=torch.int32)
            _, rS = oracle_all(sub, order=1)
            e = max_rel_err(snaps[2 * n + s], rS[0])
            assert e <= 2e-2, (n, s, e)


@pytest.mark.parametrize("method", [SINGLE, TWO])
def test_decay_first_kda_b2_h32_t32768_sampled(method):
    """B=2, H=32, T=32768, dk = dv = 128: 3 units checked against the oracle."""
    log(f"decay-first full size method={method}")
    inp = generate(WORKLOADS["kda_b2_h32_t32768_d128_bf16"], seed=3, device=DEV)
    o, ST = prefill(inp, method=method, order=D1)
    hi = host(inp)
    cu = hi["cu_seqlens"].numpy()
    worst = 0.0
    for n, h in [(0, 2), (1, 17), (1, 31)]:
        ro, rS = oracle_unit(hi, n, h, order=1)
        worst = max(worst, max_rel_err(o[cu[n]:cu[n + 1], h], ro), max_rel_err(ST[n, h], rS))
    log(f"  sampled err {worst:.2e}")
    assert worst <= 2e-2


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("dk,dv", [(16, 16), (32, 64), (128, 128), (64, 32)])
def test_decay_first_decode_chain(dtype, dk, dv):
    log(f"decay-first decode dtype={dtype} dk={dk} dv={dv}")
    w = scaled(WORKLOADS["kda_decode_b256_h32_d128"], n_seqs=3, heads=2, dk=dk, dv=dv, steps=12, dtype=dtype)
    inp = generate(w, seed=100 + dk + dv, device=DEV)
    S = inp["S"].clone()
    outs = []
    for t in range(inp["q"].shape[0]):
        o, S = kda.decode_step(inp["q"][t], inp["k"][t], inp["v"][t], inp["log_a"][t], inp["beta"][t], S,
                               order=D1)
        outs.append(o)
    torch.cuda.synchronize()
    o = torch.stack(outs)
    seq, steps, N = decode_as_sequence({k: v.cpu() for k, v in inp.items()})
    ro, rS = oracle_all(seq, order=1)
    go = np64(o).transpose(1, 0, 2, 3).reshape(ro.shape)
    eo, es = max_rel_err(go, ro), max_rel_err(S, rS)
    log(f"  err o {eo:.2e} S {es:.2e}")
    assert eo <= TOL[dtype] and es <= TOL[dtype]


def test_decay_first_prefill_then_decode():
    """A prefill's final state continues under decode steps with the same
    ordering: prefill of T tokens + 4 decode steps equals the oracle over T + 4."""
    log("decay-first prefill + decode continuation")
    w = scaled(WORKLOADS["kda_b2_h32_t32768_d128_bf16"], n_seqs=1, seqlen=100, heads=2)
    inp = generate(w, seed=101, device=DEV)
    T = 96
    pre = {k: (v[:T].contiguous() if k in ("q", "k", "v", "log_a", "beta") else v) for k, v in inp.items()}
    pre["cu_seqlens"] = torch.tensor([0, T], dtype=torch.int32, device=DEV)
    o, S = prefill(pre, order=D1)
    outs = [o]
    for t in range(T, 100):
        sl = lambda x: x[t:t + 1].contiguous()
        ot, S = kda.decode_step(sl(inp["q"]), sl(inp["k"]), sl(inp["v"]), sl(inp["log_a"]), sl(inp["beta"]), S,
                                order=D1)
        outs.append(ot)
    torch.cuda.synchronize()
    ro, rS = oracle_all(host(inp), order=1)
    eo, es = max_rel_err(torch.cat(outs), ro), max_rel_err(S, rS)
    log(f"  err o {eo:.2e} S {es:.2e}")
    assert eo <= 2e-2 and es <= 2e-2
