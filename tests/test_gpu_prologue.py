"""Input prologue on the GPU (kda_chunk_fwd_ex / kda_decode_step_ex): raw
keys, beta logits and log-decay pre-activations, transformed as the kernels load
them, against the fp64 oracle running the same prologue."""
import numpy as np
import pytest
import torch

import kda_recurrent_state_amd as kda
from kda_recurrent_state_amd.workloads import WORKLOADS, generate_raw, scaled
from tests.parity import TOL, decode_as_sequence, log, max_rel_err, np64, oracle_all, oracle_unit

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TWO = kda.METHOD_TWO_PASS
PRO = dict(normalize_k=True, beta_logits=True, log_a_raw=True, log_a_min=-8.0)


def host(inp):
    return {k: (v.cpu() if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}


def prefill(inp, pro=PRO, **kw):
    o, ST = kda.chunk_fwd(inp["q"], inp["k"], inp["v"], inp["log_a"], inp["beta"], S0=inp["S0"],
                          cu_seqlens=inp["cu_seqlens"], prologue=pro, **kw)
    torch.cuda.synchronize()
    return o, ST


def oracle_pro(inp, pro=PRO, order=0):
    from oracle import kda_oracle
    h = host(inp)
    return kda_oracle(h["q"], h["k"], h["v"], h["log_a"], h["beta"], S0=h.get("S0"),
                      cu_seqlens=h["cu_seqlens"].numpy(), order=order, pro=pro)


@pytest.mark.parametrize("order", [0, 1])
@pytest.mark.parametrize("dk,dv,scalar", [(128, 128, False), (64, 64, False), (128, 32, True), (64, 128, True)])
def test_prologue_prefill(dk, dv, scalar, order):
    log(f"prologue prefill dk={dk} dv={dv} scalar={scalar} order={order}")
    w = scaled(WORKLOADS["kda_varlen_64seq_h32_d128"], n_seqs=4, heads=3, dk=dk, dv=dv, scalar_decay=scalar)
    inp = generate_raw(w, seed=110 + dk + dv + scalar, device=DEV, lengths=[45, 0, 170, 96])
    o, ST = prefill(inp, order=order)
    ro, rS = oracle_pro(inp, order=order)
    eo, es = max_rel_err(o, ro), max_rel_err(ST, rS)
    log(f"  err o {eo:.2e} S {es:.2e}")
    assert eo <= 2e-2 and es <= 2e-2


@pytest.mark.parametrize("pro", [dict(normalize_k=True), dict(beta_logits=True), dict(log_a_raw=True),
                                 dict(log_a_raw=True, log_a_min=-3.0)])
def test_prologue_each_transform_alone(pro):
    """Each transform on its own, the other inputs already in their final form."""
    log(f"prologue alone {pro}")
    w = scaled(WORKLOADS["kda_varlen_64seq_h32_d128"], n_seqs=2, heads=2)
    raw = generate_raw(w, seed=120, device=DEV, lengths=[130, 77])
    from kda_recurrent_state_amd.workloads import generate
    fin = generate(w, seed=120, device=DEV, lengths=[130, 77])
    inp = dict(fin)
    if pro.get("normalize_k"):
        inp["k"] = raw["k"]
    if pro.get("beta_logits"):
        inp["beta"] = raw["beta"]
    if pro.get("log_a_raw"):
        inp["log_a"] = raw["log_a"]
    o, ST = prefill(inp, pro=pro)
    ro, rS = oracle_pro(inp, pro=pro)
    assert max_rel_err(o, ro) <= 2e-2 and max_rel_err(ST, rS) <= 2e-2


def test_prologue_matches_transformed_inputs():
    """The prologue in the kernels agrees with transforming the inputs first (in
    fp32 by torch) and calling without it, to the bf16 bar."""
    log("prologue vs pre-transformed inputs")
    w = scaled(WORKLOADS["kda_b2_h32_t32768_d128_bf16"], n_seqs=2, seqlen=300, heads=2)
    inp = generate_raw(w, seed=121, device=DEV)
    o1, S1 = prefill(inp)
    k = inp["k"].float()
    t = dict(inp)
    t["k"] = (k * torch.rsqrt((k * k).sum(-1, keepdim=True) + 1e-6)).to(torch.bfloat16)
    t["beta"] = torch.sigmoid(inp["beta"])
    t["log_a"] = (-torch.nn.functional.softplus(inp["log_a"])).clamp(min=-8.0)
    o2, S2 = prefill(t, pro=None)
    assert max_rel_err(o1, o2) <= 2e-2 and max_rel_err(S1, S2) <= 2e-2


def test_prologue_snapshots_and_segments():
    log("prologue with snapshots and the smallest workspace")
    w = scaled(WORKLOADS["kda_b2_h32_t32768_d128_bf16"], n_seqs=2, seqlen=256, heads=2, dk=64, dv=64)
    inp = generate_raw(w, seed=122, device=DEV)
    least = kda.chunk_workspace_size(inp["q"], inp["v"], num_seqs=2, method=TWO, max_seqlen=256, minimum=True)
    ws = torch.empty(least, dtype=torch.uint8, device=DEV)
    o, ST, snaps = kda.chunk_fwd_snapshots(inp["q"], inp["k"], inp["v"], inp["log_a"], inp["beta"], S0=inp["S0"],
                                           cu_seqlens=inp["cu_seqlens"], snapshot_every=128, prologue=PRO,
                                           workspace=ws, max_seqlen=256, method=TWO)
    torch.cuda.synchronize()
    ro, rS = oracle_pro(inp)
    assert max_rel_err(o, ro) <= 2e-2 and max_rel_err(ST, rS) <= 2e-2
    assert torch.equal(snaps[1], ST[0]) and torch.equal(snaps[3], ST[1])  # L divides both lengths


SINGLE_CASES = [
    # dtype, dk, dv, scalar, order, chunk
    (torch.float32, 32, 32, False, 0, 32), (torch.float32, 16, 16, False, 1, 32), (torch.float32, 64, 32, False, 0, 32),
    (torch.float32, 32, 16, True, 0, 32), (torch.float32, 16, 16, False, 0, 64), (torch.float32, 128, 128, False, 0, 32),
    (torch.bfloat16, 32, 32, False, 0, 32), (torch.bfloat16, 128, 64, False, 0, 32),
    (torch.bfloat16, 64, 64, True, 1, 32), (torch.bfloat16, 128, 128, False, 1, 32),
]


@pytest.mark.parametrize("dtype,dk,dv,scalar,order,chunk", SINGLE_CASES)
def test_prologue_single_pass(dtype, dk, dv, scalar, order, chunk):
    """The single-pass kernel (fp32 inputs, bf16 shapes without a two-pass kernel,
    or method SINGLE) with the whole prologue, against the oracle: the key norm
    reduced over the lanes of a row (and the two wavefronts of a row at dk = 128)."""
    log(f"prologue single-pass {dtype} dk={dk} dv={dv} scalar={scalar} order={order} chunk={chunk}")
    w = scaled(WORKLOADS["kda_varlen_64seq_h32_d128"], n_seqs=3, heads=2, dk=dk, dv=dv, dtype=dtype,
               scalar_decay=scalar)
    inp = generate_raw(w, seed=123 + dk + dv + order, device=DEV, lengths=[150, 7, 96])
    o, ST = prefill(inp, order=order, method=kda.METHOD_SINGLE, chunk_size=chunk)
    ro, rS = oracle_pro(inp, order=order)
    eo, es = max_rel_err(o, ro), max_rel_err(ST, rS)
    log(f"  err o {eo:.2e} S {es:.2e}")
    assert eo <= TOL[dtype] and es <= TOL[dtype]


@pytest.mark.parametrize("dtype,dk", [(torch.float32, 32), (torch.bfloat16, 128)])
def test_prologue_single_pass_steep_and_snapshots(dtype, dk):
    """Pre-activations up to a few hundred (log a down to about -300: the steep
    path reloads and transforms them) with snapshots, single-pass."""
    log(f"prologue single-pass steep + snapshots {dtype} dk={dk}")
    w = scaled(WORKLOADS["kda_varlen_64seq_h32_d128"], n_seqs=2, heads=2, dk=dk, dv=dk, dtype=dtype)
    inp = generate_raw(w, seed=129 + dk, device=DEV, lengths=[140, 64])
    x = inp["log_a"].clone()
    x[30:90] = x[30:90].abs() * 60.0 + 20.0
    inp["log_a"] = x.contiguous()
    pro = dict(PRO, log_a_min=None)
    o, ST, snaps = kda.chunk_fwd_snapshots(inp["q"], inp["k"], inp["v"], inp["log_a"], inp["beta"], S0=inp["S0"],
                                           cu_seqlens=inp["cu_seqlens"], snapshot_every=32, prologue=pro,
                                           method=kda.METHOD_SINGLE)
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all() and torch.isfinite(ST).all()
    ro, rS = oracle_pro(inp, pro=pro)
    eo, es = max_rel_err(o, ro), max_rel_err(ST, rS)
    log(f"  err o {eo:.2e} S {es:.2e}")
    assert eo <= TOL[dtype] and es <= TOL[dtype]
    assert torch.equal(snaps[-1], ST[1])  # 64 tokens: its last snapshot is its final state


def test_prologue_kda_b2_h32_t32768_sampled():
    """The bench batch from raw inputs: 2 units against the oracle."""
    log("prologue full size")
    inp = generate_raw(WORKLOADS["kda_b2_h32_t32768_d128_bf16"], seed=3, device=DEV)
    o, ST = prefill(inp)
    h = host(inp)
    from oracle import kda_oracle
    cu = h["cu_seqlens"].numpy()
    worst = 0.0
    for n, hh in [(0, 9), (1, 22)]:
        s, e = int(cu[n]), int(cu[n + 1])
        sl = lambda t: t[s:e, hh:hh + 1]
        ro, rS = kda_oracle(sl(h["q"]), sl(h["k"]), sl(h["v"]), sl(h["log_a"]), sl(h["beta"]),
                            S0=h["S0"][n:n + 1, hh:hh + 1], pro=PRO)
        worst = max(worst, max_rel_err(o[s:e, hh], ro[:, 0]), max_rel_err(ST[n, hh], rS[0, 0]))
    log(f"  sampled err {worst:.2e}")
    assert worst <= 2e-2


@pytest.mark.parametrize("order", [0, 1])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("dk,dv,scalar", [(128, 128, False), (32, 64, True), (64, 16, False)])
def test_prologue_decode_chain(dk, dv, scalar, dtype, order):
    log(f"prologue decode dk={dk} dv={dv} scalar={scalar} dtype={dtype} order={order}")
    w = scaled(WORKLOADS["kda_decode_b256_h32_d128"], n_seqs=3, heads=2, dk=dk, dv=dv, steps=10, dtype=dtype,
               scalar_decay=scalar)
    inp = generate_raw(w, seed=130 + dk + dv, device=DEV)
    S = inp["S"].clone()
    outs = []
    for t in range(inp["q"].shape[0]):
        o, S = kda.decode_step(inp["q"][t], inp["k"][t], inp["v"][t], inp["log_a"][t], inp["beta"][t], S,
                               order=order, prologue=PRO)
        outs.append(o)
    torch.cuda.synchronize()
    seq, steps, N = decode_as_sequence({k: v.cpu() for k, v in inp.items()})
    from oracle import kda_oracle
    ro, rS = kda_oracle(seq["q"], seq["k"], seq["v"], seq["log_a"], seq["beta"], S0=seq["S0"],
                        cu_seqlens=seq["cu_seqlens"].numpy(), order=order, pro=PRO)
    go = np64(torch.stack(outs)).transpose(1, 0, 2, 3).reshape(ro.shape)
    eo, es = max_rel_err(go, ro), max_rel_err(S, rS)
    log(f"  err o {eo:.2e} S {es:.2e}")
    assert eo <= TOL[dtype] and es <= TOL[dtype]
