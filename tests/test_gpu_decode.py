"""Decode step on the GPU against the fp64 oracle (chained steps)."""
import numpy as np
import pytest
import torch

import kda_recurrent_state_amd as kda
from kda_recurrent_state_amd.workloads import WORKLOADS, generate, scaled
from tests.parity import TOL, decode_as_sequence, log, max_rel_err, np64, oracle_all

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def run_chain(inp, in_place=True):
    S = inp["S"].clone()
    outs = []
    for t in range(inp["q"].shape[0]):
        if in_place:
            o, S = kda.decode_step(inp["q"][t], inp["k"][t], inp["v"][t], inp["log_a"][t], inp["beta"][t], S)
        else:
            S2 = torch.empty_like(S)
            o, S = kda.decode_step(inp["q"][t], inp["k"][t], inp["v"][t], inp["log_a"][t], inp["beta"][t], S,
                                   S_out=S2)
        outs.append(o)
    torch.cuda.synchronize()
    return torch.stack(outs), S


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("dk,dv", [(16, 16), (32, 64), (128, 128), (64, 32), (128, 16)])
@pytest.mark.parametrize("scalar", [False, True])
def test_decode_chain_small(dtype, dk, dv, scalar):
    log(f"decode chain dtype={dtype} dk={dk} dv={dv} scalar={scalar}")
    w = scaled(WORKLOADS["kda_decode_b256_h32_d128"], n_seqs=3, heads=2, dk=dk, dv=dv, steps=12,
               dtype=dtype, scalar_decay=scalar)
    inp = generate(w, seed=dk + dv + scalar, device=DEV)
    o, S = run_chain(inp, in_place=not scalar)
    seq, steps, N = decode_as_sequence({k: v.cpu() for k, v in inp.items()})
    ro, rS = oracle_all(seq)
    # oracle o is [N*steps, H, dv] sequence-major; GPU o is [steps, N, H, dv]
    go = np64(o).transpose(1, 0, 2, 3).reshape(ro.shape)
    eo, es = max_rel_err(go, ro), max_rel_err(S, rS)
    log(f"  err o {eo:.2e} S {es:.2e}")
    assert eo <= TOL[dtype] and es <= TOL[dtype]


@pytest.mark.timeout(300)
def test_decode_full_size():
    """256 sequences x 32 heads, dk = dv = 128, 100 chained steps: every one of
    the 8192 states and every output of every step against the oracle."""
    log("decode full size: 256 x 32 heads, 100 steps, all states")
    w = WORKLOADS["kda_decode_b256_h32_d128"]
    inp = generate(w, seed=4, device=DEV)
    o, S = run_chain(inp)
    seq, steps, N = decode_as_sequence({k: v.cpu() for k, v in inp.items()})
    del inp
    ro, rS = oracle_all(seq)
    go = np64(o).transpose(1, 0, 2, 3).reshape(ro.shape)
    eo, es = max_rel_err(go, ro), max_rel_err(S, rS)
    log(f"  err o {eo:.2e} S {es:.2e} over {N * w.heads} states")
    assert eo <= 2e-2 and es <= 2e-2
