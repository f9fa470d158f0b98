"""The prefill's gradient on the GPU (kda_chunk_bwd through the C ABI) against the
oracle's fp64 token-by-token gradient, on the same rounded inputs: every output
(dq, dk, dv, dlog_a, dbeta, dS0) element by element, with the bars of the
forward (2e-2 for bf16 inputs, 1e-4 for fp32, max error over max reference)."""
import numpy as np
import pytest
import torch

import kda_recurrent_state_amd as kda
from kda_recurrent_state_amd.workloads import WORKLOADS, generate, scaled
from oracle import kda_oracle_bwd
from tests.parity import TOL, log, max_rel_err, np64

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
NAMES = ("dq", "dk", "dv", "dlog_a", "dbeta", "dS0")


def draw(base, seed, lengths, heads=2, dtype=None, s0_std=0.5, dst=True, **kw):
    w = WORKLOADS[base]
    ch = dict(n_seqs=len(lengths), heads=heads, s0_std=s0_std, **kw)
    if dtype is not None:
        ch["dtype"] = dtype
    w = scaled(w, **ch)
    inp = generate(w, seed, DEV, lengths=lengths)
    g = torch.Generator(device=DEV)
    g.manual_seed(seed + 1000)
    T = int(np.sum(lengths))
    inp["dO"] = torch.randn((T, w.heads, w.dv), generator=g, device=DEV).to(w.dtype)
    inp["dST"] = (torch.randn((len(lengths), w.heads, w.dk, w.dv), generator=g, device=DEV) if dst else None)
    return inp


def gpu_grad(inp, **kw):
    out = kda.chunk_bwd(inp["q"], inp["k"], inp["v"], inp["log_a"], inp["beta"], inp["dO"], S0=inp["S0"],
                        cu_seqlens=inp["cu_seqlens"], dS_T=inp["dST"], **kw)
    torch.cuda.synchronize()
    return out


def oracle_grad(inp):
    c = lambda t: None if t is None else t.detach().cpu()
    return kda_oracle_bwd(c(inp["q"]), c(inp["k"]), c(inp["v"]), c(inp["log_a"]), c(inp["beta"]), S0=c(inp["S0"]),
                          cu_seqlens=inp["cu_seqlens"].cpu().numpy(), dO=c(inp["dO"]), dST=c(inp["dST"]))


def check(inp, got, tol, what, names=NAMES):
    ref = oracle_grad(inp)
    errs = {n: max_rel_err(got[n], ref[n]) for n in names if got.get(n) is not None}
    log(f"  {what}: " + " ".join(f"{n} {e:.2e}" for n, e in errs.items()))
    bad = {n: e for n, e in errs.items() if not e <= tol}
    assert not bad, f"{what}: {bad}"
    return errs


@pytest.mark.parametrize("lengths", [[130, 64, 37], [300], [16, 1, 0, 79]])
def test_bwd_bf16_d128(lengths):
    inp = draw("kda_b2_h32_t32768_d128_bf16", 1, lengths)
    check(inp, gpu_grad(inp), TOL[torch.bfloat16], f"bf16 d128 lengths {lengths}")


@pytest.mark.parametrize("d", [32, 64])
def test_bwd_bf16_smaller_heads(d):
    inp = draw("kda_b2_h32_t32768_d128_bf16", 2, [200, 45], dk=d, dv=d)
    check(inp, gpu_grad(inp), TOL[torch.bfloat16], f"bf16 d{d}")


@pytest.mark.parametrize("d,lengths", [(16, [64]), (16, [100, 3]), (32, [150]), (64, [77, 64])])
def test_bwd_fp32(d, lengths):
    inp = draw("kda_t64_d16_fp32", 3, lengths, dk=d, dv=d)
    check(inp, gpu_grad(inp), TOL[torch.float32], f"fp32 d{d} lengths {lengths}")


def test_bwd_scalar_gate_bf16():
    inp = draw("gdn_h16_t4096_d128_bf16", 4, [190, 70])
    check(inp, gpu_grad(inp), TOL[torch.bfloat16], "bf16 scalar gate")


def test_bwd_scalar_gate_fp32():
    inp = draw("kda_t64_d16_fp32", 5, [90], dk=32, dv=32, scalar_decay=True)
    check(inp, gpu_grad(inp), TOL[torch.float32], "fp32 scalar gate")


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("steep", [-10.5, -25.0])
def test_bwd_steep_decay_takes_exact_terms(dtype, steep):
    # 16-token pieces spanning 168 or 400 nats, beyond the backward's factor split
    # (160 nats), so they take one exponent per term.  The steep stretch lies in the
    # first 64 tokens: their gradients start from S0 and need no state kept by the
    # forward rerun, whose own factor split is accurate for log a >= -8 per token.
    base = "kda_t64_d16_fp32" if dtype == torch.float32 else "kda_b2_h32_t32768_d128_bf16"
    d = 32 if dtype == torch.float32 else 64
    inp = draw(base, 6, [62, 40], dk=d, dv=d)
    la = inp["log_a"].clone()
    la[30:55] = steep
    inp["log_a"] = la
    got = gpu_grad(inp)
    for n in NAMES:
        assert torch.isfinite(got[n].float()).all(), n
    check(inp, got, TOL[dtype], f"steep decay {dtype}")


def test_bwd_without_optional_arguments():
    inp = draw("kda_b2_h32_t32768_d128_bf16", 7, [100, 30], s0_std=0.0, dst=False)
    assert inp["S0"] is None and inp["dST"] is None
    got = gpu_grad(inp, initial_state_grad=False)
    assert got["dS0"] is None
    check(inp, got, TOL[torch.bfloat16], "no S0, no dS_T", names=NAMES[:-1])
    got = gpu_grad(inp)
    check(inp, got, TOL[torch.bfloat16], "dS0 at a zero start")


def test_bwd_two_pass_and_single_pass_reruns_agree():
    inp = draw("kda_b2_h32_t32768_d128_bf16", 8, [200, 64])
    a = gpu_grad(inp, method=kda.METHOD_SINGLE)
    b = gpu_grad(inp, method=kda.METHOD_TWO_PASS)
    for n in NAMES:
        e = max_rel_err(a[n], b[n])
        log(f"  single vs two-pass rerun {n} {e:.2e}")
        assert e <= 2e-2, n


@pytest.mark.parametrize("d", [32, 128])
def test_bwd_deterministic(d):
    # bit-identical results whatever the workspace held before the call
    inp = draw("kda_b2_h32_t32768_d128_bf16", 9, [150, 90], dk=d, dv=d)
    need = kda.chunk_bwd_workspace_size(inp["q"], inp["v"], num_seqs=2, max_seqlen=150)
    g = torch.Generator(device=DEV)
    outs = []
    for fill in range(3):
        g.manual_seed(fill)
        ws = torch.randint(0, 256, (need,), dtype=torch.uint8, device=DEV, generator=g)
        outs.append(gpu_grad(inp, workspace=ws))
    for o in outs[1:]:
        for n in NAMES:
            assert torch.equal(outs[0][n], o[n]), n


def test_bwd_matches_finite_difference_of_gpu_forward():
    # the gradient along a random direction of log_a equals the change of the GPU
    # forward's loss (fp32, small steps, central difference)
    inp = draw("kda_t64_d16_fp32", 10, [96], dk=32, dv=32)
    got = gpu_grad(inp)
    u = torch.randn_like(inp["log_a"]) * 0.1

    def loss(la):
        o, ST = kda.chunk_fwd(inp["q"], inp["k"], inp["v"], la, inp["beta"], S0=inp["S0"],
                              cu_seqlens=inp["cu_seqlens"])
        return float((np64(o) * np64(inp["dO"])).sum() + (np64(ST) * np64(inp["dST"])).sum())

    h = 1e-2
    fd = (loss(inp["log_a"] + h * u) - loss(inp["log_a"] - h * u)) / (2 * h)
    an = float((np64(got["dlog_a"]) * np64(u)).sum())
    log(f"  directional: analytic {an:.6g} central difference {fd:.6g}")
    assert abs(an - fd) <= 2e-3 * max(1.0, abs(fd))


def test_bwd_full_size_sampled():
    # the bench batch (2 x 32 heads x 32768 tokens, dk = dv = 128, bf16) through the
    # gradient call the bench times; the oracle walks one whole (sequence, head)
    from kda_recurrent_state_amd.workloads import WORKLOADS, generate
    w = WORKLOADS["kda_b2_h32_t32768_d128_bf16"]
    inp = generate(w, 3, DEV)
    g = torch.Generator(device=DEV)
    g.manual_seed(5)
    T = inp["q"].shape[0]
    dO = torch.randn((T, w.heads, w.dv), generator=g, device=DEV).to(w.dtype)
    dST = torch.randn((w.n_seqs, w.heads, w.dk, w.dv), generator=g, device=DEV)
    got = kda.chunk_bwd(inp["q"], inp["k"], inp["v"], inp["log_a"], inp["beta"], dO, S0=inp["S0"],
                        cu_seqlens=inp["cu_seqlens"], dS_T=dST, max_seqlen=w.seqlen)
    torch.cuda.synchronize()
    n, h = 1, 21
    s, e = n * w.seqlen, (n + 1) * w.seqlen
    c = lambda t: t[s:e, h:h + 1].cpu()
    log(f"  oracle gradient of sequence {n}, head {h} ({w.seqlen} tokens)")
    ref = kda_oracle_bwd(c(inp["q"]), c(inp["k"]), c(inp["v"]), c(inp["log_a"]), c(inp["beta"]),
                         S0=inp["S0"][n:n + 1, h:h + 1].cpu(), dO=c(dO), dST=dST[n:n + 1, h:h + 1].cpu())
    errs = {}
    for name in ("dq", "dk", "dv", "dlog_a", "dbeta"):
        errs[name] = max_rel_err(got[name][s:e, h:h + 1], ref[name])
    errs["dS0"] = max_rel_err(got["dS0"][n:n + 1, h:h + 1], ref["dS0"])
    log("  full size: " + " ".join(f"{k} {v:.2e}" for k, v in errs.items()))
    assert all(v <= TOL[torch.bfloat16] for v in errs.values()), errs
