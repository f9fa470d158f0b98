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


def oracle_grad(inp, order=0):
    c = lambda t: None if t is None else t.detach().cpu()
    return kda_oracle_bwd(c(inp["q"]), c(inp["k"]), c(inp["v"]), c(inp["log_a"]), c(inp["beta"]), S0=c(inp["S0"]),
                          cu_seqlens=inp["cu_seqlens"].cpu().numpy(), dO=c(inp["dO"]), dST=c(inp["dST"]),
                          order=order)


def check(inp, got, tol, what, names=NAMES, order=0):
    ref = oracle_grad(inp, order)
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


@pytest.mark.parametrize("dtype,dk,dv", [(torch.bfloat16, 128, 64), (torch.bfloat16, 64, 128),
                                         (torch.bfloat16, 64, 32), (torch.bfloat16, 32, 64),
                                         (torch.float32, 64, 32), (torch.float32, 32, 64),
                                         (torch.float32, 32, 16), (torch.float32, 16, 32)])
def test_bwd_dk_ne_dv(dtype, dk, dv):
    log(f"backward dk={dk} dv={dv} {dtype}")
    inp = draw("kda_b2_h32_t32768_d128_bf16", 60 + dk + dv, [150, 64, 21], dtype=dtype, dk=dk, dv=dv)
    check(inp, gpu_grad(inp), TOL[dtype], f"dk {dk} dv {dv}")


def test_bwd_scalar_gate_bf16():
    inp = draw("gdn_h16_t4096_d128_bf16", 4, [190, 70])
    check(inp, gpu_grad(inp), TOL[torch.bfloat16], "bf16 scalar gate")


def test_bwd_scalar_gate_fp32():
    inp = draw("kda_t64_d16_fp32", 5, [90], dk=32, dv=32, scalar_decay=True)
    check(inp, gpu_grad(inp), TOL[torch.float32], "fp32 scalar gate")


@pytest.mark.parametrize("dtype,steep", [(torch.float32, -10.5), (torch.float32, -25.0), (torch.bfloat16, -10.5),
                                         (torch.bfloat16, -25.0), (torch.bfloat16, -80.0)])
def test_bwd_steep_decay_mid_sequence(dtype, steep):
    # One 120-token sequence with log a = steep on tokens 30-55: 16-token pieces
    # spanning up to 1280 nats, beyond the backward's factor split (160 nats), take
    # one exponent per term, and the chunk states after the stretch come from the
    # forward rerun, whose chunks with tokens below log2 a = -12 take their own
    # exact path.
    base = "kda_t64_d16_fp32" if dtype == torch.float32 else "kda_b2_h32_t32768_d128_bf16"
    d = 32 if dtype == torch.float32 else 64
    inp = draw(base, 6, [120], dk=d, dv=d)
    la = inp["log_a"].clone()
    la[30:56] = steep
    inp["log_a"] = la
    got = gpu_grad(inp)
    for n in NAMES:
        assert torch.isfinite(got[n].float()).all(), n
    check(inp, got, TOL[dtype], f"steep decay {dtype} mid-sequence")


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


@pytest.mark.parametrize("dtype,d,lengths,scalar", [(torch.bfloat16, 128, [130, 64, 37], False),
                                                    (torch.bfloat16, 64, [300, 63, 128], True),
                                                    (torch.float32, 32, [150, 64], False)])
def test_bwd_saved_states(dtype, d, lengths, scalar):
    """The forward's states at every 64th token, passed in, give the gradients of
    the call that reruns the prefill, bit for bit, and the oracle's."""
    log(f"backward from saved states {dtype} d={d} lengths={lengths} scalar={scalar}")
    inp = draw("kda_b2_h32_t32768_d128_bf16", 21 + d, lengths, dtype=dtype, dk=d, dv=d, scalar_decay=scalar)
    _, _, states = kda.chunk_fwd_snapshots(inp["q"], inp["k"], inp["v"], inp["log_a"], inp["beta"], S0=inp["S0"],
                                           cu_seqlens=inp["cu_seqlens"], snapshot_every=64)
    assert states.shape[0] == sum(n // 64 for n in lengths)
    saved = gpu_grad(inp, states=states)
    rerun = gpu_grad(inp)
    for n in NAMES:
        assert torch.equal(saved[n], rerun[n]), n
    check(inp, saved, TOL[dtype], "saved states")


def test_bwd_saved_states_equal_lengths():
    """Without cu_seqlens (two sequences of 192 tokens): the rows are checked on
    the host, and the smaller workspace suffices."""
    log("backward from saved states, equal lengths")
    inp = draw("kda_b2_h32_t32768_d128_bf16", 33, [192, 192])
    args = (inp["q"], inp["k"], inp["v"], inp["log_a"], inp["beta"])
    _, _, states = kda.chunk_fwd_snapshots(*args, S0=inp["S0"], num_seqs=2, snapshot_every=64)
    assert states.shape[0] == 6
    need = kda.chunk_bwd_workspace_size(inp["q"], inp["v"], num_seqs=2, max_seqlen=192, saved=True)
    assert need < kda.chunk_bwd_workspace_size(inp["q"], inp["v"], num_seqs=2, max_seqlen=192)
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    got = kda.chunk_bwd(*args, inp["dO"], S0=inp["S0"], dS_T=inp["dST"], num_seqs=2, states=states, workspace=ws)
    torch.cuda.synchronize()
    check(inp, got, TOL[torch.bfloat16], "saved states, equal lengths")
    with pytest.raises(ValueError):
        kda.chunk_bwd(*args, inp["dO"], S0=inp["S0"], num_seqs=2, states=states[:5])


@pytest.mark.parametrize("dtype,dk,dv,lengths", [(torch.bfloat16, 128, 128, [130, 64, 37]),
                                                 (torch.bfloat16, 64, 64, [300, 1, 0, 79]),
                                                 (torch.bfloat16, 128, 64, [150, 20]),
                                                 (torch.float32, 32, 32, [150, 64]),
                                                 (torch.float32, 16, 16, [100, 3])])
def test_bwd_decay_first(dtype, dk, dv, lengths):
    """The decay-first order's gradient (the chunk form with each token's decay
    before its own read) against the oracle's order-1 gradient."""
    log(f"backward decay-first {dtype} dk={dk} dv={dv} lengths={lengths}")
    inp = draw("kda_b2_h32_t32768_d128_bf16", 90 + dk + dv, lengths, dtype=dtype, dk=dk, dv=dv)
    got = gpu_grad(inp, order=kda.ORDER_DECAY_FIRST)
    check(inp, got, TOL[dtype], f"decay-first {dtype} dk {dk} dv {dv}", order=1)
    # a different gradient from the erase-first one on the same inputs
    other = gpu_grad(inp)
    assert max_rel_err(other["dlog_a"], got["dlog_a"]) > 1e-3


@pytest.mark.parametrize("dtype,steep", [(torch.float32, -25.0), (torch.bfloat16, -80.0)])
def test_bwd_decay_first_steep_mid_sequence(dtype, steep):
    """Steep decays in the middle of a sequence (sub-chunks past the factor split's
    range take one exponent per term), decay-first order."""
    log(f"backward decay-first steep {dtype} {steep}")
    d = 32 if dtype == torch.float32 else 128
    inp = draw("kda_b2_h32_t32768_d128_bf16", 97, [120], dtype=dtype, dk=d, dv=d)
    la = inp["log_a"].clone()
    la[30:56, :, ::2] = steep
    inp["log_a"] = la.contiguous()
    got = gpu_grad(inp, order=kda.ORDER_DECAY_FIRST)
    check(inp, got, TOL[dtype], f"decay-first steep {dtype}", order=1)


def test_bwd_decay_first_saved_states():
    """From the decay-first forward's kept states: bit for bit the rerun's gradients."""
    inp = draw("kda_b2_h32_t32768_d128_bf16", 98, [200, 64, 33])
    _, _, states = kda.chunk_fwd_snapshots(inp["q"], inp["k"], inp["v"], inp["log_a"], inp["beta"], S0=inp["S0"],
                                           cu_seqlens=inp["cu_seqlens"], snapshot_every=64,
                                           order=kda.ORDER_DECAY_FIRST)
    saved = gpu_grad(inp, states=states, order=kda.ORDER_DECAY_FIRST)
    rerun = gpu_grad(inp, order=kda.ORDER_DECAY_FIRST)
    for n in NAMES:
        assert torch.equal(saved[n], rerun[n]), n
    check(inp, saved, TOL[torch.bfloat16], "decay-first saved states", order=1)


PRO = dict(normalize_k=True, beta_logits=True, log_a_raw=True, log_a_min=-6.0)


def raw_draw(dtype, d, lengths, seed, scalar=False):
    from kda_recurrent_state_amd.workloads import generate_raw
    w = scaled(WORKLOADS["kda_varlen_64seq_h32_d128"], n_seqs=len(lengths), heads=2, dk=d, dv=d, dtype=dtype,
               scalar_decay=scalar, s0_std=0.3)
    inp = generate_raw(w, seed, DEV, lengths=lengths)
    g = torch.Generator(device=DEV)
    g.manual_seed(seed + 1000)
    T = int(np.sum(lengths))
    inp["dO"] = torch.randn((T, 2, d), generator=g, device=DEV).to(dtype)
    inp["dST"] = torch.randn((len(lengths), 2, d, d), generator=g, device=DEV)
    return inp


def oracle_grad_pro(inp, pro):
    c = lambda t: None if t is None else t.detach().cpu()
    return kda_oracle_bwd(c(inp["q"]), c(inp["k"]), c(inp["v"]), c(inp["log_a"]), c(inp["beta"]), S0=c(inp["S0"]),
                          cu_seqlens=inp["cu_seqlens"].cpu().numpy(), dO=c(inp["dO"]), dST=c(inp["dST"]), pro=pro)


@pytest.mark.parametrize("dtype,d,scalar,saved", [(torch.bfloat16, 128, False, False), (torch.bfloat16, 64, True, False),
                                                  (torch.float32, 32, False, False), (torch.bfloat16, 128, False, True),
                                                  (torch.float32, 16, True, True)])
def test_bwd_prologue(dtype, d, scalar, saved):
    """Gradient with respect to the raw inputs of a forward that ran the input
    prologue (kda_chunk_bwd_ex), from a rerun or from the forward's kept
    states, against the oracle's gradient through the same prologue."""
    log(f"backward with prologue {dtype} d={d} scalar={scalar} saved={saved}")
    inp = raw_draw(dtype, d, [150, 64, 37], 70 + d + scalar, scalar)
    states = None
    if saved:
        _, _, states = kda.chunk_fwd_snapshots(inp["q"], inp["k"], inp["v"], inp["log_a"], inp["beta"],
                                               S0=inp["S0"], cu_seqlens=inp["cu_seqlens"], snapshot_every=64,
                                               prologue=PRO)
    got = gpu_grad(inp, prologue=PRO, states=states)
    ref = oracle_grad_pro(inp, PRO)
    errs = {n: max_rel_err(got[n], ref[n]) for n in NAMES}
    log("  " + " ".join(f"{n} {e:.2e}" for n, e in errs.items()))
    bad = {n: e for n, e in errs.items() if not e <= TOL[dtype]}
    assert not bad, bad


def test_bwd_prologue_off_is_plain():
    """An all-zero prologue is the plain call, bit for bit."""
    inp = draw("kda_b2_h32_t32768_d128_bf16", 77, [100, 30])
    a = gpu_grad(inp)
    b = gpu_grad(inp, prologue=dict())
    for n in NAMES:
        assert torch.equal(a[n], b[n]), n


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


def test_bwd_gdn_h16_t4096_full():
    """Gated DeltaNet at its full size (1 x 16 heads x 4096 tokens, d = 128,
    bf16, scalar gate): every gradient element of the whole batch against the
    oracle, both from a prefill rerun and from the forward's kept states."""
    log("backward C2 full: GDN H=16 T=4096, whole batch")
    inp = generate(WORKLOADS["gdn_h16_t4096_d128_bf16"], 2, DEV)
    g = torch.Generator(device=DEV)
    g.manual_seed(7)
    T, H = inp["q"].shape[0], inp["q"].shape[1]
    inp["dO"] = torch.randn((T, H, inp["v"].shape[2]), generator=g, device=DEV).to(inp["q"].dtype)
    inp["dST"] = torch.randn((1, H, inp["q"].shape[2], inp["v"].shape[2]), generator=g, device=DEV)
    if inp["cu_seqlens"] is None:
        inp["cu_seqlens"] = torch.tensor([0, T], dtype=torch.int32, device=DEV)
    got = gpu_grad(inp)
    check(inp, got, TOL[torch.bfloat16], "C2 whole batch")
    _, _, states = kda.chunk_fwd_snapshots(inp["q"], inp["k"], inp["v"], inp["log_a"], inp["beta"], S0=inp["S0"],
                                           cu_seqlens=inp["cu_seqlens"], snapshot_every=64)
    kept = gpu_grad(inp, states=states)
    for n in NAMES:
        if got.get(n) is not None:
            assert torch.equal(got[n], kept[n]), n  # the rerun keeps the same states
