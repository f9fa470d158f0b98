"""Pins for the oracle's gradient (``oracle.kda_oracle_bwd``).

Each pin takes a callable with the signature of ``oracle.kda_oracle_bwd`` and
raises AssertionError when it disagrees with a fact that does not come from the
backward walk itself:

- central finite differences of the forward oracle (which has pins of its own),
  along random directions in every input at once and at single elements;
- the closed form of the gradient when no token writes (beta = 0: the state only
  decays, S_t = Diag(exp(g_t)) S0, and o_t = (q_t * exp(g_t)) S0);
- torch's automatic differentiation of a plain torch token loop in float64;
- linearity of the gradient in (dO, dS_T), and the reduction of a uniform
  per-channel gate to the scalar gate (where the two orderings coincide).

The same pins run against copies of the oracle with planted mistakes in the
backward walk, each of which must break at least one of them.
"""
from __future__ import annotations

import numpy as np

import oracle
from tests.oracle_pins import _close, _random_case

NAMES = ("dq", "dk", "dv", "dlog_a", "dbeta", "dS0")


def _case(seed, T=23, H=2, dk=5, dv=4, scalar=False, cu=(0, 9, 9, 23)):
    rng = np.random.default_rng(seed)
    n = len(cu) - 1
    q, k, v, la, beta, S0 = _random_case(rng, T, H, dk, dv, scalar=scalar, n_seqs=n)
    dO = rng.standard_normal((T, H, dv))
    dST = rng.standard_normal((n, H, dk, dv))
    return [q, k, v, la, beta, S0], np.array(cu, dtype=np.int64), dO, dST, rng


def _loss(args, cu, dO, dST, order):
    o, ST = oracle.kda_oracle(*args, cu_seqlens=cu, order=order)
    return float(np.sum(o * dO) + np.sum(ST * dST))


def pin_bwd_directional_differences(bwd):
    """<grad, u> equals the central difference of the loss along u, every input."""
    for order in (0, 1):
        for scalar in (False, True):
            args, cu, dO, dST, rng = _case(11 + order + 2 * scalar, scalar=scalar)
            g = bwd(*args, cu_seqlens=cu, dO=dO, dST=dST, order=order)
            for i, name in enumerate(NAMES):
                u = rng.standard_normal(args[i].shape)
                h = 1e-6
                ap = list(args); ap[i] = args[i] + h * u
                am = list(args); am[i] = args[i] - h * u
                fd = (_loss(ap, cu, dO, dST, order) - _loss(am, cu, dO, dST, order)) / (2 * h)
                got = float(np.sum(g[name] * u))
                assert abs(got - fd) <= 1e-7 * max(1.0, abs(fd)), \
                    f"order {order} scalar {scalar} {name}: <grad,u> {got:.12g} vs {fd:.12g}"


def pin_bwd_elementwise_differences(bwd):
    """Single elements (first, last, an empty sequence's neighbour) by central differences."""
    args, cu, dO, dST, rng = _case(5)
    for order in (0, 1):
        g = bwd(*args, cu_seqlens=cu, dO=dO, dST=dST, order=order)
        for i, name in enumerate(NAMES):
            shape = args[i].shape
            picks = [tuple(0 for _ in shape), tuple(s - 1 for s in shape)]
            picks += [tuple(int(rng.integers(0, s)) for s in shape) for _ in range(3)]
            for idx in picks:
                h = 1e-6
                ap = [a.copy() for a in args]; ap[i][idx] += h
                am = [a.copy() for a in args]; am[i][idx] -= h
                fd = (_loss(ap, cu, dO, dST, order) - _loss(am, cu, dO, dST, order)) / (2 * h)
                assert abs(g[name][idx] - fd) <= 1e-7 * max(1.0, abs(fd)), \
                    f"order {order} {name}{idx}: {g[name][idx]:.12g} vs {fd:.12g}"


def pin_bwd_beta_zero_closed_form(bwd):
    """beta = 0: S_t = Diag(e^{g_t}) S0, o_t = (q_t e^{g_t}) S0, gradients in closed form."""
    rng = np.random.default_rng(3)
    T, dk, dv = 9, 4, 3
    q = rng.standard_normal((T, 1, dk)); k = rng.standard_normal((T, 1, dk))
    v = rng.standard_normal((T, 1, dv)); la = -rng.uniform(0.0, 1.0, (T, 1, dk))
    beta = np.zeros((T, 1)); S0 = rng.standard_normal((1, 1, dk, dv))
    dO = rng.standard_normal((T, 1, dv)); dST = rng.standard_normal((1, 1, dk, dv))
    s0, qq, kk, vv, do, dst = S0[0, 0], q[:, 0], k[:, 0], v[:, 0], dO[:, 0], dST[0, 0]
    gam = np.exp(np.cumsum(la[:, 0], axis=0))            # [T, dk] = e^{g_t}
    gprev = np.vstack([np.ones((1, dk)), gam[:-1]])       # e^{g_{t-1}}
    dq = gam * (do @ s0.T)                                # dq_t[c] = e^{g_tc} sum_j dO_tj S0[c,j]
    dS0 = (qq * gam).T @ do + gam[-1][:, None] * dst
    w = (qq * gam) * (do @ s0.T)                          # w[s,c] = q_sc e^{g_sc} (S0 dO_s^T)_c
    dla = np.cumsum(w[::-1], axis=0)[::-1] + gam[-1] * np.sum(s0 * dst, axis=1)
    # dbeta_t = <Lam_t, dS_t/dbeta_t>, Lam_t = sum_{s>=t} e^{g_s-g_t} q_s^T dO_s + e^{g_T-g_t} dST, and
    # dS_t/dbeta_t = -D_t k^T (k S_{t-1}) + k^T v_t (erase, then decay) or -k^T (k D_t S_{t-1}) + k^T v_t
    # (decay first), with S_{t-1} = Diag(e^{g_{t-1}}) S0.
    dbeta = np.zeros((2, T))
    for t in range(T):
        lam = sum((gam[s] / gam[t])[:, None] * np.outer(qq[s], do[s]) for s in range(t, T))
        lam = lam + (gam[-1] / gam[t])[:, None] * dst
        sp = gprev[t][:, None] * s0
        a = np.exp(la[t, 0])
        dS0_ = -(a * kk[t])[:, None] * (kk[t] @ sp)[None, :] + np.outer(kk[t], vv[t])
        dS1_ = -kk[t][:, None] * ((a * kk[t]) @ sp)[None, :] + np.outer(kk[t], vv[t])
        dbeta[0, t] = np.sum(lam * dS0_)
        dbeta[1, t] = np.sum(lam * dS1_)
    for order in (0, 1):
        g = bwd(q, k, v, la, beta, S0, dO=dO, dST=dST, order=order)
        _close(g["dq"][:, 0], dq, 1e-12, f"order {order} dq")
        _close(g["dS0"][0, 0], dS0, 1e-12, f"order {order} dS0")
        _close(g["dlog_a"][:, 0], dla, 1e-12, f"order {order} dlog_a")
        _close(g["dbeta"][:, 0], dbeta[order], 1e-12, f"order {order} dbeta")
        _close(g["dk"], np.zeros_like(k), 1e-12, f"order {order} dk")
        _close(g["dv"], np.zeros_like(v), 1e-12, f"order {order} dv")


def pin_bwd_autograd(bwd):
    """torch's reverse-mode differentiation of a plain token loop (float64)."""
    import torch
    rng = np.random.default_rng(8)
    T, H, dk, dv = 13, 2, 4, 3
    q, k, v, la, beta, S0 = _random_case(rng, T, H, dk, dv)
    dO = rng.standard_normal((T, H, dv)); dST = rng.standard_normal((1, H, dk, dv))
    for order in (0, 1):
        ts = [torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v, la, beta, S0)]
        tq, tk, tv, tla, tb, tS0 = ts
        loss = 0.0
        for h in range(H):
            S = tS0[0, h]
            for t in range(T):
                a = torch.exp(tla[t, h])
                kt = tk[t, h]
                if order == 0:
                    S = a[:, None] * (S - tb[t, h] * torch.outer(kt, kt @ S)) + tb[t, h] * torch.outer(kt, tv[t, h])
                else:
                    P = a[:, None] * S
                    S = P - tb[t, h] * torch.outer(kt, kt @ P) + tb[t, h] * torch.outer(kt, tv[t, h])
                loss = loss + torch.sum((tq[t, h] @ S) * torch.tensor(dO[t, h]))
            loss = loss + torch.sum(S * torch.tensor(dST[0, h]))
        loss.backward()
        g = bwd(q, k, v, la, beta, S0, dO=dO, dST=dST, order=order)
        for name, t_ in zip(NAMES, ts):
            _close(g[name], t_.grad.numpy(), 1e-12, f"order {order} {name} vs autograd")


def pin_bwd_linearity(bwd):
    """The gradient is linear in the upstream derivatives (dO, dS_T)."""
    args, cu, dO, dST, rng = _case(21)
    dO2 = rng.standard_normal(dO.shape); dST2 = rng.standard_normal(dST.shape)
    for order in (0, 1):
        g1 = bwd(*args, cu_seqlens=cu, dO=dO, dST=dST, order=order)
        g2 = bwd(*args, cu_seqlens=cu, dO=dO2, dST=dST2, order=order)
        g12 = bwd(*args, cu_seqlens=cu, dO=2.0 * dO - 3.0 * dO2, dST=2.0 * dST - 3.0 * dST2, order=order)
        for name in NAMES:
            _close(g12[name], 2.0 * g1[name] - 3.0 * g2[name], 1e-12, f"order {order} {name} linearity")


def pin_bwd_uniform_gate_is_scalar_gate(bwd):
    """A per-channel gate that is uniform over channels is the scalar gate; both orders agree."""
    args, cu, dO, dST, rng = _case(31, scalar=True)
    q, k, v, la_s, beta, S0 = args
    la_c = np.repeat(la_s[..., None], q.shape[2], axis=2)
    gs = bwd(q, k, v, la_s, beta, S0, cu_seqlens=cu, dO=dO, dST=dST, order=0)
    for order in (0, 1):
        gc = bwd(q, k, v, la_c, beta, S0, cu_seqlens=cu, dO=dO, dST=dST, order=order)
        for name in ("dq", "dk", "dv", "dbeta", "dS0"):
            _close(gc[name], gs[name], 1e-12, f"order {order} {name}")
        _close(gc["dlog_a"].sum(axis=2), gs["dlog_a"], 1e-12, f"order {order} dlog_a summed over channels")


ALL_BWD_PINS = [
    pin_bwd_directional_differences,
    pin_bwd_elementwise_differences,
    pin_bwd_beta_zero_closed_form,
    pin_bwd_autograd,
    pin_bwd_linearity,
    pin_bwd_uniform_gate_is_scalar_gate,
]
