"""fp64 numpy model of the chunkwise gradient that the HIP backward runs.

Test infrastructure: it documents and checks the derivation of the backward
chunk form against the oracle's token-by-token gradient.  It is neither the
oracle nor the GPU path, and the GPU path does not use it.

Forward chunk form (page "The argument, in one page", table row "Chunkwise / WY"),
per sub-chunk of n <= 16 tokens with start state S, g_i = sum_{j<=i} log a_j,
gm_i = g_{i-1} (gm_0 = 0), gC = g_{n-1}, all per key channel:

  Kb = k e^{gm}, Qb = q e^{g}, Kcc = k e^{gC-gm}, Ktc = k e^{gC-g}, gamma = e^{gC}
  A0 = strict_lower(Kb (k e^{-gm})^T)   L  = strict_lower(Kb (k e^{-g})^T)
  P1 = lower(Qb (k e^{-gm})^T)          P2 = lower(Qb (k e^{-g})^T)
  T = (I + diag(b) A0)^-1
  Y0 = Kb S + L diag(b) V,  E = -T diag(b) Y0,  Y = Y0 + A0 E   (Y_i = k_i S_{i-1}, E = -diag(b) Y)
  O = Qb S + P1 E + P2 diag(b) V,   S_next = gamma * S + Kcc^T E + Ktc^T diag(b) V

Backward, for the derivative X of the loss with respect to S_next and dO with
respect to O (derived by differentiating the lines above):

  G  = T^T (P1^T dO + Kcc X)            (G_i = (k_i * a_i) Lam_i, Lam_i = dL/dS_i)
  F  = -diag(b) G
  R  = Ktc X + P2^T dO + L^T F           (R_i = k_i Lam_i)
  X_prev = gamma * X + Qb^T dO + Kb^T F  (dL/dS)
  dv = diag(b) R,   dbeta = rowsum(R * V) - rowsum(G * Y)
  dq   = e^{g}  * (dO S^T)  + e^{g}   * [lower(dO E^T) (k e^{-gm}) + lower(dO (bV)^T) (k e^{-g})]
  gs   = e^{gm} * (G S^T)   + e^{gm}  * [strict_lower(G E^T) (k e^{-gm}) + strict_lower(G (bV)^T) (k e^{-g})]
  vds  = e^{gC-g}  * (V X^T) + e^{-g}  * [upper(V dO^T) Qb + strict_upper(V F^T) Kb]
  ayds = e^{gC-gm} * (Y X^T) + e^{-gm} * [upper(Y dO^T) Qb + strict_upper(Y F^T) Kb]
  dk = diag(b) (vds - ayds - gs)
  dlog_a_i = phi_i - b_i k_i * vds_i,  phi_i = rowsum(Lam_i * S_i) by telescoping:
      phi_{-1} = rowsum(X_prev * S),  phi_i - phi_{i-1} = k_i * dk_i + 2 b_i k_i * gs_i - q_{i-1} * dq_{i-1}
      (the last term only for i >= 1 inside the sub-chunk).

For matrix cores the decay factors inside a sub-chunk are split around a per
channel reference m = (gm_0 + gC) / 2: (k e^{-gm}) e^{g} = (k e^{m-gm}) e^{g-m}
and so on, each factor at most e^{span/2}.  When a channel's span -gC exceeds
SPAN_MAX the model (and the kernels) evaluate those products with one exponent
per term instead.

Decay-first order, S_i = (I - b_i k_i^T k_i) D_i S_{i-1} + b_i k_i^T v_i: the read of
token i sees the state after its own decay, Y_i = k_i D_i S_{i-1}, and the erase and
the write share the key.  Its chunk form is the lines above with every gm replaced
by g (Kb = k e^{g}, A0 = L, P1 = P2, Kcc = Ktc), and so are the reverse walk and the
products dq, gs, vds, ayds and dk, and the telescoping of phi.  Only the last step
of dlog_a changes: with Lam_i = dL/dS_i and P_i = D_i S_{i-1},
  dlog_a_i = rowsum(dL/dP_i * P_i) = phi_i - k_i * dk_i - 2 b_i k_i * gs_i,
since dL/dP_i = (I - b k^T k) Lam_i, P_i = S_i + b_i k_i^T (Y_i - v_i),
dk_i = b_i (Lam_i v_i^T - Lam_i Y_i^T - P_i (k_i Lam_i)^T) and gs_i = P_i (k_i Lam_i)^T:
the sum of the telescoping step's own terms taken off phi_i.

Levels, for a sequence of chunks of CH = 64 tokens split into sub-chunks of 16:
  1. forward states at every chunk start;
  2. the reverse walk X <- X_prev over all sub-chunks (X = dS_T at the end),
     keeping X at every chunk end;
  3. per chunk, its sub-chunks in reverse order with X carried, each sub-chunk's
     start state recomputed from the chunk's start state.
"""
from __future__ import annotations

import numpy as np

SUB = 16
CH = 64
SPAN_MAX = 160.0


def _tril(M, d):
    return np.tril(M, d)


def _triu(M, d):
    return np.triu(M, d)


def sub_ops(q, k, la, beta, exact=None, ord1=False):
    """Per sub-chunk operators.  q, k [n, dk]; la [n, dk]; beta [n].  ord1: the
    decay-first order (gm replaced by g)."""
    n, dk = k.shape
    G = np.vstack([np.zeros((1, dk)), np.cumsum(la, axis=0)])  # G[i] = g_{i-1}, G[n] = gC
    gm, g, gC = G[:-1], G[1:], G[-1]
    if ord1:
        gm = g
    span = float(np.max(-gC)) if n else 0.0
    if exact is None:
        exact = span > SPAN_MAX
    m = 0.5 * gC
    o = dict(n=n, q=q, k=k, beta=beta, G=G, gm=gm, g=g, gC=gC, m=m, exact=exact, ord1=ord1)
    o["Kb"] = k * np.exp(gm)
    o["Qb"] = q * np.exp(g)
    o["Kcc"] = k * np.exp(gC - gm)
    o["Ktc"] = k * np.exp(gC - g)
    o["gamma"] = np.exp(gC)

    def gram(x, hx, y, hy, d):
        # sum_c x_tc y_ic e^{hx_tc - hy_ic}, masked by tril(d)
        if exact:
            M = np.einsum("tc,ic,tic->ti", x, y, np.exp(hx[:, None, :] - hy[None, :, :]))
        else:
            M = (x * np.exp(hx - m)) @ (y * np.exp(m - hy)).T
        return _tril(M, d)

    o["A0"] = gram(k, gm, k, gm, -1)
    o["L"] = gram(k, gm, k, g, -1)
    o["P1"] = gram(q, g, k, gm, 0)
    o["P2"] = gram(q, g, k, g, 0)
    o["T"] = np.linalg.inv(np.eye(n) + beta[:, None] * o["A0"])
    return o


def masked_rows(o, M, y, hrow, hcol, sign):
    """out[t,c] = sum_i M[t,i] y_ic e^{sign (hrow_tc - hcol_ic)} for the (already masked) M."""
    m = o["m"]
    if o["exact"]:
        return np.einsum("ti,ic,tic->tc", M, y, np.exp(sign * (hrow[:, None, :] - hcol[None, :, :])))
    return np.exp(sign * (hrow - m)) * (M @ (y * np.exp(sign * (m - hcol))))


def sub_forward(o, v, S):
    b = o["beta"]
    bV = b[:, None] * v
    Y0 = o["Kb"] @ S + o["L"] @ bV
    E = -o["T"] @ (b[:, None] * Y0)
    Y = Y0 + o["A0"] @ E
    S_next = o["gamma"][:, None] * S + o["Kcc"].T @ E + o["Ktc"].T @ bV
    return E, Y, S_next


def sub_reverse(o, dO, X):
    b = o["beta"]
    G = o["T"].T @ (o["P1"].T @ dO + o["Kcc"] @ X)
    F = -b[:, None] * G
    X_prev = o["gamma"][:, None] * X + o["Qb"].T @ dO + o["Kb"].T @ F
    return G, F, X_prev


def sub_grads(o, v, dO, S, X):
    """Gradients of one sub-chunk given its start state S and the end derivative X."""
    q, k, b = o["q"], o["k"], o["beta"]
    g, gm, gC = o["g"], o["gm"], o["gC"]
    E, Y, _ = sub_forward(o, v, S)
    G, F, X_prev = sub_reverse(o, dO, X)
    bV = b[:, None] * v
    R = o["Ktc"] @ X + o["P2"].T @ dO + o["L"].T @ F
    dv = b[:, None] * R
    dbeta = np.sum(R * v, axis=1) - np.sum(G * Y, axis=1)
    dq = np.exp(g) * (dO @ S.T) + masked_rows(o, _tril(dO @ E.T, 0), k, g, gm, 1) \
        + masked_rows(o, _tril(dO @ bV.T, 0), k, g, g, 1)
    gs = np.exp(gm) * (G @ S.T) + masked_rows(o, _tril(G @ E.T, -1), k, gm, gm, 1) \
        + masked_rows(o, _tril(G @ bV.T, -1), k, gm, g, 1)
    vds = np.exp(gC - g) * (v @ X.T) + masked_rows(o, _triu(v @ dO.T, 0), q, g, g, -1) \
        + masked_rows(o, _triu(v @ F.T, 1), k, g, gm, -1)
    ayds = np.exp(gC - gm) * (Y @ X.T) + masked_rows(o, _triu(Y @ dO.T, 0), q, gm, g, -1) \
        + masked_rows(o, _triu(Y @ F.T, 1), k, gm, gm, -1)
    dk = b[:, None] * (vds - ayds - gs)
    own = k * dk + 2.0 * b[:, None] * k * gs
    diff = own.copy()
    diff[1:] -= q[:-1] * dq[:-1]
    phi = np.sum(X_prev * S, axis=1)[None, :] + np.cumsum(diff, axis=0)
    dla = phi - own if o["ord1"] else phi - b[:, None] * k * vds
    return dict(dq=dq, dk=dk, dv=dv, dlog_a=dla, dbeta=dbeta), X_prev


def chunk_backward(q, k, v, la, beta, S0, dO, dST, exact=None, ord1=False):
    """One (sequence, head): returns the oracle's gradient dict (without batch axes)."""
    T, dk = q.shape
    dv = v.shape[1]
    subs = [(s, min(s + SUB, T)) for s in range(0, T, SUB)]
    ops = [sub_ops(q[s:e], k[s:e], la[s:e], beta[s:e], exact, ord1) for s, e in subs]
    per_chunk = CH // SUB
    # level 1: states at chunk starts
    S = S0.copy()
    starts = []
    for i, (s, e) in enumerate(subs):
        if i % per_chunk == 0:
            starts.append(S.copy())
        _, _, S = sub_forward(ops[i], v[s:e], S)
    # level 2: reverse walk, X at every chunk end
    X = dST.copy()
    ends = [None] * len(starts)
    for i in reversed(range(len(subs))):
        s, e = subs[i]
        if i % per_chunk == per_chunk - 1 or i == len(subs) - 1:
            ends[i // per_chunk] = X.copy()
        _, _, X = sub_reverse(ops[i], dO[s:e], X)
    dS0 = X
    # level 3: per chunk, sub-chunks in reverse with recomputed start states
    out = {n: np.zeros_like(a) for n, a in (("dq", q), ("dk", k), ("dv", v), ("dlog_a", la))}
    out["dbeta"] = np.zeros(T)
    for c in range(len(starts)):
        idx = list(range(c * per_chunk, min((c + 1) * per_chunk, len(subs))))
        X = ends[c]
        for j in reversed(range(len(idx))):
            S = starts[c]
            for jj in range(j):
                s, e = subs[idx[jj]]
                _, _, S = sub_forward(ops[idx[jj]], v[s:e], S)
            s, e = subs[idx[j]]
            g, X = sub_grads(ops[idx[j]], v[s:e], dO[s:e], S, X)
            for n_ in g:
                out[n_][s:e] = g[n_]
    out["dS0"] = dS0
    return out
