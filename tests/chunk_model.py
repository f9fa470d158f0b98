"""fp64 numpy model of the chunkwise (WY) algorithm that the HIP prefill runs.

Test infrastructure: it documents and checks the derivation of the chunk form
(page "The argument, in one page", table row "Chunkwise / WY": the same update,
reorganised so each chunk of C tokens needs one C x C triangular solve plus dense
products) against the token-by-token oracle.  It is neither the oracle nor the
GPU path, and the GPU path does not use it.

Derivation, per (sequence, head) and chunk, local tokens t = 0..C-1, state S0 at
the chunk start, g_t = sum_{j<=t} log a_j (per key channel), with X_t = Diag(e^-g_t) S_t:

  X_t = X_{t-1} + kc_t^T e_t + kt_t^T (b_t v_t),   e_t = -b_t kb_t X_{t-1}
  kb_t = k_t e^{g_{t-1}}, kc_t = k_t e^{-g_{t-1}}, kt_t = k_t e^{-g_t}, qb_t = q_t e^{g_t}

Solving the recurrence for the rows e_t of E gives (I + A) E = -diag(b) Kb S0 - diag(b) L diag(b) V:

  A  = strict_lower(diag(b) Kb Kc^T)      L  = strict_lower(Kb Kt^T)
  P1 = lower(Qb Kc^T)                      P2 = lower(Qb Kt^T)
  T = (I + A)^-1,  W = T diag(b) Kb,  U = T diag(b) L diag(b) V,  E = -(W S0 + U)
  O   = Qb S0 + P1 E + P2 diag(b) V
  S_C = Diag(e^{g_C}) S0 + (Kc Diag(e^{g_C}))^T E + (Kt Diag(e^{g_C}))^T diag(b) V

Every exponent kept by the masks is <= 0.  For the products on matrix cores the
decay factors are split into a row factor and a column factor around a
reference per 16-token sub-block: the mid-block value of g for blocks on the
diagonal (both factors stay within e^{+-8*8.5} for |log a| <= 8), and for a
block pair (bt > bi) the row factor is additionally scaled by e^{mu_bt - mu_bi}
<= 1; that product can only underflow where the true term is below ~1e-8 of
the largest factor product, so dropping it is harmless.
"""
from __future__ import annotations

import numpy as np

SUB = 16  # sub-block length for the decay references


def _bf16(x):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16).to(
        torch.float64).numpy()


def _unit_lower_inverse(A):
    """(I + A)^-1 for strictly lower A by 16x16 blocks: diagonal blocks by
    forward substitution, off-diagonal blocks by T_ij = -T_ii sum_k A_ik T_kj."""
    C = A.shape[0]
    nb = (C + SUB - 1) // SUB
    T = np.zeros_like(A)
    for b in range(nb):
        s = slice(b * SUB, min(C, (b + 1) * SUB))
        Ab = A[s, s]
        n = Ab.shape[0]
        Tb = np.eye(n)
        for r in range(n):
            for j in range(r):
                Tb[r, j] = -Ab[r, j:r] @ Tb[j:r, j]
        T[s, s] = Tb
    for bi in range(nb):
        for bj in range(bi):
            si = slice(bi * SUB, min(C, (bi + 1) * SUB))
            acc = np.zeros((si.stop - si.start, min(C, (bj + 1) * SUB) - bj * SUB))
            for bk in range(bj, bi):
                sk = slice(bk * SUB, min(C, (bk + 1) * SUB))
                acc += A[si, sk] @ T[sk, bj * SUB:min(C, (bj + 1) * SUB)]
            T[si, bj * SUB:min(C, (bj + 1) * SUB)] = -T[si, si] @ acc
    return T


def chunk_step(q, k, v, la, beta, S, bf16=False):
    """One chunk (C tokens, C a multiple of 16) of one (sequence, head).
    q, k [C, dk]; v [C, dv]; la [C, dk]; beta [C]; S [dk, dv].  Returns (O, S_C).
    bf16=True rounds every matrix-core operand to bf16 as the GPU path does."""
    C, dk = q.shape
    rnd = _bf16 if bf16 else (lambda x: x)
    nb = C // SUB
    # cumulative log-decay, local to each sub-block, and block offsets
    lam = np.zeros((C, dk))
    Lam = np.zeros((nb, dk))
    for b in range(nb):
        lam[b * SUB:(b + 1) * SUB] = np.cumsum(la[b * SUB:(b + 1) * SUB], axis=0)
        Lam[b] = lam[(b + 1) * SUB - 1]
    rho = np.concatenate([np.zeros((1, dk)), np.cumsum(Lam, axis=0)])  # [nb+1, dk]
    gC = rho[nb]
    mid = np.array([lam[b * SUB + SUB // 2 - 1] for b in range(nb)])  # local g at mid
    mu = rho[:nb] + mid  # absolute g at mid
    rin = np.zeros((C, dk))
    rex = np.zeros((C, dk))
    for t in range(C):
        b = t // SUB
        rin[t] = np.exp(lam[t] - mid[b])
        prev = lam[t - 1] if t % SUB else np.zeros(dk)
        rex[t] = np.exp(prev - mid[b])
    cin, cex = 1.0 / rin, 1.0 / rex
    blk = np.arange(C) // SUB
    emu = np.exp(mu)[blk]  # e^{mu_b} per token row
    ecmu = np.exp(gC[None, :] - mu)[blk]
    Kr, Qr, Kce, Kci = rnd(k * rex), rnd(q * rin), rnd(k * cex), rnd(k * cin)
    Kbar = rnd(k * rex * emu)
    Qbar = rnd(q * rin * emu)
    Kcc = rnd(k * cex * ecmu)
    Ktc = rnd(k * cin * ecmu)
    A = np.zeros((C, C)); L = np.zeros((C, C)); P1 = np.zeros((C, C)); P2 = np.zeros((C, C))
    for bt in range(nb):
        st = slice(bt * SUB, (bt + 1) * SUB)
        for bi in range(bt + 1):
            si = slice(bi * SUB, (bi + 1) * SUB)
            if bt == bi:
                kr, qr = Kr[st], Qr[st]
            else:
                F = np.exp(mu[bt] - mu[bi])
                kr, qr = rnd(Kr[st] * F), rnd(Qr[st] * F)
            A[st, si] = kr @ Kce[si].T
            L[st, si] = kr @ Kci[si].T
            P1[st, si] = qr @ Kce[si].T
            P2[st, si] = qr @ Kci[si].T
    A = np.tril(A, -1) * beta[:, None]
    L = np.tril(L, -1)
    P1 = np.tril(P1)
    P2 = np.tril(P2)
    T = _unit_lower_inverse(A)
    bV = rnd(beta[:, None] * v)
    Tb = rnd(T * beta[None, :])  # T diag(b), shared by W and U
    W = rnd(Tb @ Kbar)
    U = Tb @ rnd(rnd(L) @ bV)
    E = -(W @ rnd(S) + U)
    Er = rnd(E)
    O = Qbar @ rnd(S) + rnd(P1) @ Er + rnd(P2) @ bV
    S_new = np.exp(gC)[:, None] * S + Kcc.T @ Er + Ktc.T @ bV
    return O, S_new


def chunk_forward(q, k, v, la, beta, S0=None, C=64, bf16=False):
    """Whole sequence of one head: q, k [T, dk], v [T, dv], la [T, dk] or [T],
    beta [T].  Partial last chunk padded with k=q=v=0, beta=0, log a=0."""
    T, dk = q.shape
    dv = v.shape[1]
    if la.ndim == 1:
        la = np.repeat(la[:, None], dk, axis=1)
    S = np.zeros((dk, dv)) if S0 is None else np.array(S0, dtype=np.float64)
    O = np.zeros((T, dv))
    for s in range(0, T, C):
        e = min(T, s + C)
        n = e - s
        pad = lambda x, w: np.concatenate([x[s:e], np.zeros((C - n,) + x.shape[1:])]) if n < C else x[s:e]
        Oc, S = chunk_step(pad(q, 0), pad(k, 0), pad(v, 0), pad(la, 0), pad(beta, 0), S, bf16=bf16)
        O[s:e] = Oc[:n]
    return O, S


def chunk_operators(q, k, la, beta, bf16=False):
    """The value-independent operators of one chunk, in the factored form the
    two-kernel GPU prefill uses (a chunk-parallel pass computes these; the
    sequential pass only applies them):

      W  = T diag(b) Kb              M1 = T diag(b) L diag(b)
      Q' = Qb - P1 W                 M2 = P2 diag(b) - P1 M1
      Kc' = Kc Diag(e^{g_C})         Kt' = diag(b) Kt Diag(e^{g_C}),   G = e^{g_C}

    so that, with E = -(W S + M1 V):
      O = Q' S + M2 V,   S_C = Diag(G) S + Kc'^T E + Kt'^T V.
    bf16=True rounds each operator once, where the GPU stores it."""
    C, dk = q.shape
    rnd = _bf16 if bf16 else (lambda x: x)
    nb = C // SUB
    lam = np.zeros((C, dk))
    Lam = np.zeros((nb, dk))
    for b in range(nb):
        lam[b * SUB:(b + 1) * SUB] = np.cumsum(la[b * SUB:(b + 1) * SUB], axis=0)
        Lam[b] = lam[(b + 1) * SUB - 1]
    rho = np.concatenate([np.zeros((1, dk)), np.cumsum(Lam, axis=0)])
    gC = rho[nb]
    mid = np.array([lam[b * SUB + SUB // 2 - 1] for b in range(nb)])
    mu = rho[:nb] + mid
    rin = np.zeros((C, dk))
    rex = np.zeros((C, dk))
    for t in range(C):
        b = t // SUB
        rin[t] = np.exp(lam[t] - mid[b])
        prev = lam[t - 1] if t % SUB else np.zeros(dk)
        rex[t] = np.exp(prev - mid[b])
    cin, cex = 1.0 / rin, 1.0 / rex
    blk = np.arange(C) // SUB
    emu = np.exp(mu)[blk]
    ecmu = np.exp(gC[None, :] - mu)[blk]
    Kr, Qr, Kce, Kci = rnd(k * rex), rnd(q * rin), rnd(k * cex), rnd(k * cin)
    Kbar = rnd(k * rex * emu)
    Qbar = q * rin * emu
    A = np.zeros((C, C)); L = np.zeros((C, C)); P1 = np.zeros((C, C)); P2 = np.zeros((C, C))
    for bt in range(nb):
        st = slice(bt * SUB, (bt + 1) * SUB)
        for bi in range(bt + 1):
            si = slice(bi * SUB, (bi + 1) * SUB)
            if bt == bi:
                kr, qr = Kr[st], Qr[st]
            else:
                F = np.exp(mu[bt] - mu[bi])
                kr, qr = rnd(Kr[st] * F), rnd(Qr[st] * F)
            A[st, si] = kr @ Kce[si].T
            L[st, si] = kr @ Kci[si].T
            P1[st, si] = qr @ Kce[si].T
            P2[st, si] = qr @ Kci[si].T
    A = np.tril(A, -1) * beta[:, None]
    Lb = rnd(np.tril(L, -1) * beta[None, :])
    P1 = rnd(np.tril(P1))
    P2b = np.tril(P2) * beta[None, :]
    Tb = rnd(_unit_lower_inverse(A) * beta[None, :])
    W = rnd(Tb @ Kbar)
    M1 = rnd(Tb @ Lb)
    Qp = rnd(Qbar - P1 @ W)
    M2 = rnd(P2b - P1 @ M1)
    Kc2 = rnd(k * cex * ecmu)
    Kt2 = rnd(beta[:, None] * k * cin * ecmu)
    return dict(W=W, Qp=Qp, M1=M1, M2=M2, Kc=Kc2, Kt=Kt2, G=np.exp(gC))


def chunk_apply(ops, v, S, bf16=False):
    """The sequential part: apply one chunk's operators to the state."""
    rnd = _bf16 if bf16 else (lambda x: x)
    V = rnd(v)
    Sr = rnd(S)
    E = rnd(-(ops["W"] @ Sr + ops["M1"] @ V))
    O = ops["Qp"] @ Sr + ops["M2"] @ V
    S_new = ops["G"][:, None] * S + ops["Kc"].T @ E + ops["Kt"].T @ V
    return O, S_new


def chunk_forward_split(q, k, v, la, beta, S0=None, C=32, bf16=False):
    """chunk_forward through chunk_operators / chunk_apply (same padding)."""
    T, dk = q.shape
    dv = v.shape[1]
    if la.ndim == 1:
        la = np.repeat(la[:, None], dk, axis=1)
    S = np.zeros((dk, dv)) if S0 is None else np.array(S0, dtype=np.float64)
    O = np.zeros((T, dv))
    for s in range(0, T, C):
        e = min(T, s + C)
        n = e - s
        pad = lambda x: np.concatenate([x[s:e], np.zeros((C - n,) + x.shape[1:])]) if n < C else x[s:e]
        ops = chunk_operators(pad(q), pad(k), pad(la), pad(beta), bf16=bf16)
        Oc, S = chunk_apply(ops, pad(v), S, bf16=bf16)
        O[s:e] = Oc[:n]
    return O, S


def exact_chunk_step(q, k, v, la, beta, S, order=0, dtype=np.float32):
    """One chunk by the path the kernels take for a chunk whose decay is too steep
    for the factor split: every decay factor is 2^(a run of consecutive log2
    decays, summed in order), evaluated in `dtype` (float32 as on the GPU); no
    exponent is the difference of two large sums.
      A  (t,i) = b_t sum_c k_t k_i 2^{la_i + .. + la_{t-1}}    (order 1: 2^{la_{i+1} + .. + la_t})
      L  (t,i) =     sum_c k_t k_i 2^{la_{i+1} + .. + la_{t-1}}
      P1 (t,i) =     sum_c q_t k_i 2^{la_i + .. + la_t}
      P2 (t,i) =     sum_c q_t k_i 2^{la_{i+1} + .. + la_t}
    with running sums over t for each key row i, and the chunk-referenced
    operands from prefix (g_{t-1}, g_t) and suffix (g_C - g_{t-1}, g_C - g_t) sums.
    Returns (O, S_C) in float64."""
    C, dk = q.shape
    f = lambda x: np.asarray(x, dtype=dtype)
    l2 = f(la * np.log2(np.e))
    kq, qq = f(k), f(q)
    A = np.zeros((C, C)); Lm = np.zeros((C, C)); P1 = np.zeros((C, C)); P2 = np.zeros((C, C))
    for i in range(C):
        s = np.zeros(dk, dtype=dtype)  # la_{i+1} + ... + la_{t-1}
        for t in range(i, C):
            kk, qk = kq[t] * kq[i], qq[t] * kq[i]
            if t == i:
                P1[t, i] = np.sum(qk * np.exp2(l2[t]))
                P2[t, i] = np.sum(qk)
                continue
            e2 = s + l2[t]
            P2[t, i] = np.sum(qk * np.exp2(e2))
            if order:
                A[t, i] = beta[t] * np.sum(kk * np.exp2(e2))
            else:
                A[t, i] = beta[t] * np.sum(kk * np.exp2(s + l2[i]))
                Lm[t, i] = np.sum(kk * np.exp2(s))
                P1[t, i] = np.sum(qk * np.exp2(e2 + l2[i]))
            s = s + l2[t]
    pre = np.zeros((C, dk), dtype=dtype)   # g_{t-1}
    suf = np.zeros((C, dk), dtype=dtype)   # g_C - g_t
    run = np.zeros(dk, dtype=dtype)
    for t in range(C):
        pre[t] = run
        run = run + l2[t]
    gC = run
    run = np.zeros(dk, dtype=dtype)
    for t in range(C - 1, -1, -1):
        suf[t] = run
        run = run + l2[t]
    g = pre + l2
    T = np.linalg.inv(np.eye(C) + A)
    bV = beta[:, None] * v
    Qb = q * np.exp2(g)
    gam = np.exp2(gC)[:, None]
    if order:
        Kd = k * np.exp2(g)
        U = T @ (beta[:, None] * (v - Kd @ S))
        O = Qb @ S + P2 @ U
        S_C = gam * S + (k * np.exp2(suf)).T @ U
        return O, S_C
    Kb = k * np.exp2(pre)
    E = -(T @ (beta[:, None] * (Kb @ S)) + T @ (beta[:, None] * (Lm @ bV)))
    O = Qb @ S + P1 @ E + P2 @ bV
    S_C = gam * S + (k * np.exp2(suf + l2)).T @ E + (k * np.exp2(suf)).T @ bV
    return O, S_C


def exact_chunk_forward(q, k, v, la, beta, S0=None, C=32, order=0, dtype=np.float32):
    """exact_chunk_step over a whole sequence (the last chunk may be partial)."""
    T, dk = q.shape
    S = np.zeros((dk, v.shape[1])) if S0 is None else np.array(S0, dtype=np.float64)
    O = np.zeros((T, v.shape[1]))
    for c0 in range(0, T, C):
        c1 = min(T, c0 + C)
        O[c0:c1], S = exact_chunk_step(q[c0:c1], k[c0:c1], v[c0:c1], la[c0:c1], beta[c0:c1], S, order, dtype)
    return O, S
