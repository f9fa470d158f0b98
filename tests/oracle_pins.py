"""Pins for the fp64 oracle: facts fixed by the pages or by mathematics.

Each pin takes an oracle callable with the signature of ``oracle.kda_oracle`` and
raises AssertionError when the oracle disagrees.  The same pins run against the
real oracle (all must hold) and against copies of it with planted mistakes (each
mistake must break at least one pin), so a dropped term, a wrong sign, a wrong
index or a swapped operand anywhere in the recurrence is caught.

None of these re-types the oracle's loop: they use a hand-worked example, closed
forms, exact rational arithmetic, transition-matrix products, and reductions to
textbook objects (a masked matrix product, a scalar first-order recurrence).
"""
from __future__ import annotations

import json
import os
from fractions import Fraction

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _close(x, y, tol, what):
    x = np.asarray(x, dtype=np.float64)
    y = np.asarray(y, dtype=np.float64)
    assert x.shape == y.shape, f"{what}: shape {x.shape} vs {y.shape}"
    scale = max(1.0, float(np.max(np.abs(y))) if y.size else 1.0)
    err = float(np.max(np.abs(x - y))) / scale if x.size else 0.0
    assert err <= tol, f"{what}: error {err:.3e} > {tol:.1e}"


def _unit_rows(rng, n, d):
    x = rng.standard_normal((n, d))
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def _random_case(rng, T, H, dk, dv, scalar=False, n_seqs=1):
    q = rng.standard_normal((T, H, dk))
    k = _unit_rows(rng, T * H, dk).reshape(T, H, dk)
    v = rng.standard_normal((T, H, dv))
    la = -np.log1p(np.exp(rng.standard_normal((T, H) if scalar else (T, H, dk))))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((T, H))))
    S0 = 0.5 * rng.standard_normal((n_seqs, H, dk, dv))
    return q, k, v, la, beta, S0


# --- 1. hand-worked example ------------------------------------------------------
def pin_worked_example(oracle):
    """Page 'The argument, in one page', table row KDA; values worked by hand."""
    with open(os.path.join(GOLDEN, "worked_example.json")) as f:
        g = json.load(f)
    toks = g["tokens"]
    q = np.array([[t["q"]] for t in toks])
    k = np.array([[t["k"]] for t in toks])
    v = np.array([[t["v"]] for t in toks])
    beta = np.array([[t["beta"]] for t in toks])
    la = np.log(np.array([[t["a"]] for t in toks]))
    S0 = np.array(g["S0"])[None, None]
    for order, key in ((0, "order0"), (1, "order1")):
        exp = g[key]
        # whole sequence
        o, ST = oracle(q, k, v, la, beta, S0=S0, order=order)
        _close(o[:, 0, 0], [exp["o1"], exp["o2"]], 1e-13, f"{key} outputs")
        _close(ST[0, 0, :, 0], exp["S2"], 1e-13, f"{key} S2")
        # first token alone gives S1
        o1, S1 = oracle(q[:1], k[:1], v[:1], la[:1], beta[:1], S0=S0, order=order)
        _close(S1[0, 0, :, 0], exp["S1"], 1e-13, f"{key} S1")
        _close(o1[0, 0, 0], exp["o1"], 1e-13, f"{key} o1")


# --- 2. closed forms without writes ------------------------------------------------
def pin_beta_zero_closed_form(oracle):
    """beta = 0: no erase and no write, so S_t = Diag(exp(g_t)) S0 with g_t the
    running sum of log a (rows decay independently: one lifetime per row, page
    'The efficiency lineage', item 10) and o_t = (q_t * exp(g_t)) S0."""
    rng = np.random.default_rng(11)
    T, H, dk, dv = 9, 2, 5, 3
    for scalar in (False, True):
        q, k, v, la, beta, S0 = _random_case(rng, T, H, dk, dv, scalar=scalar, n_seqs=2)
        beta = np.zeros_like(beta)
        cu = np.array([0, 4, T])
        for order in (0, 1):
            o, ST = oracle(q, k, v, la, beta, S0=S0, cu_seqlens=cu, order=order)
            lae = la if not scalar else np.repeat(la[:, :, None], dk, axis=2)
            for n in range(2):
                g = np.cumsum(lae[cu[n]:cu[n + 1]], axis=0)  # [L, H, dk]
                for h in range(H):
                    want_o = (q[cu[n]:cu[n + 1], h] * np.exp(g[:, h])) @ S0[n, h]
                    _close(o[cu[n]:cu[n + 1], h], want_o, 1e-13, "beta=0 outputs")
                    _close(ST[n, h], np.exp(g[-1, h])[:, None] * S0[n, h], 1e-13, "beta=0 state")


def pin_identity_when_no_gate_no_write(oracle):
    """beta = 0 and a = 1: the state never changes and o_t = q_t S0."""
    rng = np.random.default_rng(12)
    q, k, v, la, beta, S0 = _random_case(rng, 7, 3, 4, 6)
    o, ST = oracle(q, k, v, np.zeros_like(la), np.zeros_like(beta), S0=S0)
    _close(ST, S0, 0.0, "state unchanged")
    _close(o, np.einsum("thc,hcj->thj", q, S0[0]), 1e-14, "o = q S0")


# --- 3. content-addressed recall --------------------------------------------------
def pin_orthonormal_recall(oracle):
    """a = 1, beta = 1, keys drawn (with repeats) from an orthonormal basis: each
    write erases exactly what that key held (delta-rule row of the table), so a
    query equal to a basis key reads the last value written to it, or k S0 if
    that key was never written (capacity of d orthogonal directions, same page)."""
    rng = np.random.default_rng(13)
    dk, dv, T = 6, 4, 20
    basis, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
    basis = basis.T  # rows orthonormal
    kid = rng.integers(0, dk - 1, size=T)  # key dk-1 is never written
    qid = rng.integers(0, dk, size=T)
    k = basis[kid][:, None]
    q = basis[qid][:, None]
    v = rng.standard_normal((T, 1, dv))
    S0 = rng.standard_normal((1, 1, dk, dv))
    for order in (0, 1):
        o, ST = oracle(q, k, v, np.zeros((T, 1, dk)), np.ones((T, 1)), S0=S0, order=order)
        for t in range(T):
            writes = [s for s in range(t + 1) if kid[s] == qid[t]]
            want = v[writes[-1], 0] if writes else basis[qid[t]] @ S0[0, 0]
            _close(o[t, 0], want, 1e-12, f"recall t={t}")
        for j in range(dk):
            writes = [s for s in range(T) if kid[s] == j]
            want = v[writes[-1], 0] if writes else basis[j] @ S0[0, 0]
            _close(basis[j] @ ST[0, 0], want, 1e-12, f"final recall key {j}")


# --- 4. uniform gate --------------------------------------------------------------
def pin_uniform_gate_is_gated_deltanet(oracle):
    """A per-channel gate that is equal on every channel is the scalar gate of the
    Gated DeltaNet row (KDA row vs Gated DeltaNet row of the table); with a
    uniform gate both orderings of decay and erase give the same map."""
    rng = np.random.default_rng(14)
    q, k, v, la_s, beta, S0 = _random_case(rng, 11, 2, 5, 3, scalar=True)
    la_c = np.repeat(la_s[:, :, None], 5, axis=2)
    o_s, S_s = oracle(q, k, v, la_s, beta, S0=S0)
    for order in (0, 1):
        o_c, S_c = oracle(q, k, v, la_c, beta, S0=S0, order=order)
        _close(o_c, o_s, 1e-13, "uniform per-channel vs scalar (o)")
        _close(S_c, S_s, 1e-13, "uniform per-channel vs scalar (S)")
    o_1, S_1 = oracle(q, k, v, la_s, beta, S0=S0, order=1)
    _close(o_1, o_s, 1e-13, "scalar gate, order 1 vs 0")


def pin_scalar_gate_rescales_delta_rule(oracle):
    """Scalar gate alpha_t: dividing the state by P_t = prod_{s<=t} alpha_s turns
    S_t = alpha_t (I - b k^T k) S_{t-1} + b k^T v_t into the plain delta rule
    X_t = (I - b k^T k) X_{t-1} + b k^T (v_t / P_t), with o_t = P_t q_t X_t."""
    rng = np.random.default_rng(15)
    T, dk, dv = 12, 4, 3
    q, k, v, la, beta, S0 = _random_case(rng, T, 1, dk, dv, scalar=True)
    P = np.exp(np.cumsum(la[:, 0]))
    o, ST = oracle(q, k, v, la, beta, S0=S0)
    o2, X = oracle(q, k, v / P[:, None, None], np.zeros_like(la), beta, S0=S0)
    _close(o, o2 * P[:, None, None], 1e-12, "rescaled outputs")
    _close(ST, X * P[-1], 1e-12, "rescaled state")


# --- 5. brute force: transition-matrix products and exact rationals -----------------
def pin_transition_products(oracle):
    """Tiny cases: S_T = M_T...M_1 S0 + sum_t M_T...M_{t+1} b_t k_t^T v_t, with
    M_t = Diag(a_t)(I - b_t k_t^T k_t) (order 0) or (I - b_t k_t^T k_t)Diag(a_t)
    (order 1), evaluated as explicit dk x dk matrix products."""
    rng = np.random.default_rng(16)
    for dk, dv, T in ((3, 2, 6), (4, 1, 8), (2, 3, 5)):
        q, k, v, la, beta, S0 = _random_case(rng, T, 1, dk, dv)
        for order in (0, 1):
            o, ST = oracle(q, k, v, la, beta, S0=S0, order=order)
            Ms = []
            for t in range(T):
                D = np.diag(np.exp(la[t, 0]))
                E = np.eye(dk) - beta[t, 0] * np.outer(k[t, 0], k[t, 0])
                Ms.append(D @ E if order == 0 else E @ D)
            for t in range(T):
                # state after token t from the expansion
                St = np.eye(dk)
                for s in range(t, -1, -1):
                    St = St @ Ms[s]
                St = St @ S0[0, 0]
                for s in range(t + 1):
                    Pm = np.eye(dk)
                    for r in range(t, s, -1):
                        Pm = Pm @ Ms[r]
                    St = St + Pm @ (beta[s, 0] * np.outer(k[s, 0], v[s, 0]))
                _close(o[t, 0], q[t, 0] @ St, 1e-12, f"expansion o[{t}]")
            _close(ST[0, 0], St, 1e-12, "expansion S_T")


def pin_exact_rational(oracle):
    """Exact arithmetic with Fractions on rational a, beta, k, v, q: the fp64
    oracle must agree with the exact result to a few ulps."""
    rng = np.random.default_rng(17)
    dk, dv, T = 3, 2, 5

    def rat(lo, hi, den=8):
        return Fraction(int(rng.integers(int(round(lo * den)), int(round(hi * den)) + 1)), den)

    a = [[rat(0.25, 1.0) for _ in range(dk)] for _ in range(T)]  # in [1/4, 1]
    b = [rat(0, 1) for _ in range(T)]
    k = [[rat(-1, 1) for _ in range(dk)] for _ in range(T)]
    v = [[rat(-2, 2) for _ in range(dv)] for _ in range(T)]
    q = [[rat(-1, 1) for _ in range(dk)] for _ in range(T)]
    S = [[rat(-1, 1) for _ in range(dv)] for _ in range(dk)]
    S0 = np.array([[float(x) for x in row] for row in S])[None, None]
    fl = lambda M: np.array([[float(x) for x in r] for r in M])
    for order in (0, 1):
        Se = [row[:] for row in S]
        outs = []
        for t in range(T):
            if order == 1:
                Se = [[a[t][c] * Se[c][j] for j in range(dv)] for c in range(dk)]
            y = [sum(k[t][c] * Se[c][j] for c in range(dk)) for j in range(dv)]
            Se = [[Se[c][j] - b[t] * k[t][c] * y[j] for j in range(dv)] for c in range(dk)]
            if order == 0:
                Se = [[a[t][c] * Se[c][j] for j in range(dv)] for c in range(dk)]
            Se = [[Se[c][j] + b[t] * k[t][c] * v[t][j] for j in range(dv)] for c in range(dk)]
            outs.append([sum(q[t][c] * Se[c][j] for c in range(dk)) for j in range(dv)])
        o, ST = oracle(fl(q)[:, None], fl(k)[:, None], fl(v)[:, None],
                       np.log(fl(a))[:, None], fl([b])[0][:, None], S0=S0, order=order)
        _close(o[:, 0], fl(outs), 1e-13, "exact rational outputs")
        _close(ST[0, 0], fl(Se), 1e-13, "exact rational state")


# --- 6. reductions to textbook objects -------------------------------------------
def pin_linear_attention_limit(oracle):
    """a = 1, S0 = 0 and mutually orthogonal keys: the erase term reads nothing
    (k_t S_{t-1} = 0), so the delta rule is plain linear attention (rows 'Linear
    attention' and 'Delta rule' of the table) and the outputs are the causal
    masked product o = tril(Q K^T) (beta * V)."""
    rng = np.random.default_rng(18)
    dk, dv, T = 8, 5, 8
    basis, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
    k = (basis.T * rng.uniform(0.5, 2.0, size=(T, 1)))[:, None]  # orthogonal, not unit
    q = rng.standard_normal((T, 1, dk))
    v = rng.standard_normal((T, 1, dv))
    beta = rng.uniform(0.1, 0.9, size=(T, 1))
    for order in (0, 1):
        o, ST = oracle(q, k, v, np.zeros((T, 1, dk)), beta, order=order)
        want = np.tril(q[:, 0] @ k[:, 0].T) @ (beta * v[:, 0])
        _close(o[:, 0], want, 1e-13, "linear attention outputs")
        _close(ST[0, 0], k[:, 0].T @ (beta * v[:, 0]), 1e-13, "linear attention state")


def pin_single_channel_recurrence(oracle):
    """dk = 1: the state is one row x_t (1 x dv) obeying the scalar first-order
    recurrence x_t = m_t x_{t-1} + b_t k_t v_t with m_t = a_t (1 - b_t k_t^2),
    whose solution is x_t = P_t (x_0 + sum_{s<=t} b_s k_s v_s / P_s) with P the
    cumulative product of m; o_t = q_t x_t."""
    rng = np.random.default_rng(19)
    T, dv = 15, 3
    q = rng.standard_normal((T, 1, 1))
    k = rng.uniform(-1, 1, size=(T, 1, 1))
    v = rng.standard_normal((T, 1, dv))
    la = -rng.uniform(0, 0.5, size=(T, 1, 1))
    beta = rng.uniform(0, 0.9, size=(T, 1))
    S0 = rng.standard_normal((1, 1, 1, dv))
    m = np.exp(la[:, 0, 0]) * (1 - beta[:, 0] * k[:, 0, 0] ** 2)
    P = np.cumprod(m)
    terms = (beta[:, 0] * k[:, 0, 0])[:, None] * v[:, 0] / P[:, None]
    x = P[:, None] * (S0[0, 0, 0][None, :] + np.cumsum(terms, axis=0))
    for order in (0, 1):
        o, ST = oracle(q, k, v, la, beta, S0=S0, order=order)
        _close(o[:, 0], q[:, 0] * x, 1e-12, "dk=1 outputs")
        _close(ST[0, 0, 0], x[-1], 1e-12, "dk=1 state")


# --- 7. structural properties ------------------------------------------------------
def pin_linearity(oracle):
    """For fixed q, k, a, beta the map (S0, V) -> (O, S_T) is linear."""
    rng = np.random.default_rng(20)
    q, k, v1, la, beta, S1 = _random_case(rng, 10, 2, 4, 3)
    v2 = rng.standard_normal(v1.shape)
    S2 = rng.standard_normal(S1.shape)
    c = -1.7
    oa, Sa = oracle(q, k, v1, la, beta, S0=S1)
    ob, Sb = oracle(q, k, v2, la, beta, S0=S2)
    oc, Sc = oracle(q, k, v1 + c * v2, la, beta, S0=S1 + c * S2)
    _close(oc, oa + c * ob, 1e-12, "superposition o")
    _close(Sc, Sa + c * Sb, 1e-12, "superposition S")


def pin_continuation_and_packing(oracle):
    """The state is the whole memory (glossary page 'Linear attention', 'Why it
    matters': reuse needs the state itself): running a prefix, exporting S and
    resuming from it equals one run; packed sequences equal separate runs."""
    rng = np.random.default_rng(21)
    T, H, dk, dv = 13, 2, 4, 5
    q, k, v, la, beta, S0 = _random_case(rng, T, H, dk, dv)
    o, ST = oracle(q, k, v, la, beta, S0=S0)
    for cut in (1, 5, 12):
        oa, Sa = oracle(q[:cut], k[:cut], v[:cut], la[:cut], beta[:cut], S0=S0)
        ob, Sb = oracle(q[cut:], k[cut:], v[cut:], la[cut:], beta[cut:], S0=Sa)
        _close(np.concatenate([oa, ob]), o, 1e-13, f"continuation at {cut} (o)")
        _close(Sb, ST, 1e-13, f"continuation at {cut} (S)")
    # packing: three sequences (one empty) vs separate runs
    q2, k2, v2, la2, b2, S02 = _random_case(rng, 9, H, dk, dv, n_seqs=3)
    cu = np.array([0, 4, 4, 9])
    o2, ST2 = oracle(q2, k2, v2, la2, b2, S0=S02, cu_seqlens=cu)
    for n in range(3):
        s, e = cu[n], cu[n + 1]
        on, Sn = oracle(q2[s:e], k2[s:e], v2[s:e], la2[s:e], b2[s:e], S0=S02[n:n + 1])
        _close(o2[s:e], on, 0.0, f"packed seq {n} (o)")
        _close(ST2[n], Sn[0], 0.0, f"packed seq {n} (S)")
    _close(ST2[1], S02[1], 0.0, "empty sequence keeps S0")


def pin_norm_bound(oracle):
    """Unit keys, beta in [0, 1], a in (0, 1]: (I - b k^T k) and Diag(a) are
    contractions, so ||S_t||_2 <= ||S_{t-1}||_2 + b_t ||v_t||  (sanity bound)."""
    rng = np.random.default_rng(22)
    q, k, v, la, beta, S0 = _random_case(rng, 12, 1, 4, 3)
    prev = np.linalg.norm(S0[0, 0], 2)
    for t in range(12):
        _, St = oracle(q[:t + 1], k[:t + 1], v[:t + 1], la[:t + 1], beta[:t + 1], S0=S0)
        cur = np.linalg.norm(St[0, 0], 2)
        assert cur <= prev + beta[t, 0] * np.linalg.norm(v[t, 0]) + 1e-12, "norm bound"
        prev = cur


ALL_PINS = [
    pin_worked_example,
    pin_beta_zero_closed_form,
    pin_identity_when_no_gate_no_write,
    pin_orthonormal_recall,
    pin_uniform_gate_is_gated_deltanet,
    pin_scalar_gate_rescales_delta_rule,
    pin_transition_products,
    pin_exact_rational,
    pin_linear_attention_limit,
    pin_single_channel_recurrence,
    pin_linearity,
    pin_continuation_and_packing,
    pin_norm_bound,
]
