"""The backward chunk form (sub-chunk operators, reverse walk, recomputed start
states, factor split around per-channel references) against the oracle's
token-by-token gradient (CPU only)."""
import numpy as np
import pytest

from oracle import kda_oracle_bwd
from tests.chunk_bwd_model import chunk_backward, sub_ops


def draw(T, dk, dv, seed, la_std=2.0, clip=-8.0, scalar=False):
    r = np.random.default_rng(seed)
    q = r.standard_normal((T, dk))
    k = r.standard_normal((T, dk))
    k /= np.linalg.norm(k, axis=1, keepdims=True)
    v = r.standard_normal((T, dv))
    pre = r.standard_normal((T, 1) if scalar else (T, dk)) * la_std
    la = np.clip(-np.logaddexp(0.0, pre), clip, 0.0) * np.ones((1, dk))
    beta = 1.0 / (1.0 + np.exp(-r.standard_normal(T)))
    S0 = r.standard_normal((dk, dv)) * 0.5
    dO = r.standard_normal((T, dv))
    dST = r.standard_normal((dk, dv))
    return q, k, v, la, beta, S0, dO, dST


def oracle_one(q, k, v, la, beta, S0, dO, dST, order=0):
    g = kda_oracle_bwd(q[:, None], k[:, None], v[:, None], la[:, None], beta[:, None], S0[None, None],
                       dO=dO[:, None], dST=dST[None, None], order=order)
    return {n: (x[:, 0] if n != "dS0" else x[0, 0]) for n, x in g.items()}


def rel(a, b):
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


@pytest.mark.parametrize("T,dk,dv,seed", [(1, 4, 3, 0), (16, 8, 6, 1), (37, 8, 8, 2), (64, 16, 8, 3),
                                          (130, 16, 16, 4), (200, 8, 4, 5)])
def test_model_matches_oracle(T, dk, dv, seed):
    x = draw(T, dk, dv, seed)
    ref = oracle_one(*x)
    got = chunk_backward(*x)
    for n in ref:
        assert rel(got[n], ref[n]) < 1e-10, n


def test_model_exact_path_matches_factored():
    x = draw(100, 8, 8, 7)
    a = chunk_backward(*x, exact=False)
    b = chunk_backward(*x, exact=True)
    for n in a:
        assert rel(a[n], b[n]) < 1e-11, n


def test_model_large_spans_switch_to_exact():
    # decays of -25 per token: a 16-token sub-chunk spans 400 nats, beyond the factor split
    q, k, v, la, beta, S0, dO, dST = draw(80, 8, 8, 8)
    la = la.copy()
    la[20:40] = -25.0
    assert sub_ops(q[16:32], k[16:32], la[16:32], beta[16:32])["exact"]
    ref = oracle_one(q, k, v, la, beta, S0, dO, dST)
    got = chunk_backward(q, k, v, la, beta, S0, dO, dST)
    for n in ref:
        assert np.all(np.isfinite(got[n])), n
        assert rel(got[n], ref[n]) < 1e-9, n


def test_model_scalar_gate():
    x = draw(90, 8, 8, 9, scalar=True)
    ref = oracle_one(*x)
    got = chunk_backward(*x)
    for n in ref:
        assert rel(got[n], ref[n]) < 1e-10, n


@pytest.mark.parametrize("T,dk,dv,seed", [(1, 4, 3, 10), (16, 8, 6, 11), (37, 8, 8, 12), (130, 16, 16, 13),
                                          (200, 8, 4, 14)])
def test_model_decay_first_matches_oracle(T, dk, dv, seed):
    """The decay-first chunk form (gm replaced by g, the dlog_a rule of that
    order) against the oracle's order-1 gradient."""
    x = draw(T, dk, dv, seed)
    ref = oracle_one(*x, order=1)
    got = chunk_backward(*x, ord1=True)
    for n in ref:
        assert rel(got[n], ref[n]) < 1e-10, n
    # and the erase-first rule on the same inputs is a different gradient
    assert rel(chunk_backward(*x)["dlog_a"], ref["dlog_a"]) > 1e-3 or T == 1


def test_model_decay_first_exact_path():
    q, k, v, la, beta, S0, dO, dST = draw(80, 8, 8, 15)
    la = la.copy()
    la[20:40] = -25.0
    ref = oracle_one(q, k, v, la, beta, S0, dO, dST, order=1)
    got = chunk_backward(q, k, v, la, beta, S0, dO, dST, ord1=True)
    for n in ref:
        assert rel(got[n], ref[n]) < 1e-9, n
