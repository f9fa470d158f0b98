"""The oracle's input prologue (unit keys, logistic beta, negative-softplus
log-decay) against closed forms and identities (CPU only)."""
import math

import numpy as np
import pytest

from oracle import PROLOGUE_EPS, kda_oracle, prologue


def test_logistic_beta_closed_forms():
    x = np.array([0.0, 1.0, -1.0, 30.0, -30.0, 2.5])
    _, _, b = prologue(np.ones((6, 1, 2)), np.zeros((6, 1)), x, beta_logits=True)
    assert b[0] == 0.5
    assert abs(b[1] - 1.0 / (1.0 + math.e ** -1.0)) < 1e-15
    assert abs(b[1] + b[2] - 1.0) < 1e-15          # sigma(x) + sigma(-x) = 1
    assert abs(b[3] - 1.0) < 1e-12 and 0.0 < b[4] < 1e-12
    assert abs(math.log(b[5] / (1.0 - b[5])) - 2.5) < 1e-12  # the logit inverts it


def test_negative_softplus_closed_forms():
    x = np.array([0.0, 1.0, -1.0, 40.0, -40.0, 3.0])
    _, la, _ = prologue(np.ones((6, 1, 2)), x.reshape(6, 1), np.zeros((6, 1)), log_a_raw=True)
    la = la[:, 0]
    assert abs(la[0] + math.log(2.0)) < 1e-15
    assert abs((-la[1]) - (-la[2]) - 1.0) < 1e-14   # softplus(x) - softplus(-x) = x
    assert abs(-la[3] - 40.0) < 1e-14                 # softplus(x) -> x
    assert 0.0 > la[4] > -1e-16                       # softplus(x) -> e^x
    assert abs(math.exp(la[5]) - 1.0 / (1.0 + math.e ** 3.0)) < 1e-15  # a = sigma(-x)
    assert np.all(la <= 0.0)
    _, lac, _ = prologue(np.ones((6, 1, 2)), x.reshape(6, 1), np.zeros((6, 1)), log_a_raw=True, log_a_min=-8.0)
    assert lac[3, 0] == -8.0 and lac[0, 0] == la[0]  # the clip touches only the tail


def test_key_normalisation():
    rng = np.random.default_rng(0)
    k = rng.normal(size=(7, 3, 16)) * rng.uniform(0.5, 4.0, size=(7, 3, 1))
    kn, _, _ = prologue(k, np.zeros((7, 3)), np.zeros((7, 3)), normalize_k=True)
    norms = np.linalg.norm(kn, axis=-1)
    sq = np.sum(k * k, axis=-1)
    assert np.allclose(norms, np.sqrt(sq / (sq + PROLOGUE_EPS)), rtol=1e-14)  # unit up to eps
    cos = np.sum(kn * k, axis=-1) / (np.linalg.norm(kn, axis=-1) * np.linalg.norm(k, axis=-1))
    assert np.allclose(cos, 1.0, atol=1e-14)          # direction kept
    z, _, _ = prologue(np.zeros((2, 1, 4)), np.zeros((2, 1)), np.zeros((2, 1)), normalize_k=True)
    assert np.all(z == 0.0)                           # a zero key stays zero (eps keeps it finite)


def test_prologue_is_scale_invariant_in_k():
    """With normalised keys the layer does not see the scale of k (up to eps)."""
    rng = np.random.default_rng(1)
    T, H, dk, dv = 9, 2, 8, 4
    q, k, v = rng.normal(size=(T, H, dk)), rng.normal(size=(T, H, dk)), rng.normal(size=(T, H, dv))
    la, b = rng.normal(size=(T, H, dk)), rng.normal(size=(T, H))
    pro = dict(normalize_k=True, beta_logits=True, log_a_raw=True)
    o1, s1 = kda_oracle(q, k, v, la, b, pro=pro)
    o2, s2 = kda_oracle(q, 5.0 * k, v, la, b, pro=pro)
    assert np.max(np.abs(o1 - o2)) < 1e-6 * np.max(np.abs(o1))
    assert np.max(np.abs(s1 - s2)) < 1e-6 * np.max(np.abs(s1))


@pytest.mark.parametrize("order", [0, 1])
def test_prologue_feeds_the_recurrence(order):
    """Oracle with the prologue equals the oracle on inputs transformed in closed
    form by numpy's own logistic and log-add-exp (a different route to the same
    values)."""
    rng = np.random.default_rng(2 + order)
    T, H, dk, dv = 11, 2, 6, 5
    q, k, v = rng.normal(size=(T, H, dk)), rng.normal(size=(T, H, dk)) * 3.0, rng.normal(size=(T, H, dv))
    x, b = rng.normal(size=(T, H, dk)) * 2.0, rng.normal(size=(T, H))
    o1, s1 = kda_oracle(q, k, v, x, b, order=order,
                        pro=dict(normalize_k=True, beta_logits=True, log_a_raw=True, log_a_min=-3.0))
    kn = k / np.sqrt(np.einsum("thc,thc->th", k, k)[..., None] + PROLOGUE_EPS)
    la = np.maximum(-np.logaddexp(0.0, x), -3.0)
    bb = np.exp(-np.logaddexp(0.0, -b))
    o2, s2 = kda_oracle(q, kn, v, la, bb, order=order)
    assert np.max(np.abs(o1 - o2)) < 1e-12 and np.max(np.abs(s1 - s2)) < 1e-12


# ---- the gradient through the prologue (oracle.prologue_bwd) -----------------------
PRO_ALL = dict(normalize_k=True, beta_logits=True, log_a_raw=True, log_a_min=-2.0)


def _raw_case(seed, scalar=False, T=9, H=2, dk=4, dv=3):
    rng = np.random.default_rng(seed)
    q, v = rng.normal(size=(T, H, dk)), rng.normal(size=(T, H, dv))
    k = rng.normal(size=(T, H, dk)) * 2.0
    x = rng.normal(size=(T, H) if scalar else (T, H, dk)) * 2.0
    # keep every pre-activation away from the clip's corner at -softplus(y) = -2
    y = -np.logaddexp(0.0, x)
    x = np.where(np.abs(y + 2.0) < 1e-3, x + 0.1, x)
    z = rng.normal(size=(T, H))
    S0 = rng.normal(size=(2, H, dk, dv)) * 0.3
    dO, dST = rng.normal(size=(T, H, dv)), rng.normal(size=(2, H, dk, dv))
    return q, k, v, x, z, S0, np.array([0, 4, T]), dO, dST


def _grad_fd(case, pro, name, idx, h=1e-6):
    q, k, v, x, z, S0, cu, dO, dST = case
    args = dict(k=k, log_a=x, beta=z)

    def loss(val):
        a = {n: t.copy() for n, t in args.items()}
        a[name][idx] = val
        o, S = kda_oracle(q, a["k"], v, a["log_a"], a["beta"], S0=S0, cu_seqlens=cu, pro=pro)
        return float(np.sum(o * dO) + np.sum(S * dST))
    x0 = args[name][idx]
    return (loss(x0 + h) - loss(x0 - h)) / (2 * h)


def _check_against_fd(case, grads, pro):
    """Every raw element of k, log_a and beta against a central difference of
    the forward oracle with the prologue (its own pins are above)."""
    worst = 0.0
    for name, key in (("k", "dk"), ("log_a", "dlog_a"), ("beta", "dbeta")):
        g = grads[key]
        scale = max(np.max(np.abs(g)), 1e-3)
        for idx in np.ndindex(g.shape):
            worst = max(worst, abs(_grad_fd(case, pro, name, idx) - g[idx]) / scale)
    return worst


@pytest.mark.parametrize("scalar", [False, True])
def test_prologue_gradient_matches_finite_differences(scalar):
    from oracle import kda_oracle_bwd
    case = _raw_case(11 + scalar, scalar)
    q, k, v, x, z, S0, cu, dO, dST = case
    g = kda_oracle_bwd(q, k, v, x, z, S0=S0, cu_seqlens=cu, dO=dO, dST=dST, pro=PRO_ALL)
    y = -np.logaddexp(0.0, x)
    assert np.any(y < -2.0) and np.any(y > -2.0)      # both sides of the clip are exercised
    assert np.all(g["dlog_a"][y < -2.0] == 0.0)
    assert _check_against_fd(case, g, PRO_ALL) < 1e-6


def test_prologue_gradient_each_transform_alone():
    from oracle import kda_oracle_bwd
    case = _raw_case(13)
    q, k, v, x, z, S0, cu, dO, dST = case
    for pro in (dict(normalize_k=True), dict(beta_logits=True), dict(log_a_raw=True)):
        xx = x if pro.get("log_a_raw") else -np.abs(x) * 0.3   # a valid log a when taken as given
        zz = z if pro.get("beta_logits") else 1.0 / (1.0 + np.exp(-z))
        c = (q, k, v, xx, zz, S0, cu, dO, dST)
        g = kda_oracle_bwd(q, k, v, xx, zz, S0=S0, cu_seqlens=cu, dO=dO, dST=dST, pro=pro)
        assert _check_against_fd(c, g, pro) < 1e-6, pro


def _mutant_grads(case, which):
    """The chain rule with one planted mistake, from the oracle's gradient on the
    transformed inputs."""
    from oracle import kda_oracle_bwd
    q, k, v, x, z, S0, cu, dO, dST = case
    kt, lat, bt = prologue(k, x, z, **PRO_ALL)
    g = dict(kda_oracle_bwd(q, kt, v, lat, bt, S0=S0, cu_seqlens=cu, dO=dO, dST=dST))
    n = np.sqrt(np.sum(k * k, axis=-1, keepdims=True) + PROLOGUE_EPS)
    u, du = k / n, g["dk"]
    g["dk"] = (du - u * np.sum(u * du, axis=-1, keepdims=True)) / n
    if which == "no projection":
        g["dk"] = du / n
    b = 1.0 / (1.0 + np.exp(-z))
    g["dbeta"] = g["dbeta"] * (b if which == "beta slope" else b * (1.0 - b))
    sig = 1.0 / (1.0 + np.exp(-x))
    d = (1.0 if which == "log a sign" else -1.0) * g["dlog_a"] * sig
    y = -np.logaddexp(0.0, x)
    g["dlog_a"] = d if which == "no clip mask" else np.where(y >= -2.0, d, 0.0)
    return g


@pytest.mark.parametrize("which", ["no projection", "beta slope", "log a sign", "no clip mask"])
def test_prologue_gradient_pins_catch_planted_mistakes(which):
    case = _raw_case(17)
    assert _check_against_fd(case, _mutant_grads(case, "none"), PRO_ALL) < 1e-6
    assert _check_against_fd(case, _mutant_grads(case, which), PRO_ALL) > 1e-3
