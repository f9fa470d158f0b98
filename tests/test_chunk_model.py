"""The chunkwise (WY) derivation against the token-by-token oracle (CPU only).

The chunk form computes the same map as the KDA row of the table on page "The
argument, in one page" (the "Chunkwise / WY" row of that table: same update,
reorganised per chunk).  These tests check the numpy model of that
reorganisation, including its split of decay factors around 16-token
references, and the padding rule the GPU kernel relies on for ragged chunks.
"""
import numpy as np
import pytest

from oracle import kda_oracle
from tests.chunk_model import chunk_forward, chunk_forward_split


def draw(T, dk, dv, seed, la_std=2.0, clip=-8.0, scalar=False, s0=0.02):
    r = np.random.default_rng(seed)
    q = r.standard_normal((T, dk))
    k = r.standard_normal((T, dk))
    k /= np.linalg.norm(k, axis=1, keepdims=True)
    v = r.standard_normal((T, dv))
    pre = r.standard_normal((T,) if scalar else (T, dk)) * la_std
    la = np.clip(-np.logaddexp(0.0, pre), clip, 0.0)
    beta = 1.0 / (1.0 + np.exp(-r.standard_normal(T)))
    S0 = r.standard_normal((dk, dv)) * s0
    return q, k, v, la, beta, S0


def oracle_one(q, k, v, la, beta, S0):
    o, S = kda_oracle(q[:, None], k[:, None], v[:, None], la[:, None], beta[:, None],
                      S0=S0[None, None])
    return o[:, 0], S[0, 0]


def rel(x, r):
    return float(np.abs(x - r).max() / np.abs(r).max())


@pytest.mark.parametrize("T,C", [(100, 64), (100, 32), (64, 64), (17, 32), (160, 16)])
def test_chunk_form_equals_token_loop(T, C):
    q, k, v, la, beta, S0 = draw(T, 16, 8, seed=T + C)
    ro, rS = oracle_one(q, k, v, la, beta, S0)
    o, S = chunk_forward(q, k, v, la, beta, S0=S0, C=C)
    assert rel(o, ro) < 1e-10 and rel(S, rS) < 1e-10


def test_chunk_form_scalar_gate():
    q, k, v, la, beta, S0 = draw(130, 16, 16, seed=5, la_std=1.0, clip=-30.0, scalar=True)
    ro, rS = oracle_one(q, k, v, np.repeat(la[:, None], 16, axis=1), beta, S0)
    o, S = chunk_forward(q, k, v, la, beta, S0=S0, C=64)
    assert rel(o, ro) < 1e-10 and rel(S, rS) < 1e-10


def test_chunk_form_with_bf16_operands_meets_bf16_bar():
    """Operands rounded to bf16 where the kernel feeds them to the matrix cores,
    fp32-range decay factors at the stress clip of -8 per token: still within
    the 2e-2 bar for bf16 inputs."""
    q, k, v, la, beta, S0 = draw(192, 64, 32, seed=11)
    ro, rS = oracle_one(q, k, v, la, beta, S0)
    o, S = chunk_forward(q, k, v, la, beta, S0=S0, C=64, bf16=True)
    assert rel(o, ro) < 2e-2 and rel(S, rS) < 2e-2


def test_padding_rows_change_nothing():
    """A padded row that repeats the last real token's q, k, v but carries
    beta = 0 and log a = 0 leaves the state and every earlier output unchanged:
    the kernel pads ragged chunks this way instead of zeroing q, k and v."""
    T, pad = 45, 19
    q, k, v, la, beta, S0 = draw(T, 16, 8, seed=3)
    rep = lambda x: np.concatenate([x, np.repeat(x[-1:], pad, axis=0)])
    qp, kp, vp = rep(q), rep(k), rep(v)
    lap = np.concatenate([la, np.zeros((pad, 16))])
    bp = np.concatenate([beta, np.zeros(pad)])
    ro, rS = oracle_one(q, k, v, la, beta, S0)
    po, pS = oracle_one(qp, kp, vp, lap, bp, S0)
    np.testing.assert_array_equal(po[:T], ro)
    np.testing.assert_array_equal(pS, rS)
    # and the chunk model, padded the same way, agrees over a ragged last chunk
    o, S = chunk_forward(qp, kp, vp, lap, bp, S0=S0, C=32)
    assert rel(o[:T], ro) < 1e-10 and rel(S, rS) < 1e-10


@pytest.mark.parametrize("T,C", [(100, 32), (96, 64), (33, 32)])
def test_factored_operators_equal_token_loop(T, C):
    """The factored form (value-independent operators W, Q', M1, M2, Kc', Kt',
    G per chunk, then O = Q' S + M2 V, S <- G S + Kc'^T E + Kt'^T V with
    E = -(W S + M1 V)) is the same map."""
    q, k, v, la, beta, S0 = draw(T, 16, 8, seed=2 * T + C)
    ro, rS = oracle_one(q, k, v, la, beta, S0)
    o, S = chunk_forward_split(q, k, v, la, beta, S0=S0, C=C)
    assert rel(o, ro) < 1e-10 and rel(S, rS) < 1e-10


def test_factored_operators_in_bf16_meet_bf16_bar():
    q, k, v, la, beta, S0 = draw(160, 128, 32, seed=4)
    ro, rS = oracle_one(q, k, v, la, beta, S0)
    o, S = chunk_forward_split(q, k, v, la, beta, S0=S0, C=32, bf16=True)
    assert rel(o, ro) < 2e-2 and rel(S, rS) < 2e-2


@pytest.mark.parametrize("order", [0, 1])
@pytest.mark.parametrize("steep", [-9.0, -12.0, -25.0, -80.0, -1000.0])
def test_exact_path_equals_token_loop_for_steep_decay(steep, order):
    """The steep-chunk path of the kernels (one exponential of a running sum of
    consecutive log2 decays per term, float32) against the oracle, with a steep
    stretch in the middle of the sequence on two channels in three: within 1e-6,
    far inside the fp32 bar, for any decay."""
    from tests.chunk_model import exact_chunk_forward
    q, k, v, la, beta, S0 = draw(150, 24, 8, seed=int(-steep) + order, s0=0.3)
    la = la.copy()
    la[40:76, np.arange(24) % 3 != 0] = steep
    o, S = exact_chunk_forward(q, k, v, la, beta, S0, C=32, order=order)
    ro, rS = kda_oracle(q[:, None], k[:, None], v[:, None], la[:, None], beta[:, None], S0=S0[None, None],
                        order=order)
    assert rel(o, ro[:, 0]) < 1e-6 and rel(S, rS[0, 0]) < 1e-6


def test_difference_of_prefix_sums_is_what_the_exact_path_avoids():
    """Why the exponents are running sums: with a steep stretch the chunk's prefix
    sums reach thousands (log2), and a factor formed as 2^(P_t - P_i) carries
    float32 rounding of that size, far above the fp32 bar for a factor near 1."""
    r = np.random.default_rng(0)
    l2 = np.concatenate([np.full(24, -115.0), -r.random(8)]).astype(np.float32)
    P = np.cumsum(l2, dtype=np.float32)
    exact = float(np.sum(l2[27:31].astype(np.float64)))
    diff = float(P[30] - P[26])
    run = np.float32(0)
    for x in l2[27:31]:
        run = np.float32(run + x)
    assert abs(float(run) - exact) < 1e-6
    assert abs(diff - exact) > 1e-5
