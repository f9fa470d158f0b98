"""The oracle's gradient against its pins, and planted mistakes against the pins (CPU only)."""
import functools
import os

import numpy as np
import pytest

import oracle
from tests.oracle_bwd_pins import ALL_BWD_PINS

SRC = os.path.join(os.path.dirname(oracle.__file__), "kda_oracle.c")


@pytest.mark.parametrize("pin", ALL_BWD_PINS, ids=lambda p: p.__name__)
def test_oracle_bwd_pin(pin):
    pin(oracle.kda_oracle_bwd)


def test_oracle_bwd_empty_and_zero_upstream():
    rng = np.random.default_rng(0)
    T, H, dk, dv = 5, 1, 3, 2
    q, k, v = (rng.standard_normal((T, H, d)) for d in (dk, dk, dv))
    la = -np.ones((T, H, dk)); beta = np.full((T, H), 0.5)
    S0 = rng.standard_normal((2, H, dk, dv))
    g = oracle.kda_oracle_bwd(q, k, v, la, beta, S0, np.array([0, 0, T]), dO=None, dST=None)
    for name, x in g.items():
        assert np.all(x == 0.0), name
    dST = rng.standard_normal((2, H, dk, dv))
    g = oracle.kda_oracle_bwd(q, k, v, la, beta, S0, np.array([0, 0, T]), dST=dST)
    np.testing.assert_array_equal(g["dS0"][0], dST[0])   # empty sequence: S_T = S0


# Planted mistakes in the backward walk (a copy of the source is edited; the real
# file is never modified).  Each must break at least one pin.
LAMQ = "                for (int64_t j = 0; j < dv; ++j) Lam[c * dv + j] += qt[c] * dot[j];"
DQ = "                for (int64_t j = 0; j < dv; ++j) acc += dot[j] * Sc[c * dv + j];"
G0 = "                        ag += kt[c] * a[c] * Lam[c * dv + j];"
DB0 = "                    db += r[j] * vt[j] - g[j] * y[j];"
DK0 = "                    J->dk_out[th * dk + c] = b * (lv - a[c] * ly - sg);"
DL0 = "                        dl += Lam[c * dv + j] * (Sc[c * dv + j] - b * kt[c] * vt[j]);"
LAM0 = "                        Lam[c * dv + j] = a[c] * Lam[c * dv + j] - b * kt[c] * g[j];"
DP1 = "                    for (int64_t j = 0; j < dv; ++j) dP[c * dv + j] = Lam[c * dv + j] - b * kt[c] * r[j];"
LAM1 = "                    for (int64_t j = 0; j < dv; ++j) Lam[c * dv + j] = a[c] * dP[c * dv + j];"
DK1 = "                    J->dk_out[th * dk + c] = b * (lv - ly - a[c] * sr);"
DB1 = "                    db += r[j] * (vt[j] - y[j]);"
DL1 = "                        dl += dP[c * dv + j] * a[c] * Sp[c * dv + j];"
SP = "            const double* Sp = st + SZ * (size_t)(t - s);      /* S_{t-1} */"
SUM = "                    if (J->scalar_decay) dla_sum += dl;"

MUTANTS = {
    "bwd_no_read_term": [(LAMQ, "", 1)],
    "bwd_dq_previous_state": [(DQ, DQ.replace("Sc[", "Sp["), 1)],
    "bwd_g_without_decay": [(G0, "                        ag += kt[c] * Lam[c * dv + j];", 1)],
    "bwd_dbeta_sign": [(DB0, "                    db += r[j] * vt[j] + g[j] * y[j];", 1)],
    "bwd_dk_drop_decay": [(DK0, DK0.replace("a[c] * ly", "ly"), 1)],
    "bwd_dk_drop_state_term": [(DK0, DK0.replace(" - sg);", ");"), 1)],
    "bwd_dla_drop_write": [(DL0, "                        dl += Lam[c * dv + j] * Sc[c * dv + j];", 1)],
    "bwd_lam_no_decay": [(LAM0, LAM0.replace("a[c] * Lam", "Lam"), 1)],
    "bwd_lam_no_erase": [(LAM0, LAM0.replace(" - b * kt[c] * g[j]", ""), 1)],
    "bwd1_dp_no_beta": [(DP1, DP1.replace("- b * kt[c]", "- kt[c]"), 1)],
    "bwd1_lam_no_decay": [(LAM1, LAM1.replace("a[c] * dP", "dP"), 1)],
    "bwd1_dk_drop_decay": [(DK1, DK1.replace("a[c] * sr", "sr"), 1)],
    "bwd1_dbeta_drop_read": [(DB1, "                    db += r[j] * vt[j];", 1)],
    "bwd1_dla_undecayed": [(DL1, DL1.replace("a[c] * Sp", "Sp"), 1)],
    "bwd_replay_off_by_one": [(SP, SP.replace("(t - s)", "(t - s + 1)"), 1)],
    "bwd_scalar_gate_last_channel": [(SUM, "                    if (J->scalar_decay) dla_sum = dl;", 2)],
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_bwd_mutant_is_caught(name, tmp_path):
    with open(SRC) as f:
        src = f.read()
    text = src
    for old, new, count in MUTANTS[name]:
        assert text.count(old) >= count, f"mutation anchor not found: {old[:60]!r}"
        text = text.replace(old, new, count)
    assert text != src
    c_path = tmp_path / f"mut_{name}.c"
    c_path.write_text(text)
    lib_path = str(tmp_path / f"libmut_{name}.so")
    oracle.build(str(c_path), lib_path)
    lib = oracle.load_library(lib_path)
    fn = functools.partial(oracle.kda_oracle_bwd, lib=lib)
    failed = []
    for pin in ALL_BWD_PINS:
        try:
            pin(fn)
        except Exception:
            failed.append(pin.__name__)
    assert failed, f"mutant {name} passed every pin"
