"""Planted mistakes in the oracle must break at least one pin (CPU only).

Each mutant is a textual edit of a copy of ``oracle/kda_oracle.c`` (the real
source is never modified), compiled with gcc into a temporary directory and run
against every pin in ``tests/oracle_pins.py``.  A mutant that passes all pins
would mean the pins cannot see that class of mistake.
"""
import functools
import os

import pytest

import oracle
from tests.oracle_pins import ALL_PINS

SRC = os.path.join(os.path.dirname(oracle.__file__), "kda_oracle.c")

READ_BLOCK = """        /* read after the update: o_t = q_t S_t */
        double* ot = J->o + th * dv;
        for (int64_t j = 0; j < dv; ++j) {
            double acc = 0.0;
            for (int64_t c = 0; c < dk; ++c) acc += qt[c] * S[c * dv + j];
            ot[j] = acc;
        }
"""
BETA_LINE = "        const double b = J->beta[th];\n"
ERASE0 = "S[c * dv + j] = a[c] * (S[c * dv + j] - b * kt[c] * y[j]) + b * kt[c] * vt[j];"
DECAY = "a[c] = exp(J->scalar_decay ? J->log_a[th] : J->log_a[th * dk + c]);"
KDOT = "for (int64_t c = 0; c < dk; ++c) acc += kt[c] * S[c * dv + j];"

# name -> list of (old, new, count) edits; count = how many occurrences to replace
MUTANTS = {
    "drop_erase": [(ERASE0, "S[c * dv + j] = a[c] * (S[c * dv + j]) + b * kt[c] * vt[j];", 1)],
    "erase_sign": [(ERASE0, ERASE0.replace("- b * kt[c] * y[j]", "+ b * kt[c] * y[j]"), 1)],
    "decay_covers_write": [(ERASE0, "S[c * dv + j] = a[c] * (S[c * dv + j] - b * kt[c] * y[j] + b * kt[c] * vt[j]);", 1)],
    "decay_uniform_channel0": [(DECAY, DECAY.replace("th * dk + c]", "th * dk + 0]"), 1)],
    "decay_sign": [(DECAY, "a[c] = exp(-(J->scalar_decay ? J->log_a[th] : J->log_a[th * dk + c]));", 1)],
    "decay_base2": [(DECAY, DECAY.replace("exp(", "exp2("), 1)],
    "erase_reads_with_q": [(KDOT, KDOT.replace("kt[c]", "qt[c]"), 1)],
    "write_with_q": [(ERASE0, ERASE0.replace("+ b * kt[c] * vt[j]", "+ b * qt[c] * vt[j]"), 1)],
    "write_without_beta": [(ERASE0, ERASE0.replace("+ b * kt[c] * vt[j]", "+ kt[c] * vt[j]"), 1)],
    "ignore_S0": [("    if (J->S0)\n        memcpy", "    if (0)\n        memcpy", 1)],
    "read_with_k": [("acc += qt[c] * S[c * dv + j];", "acc += kt[c] * S[c * dv + j];", 1)],
    "read_before_update": [(READ_BLOCK, "", 1), (BETA_LINE, BETA_LINE + READ_BLOCK, 1)],
    "order1_is_order0": [("if (J->order == 0) {", "if (1) {", 1)],
    "head_index_dropped": [("const int64_t th = t * H + h;", "const int64_t th = t * H;", 1)],
    "read_uses_previous_state_row": [("acc += qt[c] * S[c * dv + j];",
                                      "acc += qt[c] * S[((c + 1) % dk) * dv + j];", 1)],
}


def _mutate(text, edits):
    for old, new, count in edits:
        assert text.count(old) >= count, f"mutation anchor not found: {old[:60]!r}"
        text = text.replace(old, new, count)
    return text


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    with open(SRC) as f:
        src = f.read()
    mutated = _mutate(src, MUTANTS[name])
    assert mutated != src
    c_path = tmp_path / f"mut_{name}.c"
    c_path.write_text(mutated)
    lib_path = str(tmp_path / f"libmut_{name}.so")
    oracle.build(str(c_path), lib_path)
    lib = oracle.load_library(lib_path)
    fn = functools.partial(oracle.kda_oracle, lib=lib)
    failed = []
    for pin in ALL_PINS:
        try:
            pin(fn)
        except Exception:  # AssertionError, or a crash-free error from the mutant
            failed.append(pin.__name__)
    assert failed, f"mutant {name} passed every pin"
