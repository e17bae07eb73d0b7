"""Plant one mistake at a time in a copy of the oracle (CPU only) and check that
the pins catch every one of them. The real oracle is never modified."""
import functools

import pytest

import oracle
from tests.mutant_build import build_mutant
from tests.test_oracle_pins import PINS

# (name, text in the oracle, replacement)
MUTANTS = [
    ("erase_sign", "S[(size_t)i * dv + j] -= e * r[j];", "S[(size_t)i * dv + j] += e * r[j];"),
    ("no_erase_gate", "const double e = bt[i] * kt[i];", "const double e = kt[i];"),
    ("no_write_gate", "kt[i] * (wt[j] * vt[j])", "kt[i] * vt[j]"),
    ("write_gated_by_b", "kt[i] * (wt[j] * vt[j])", "bt[i] * kt[i] * (wt[j] * vt[j])"),
    ("no_decay", "S[(size_t)i * dv + j] *= at[i];", "S[(size_t)i * dv + j] *= 1.0;"),
    ("decay_squared", "S[(size_t)i * dv + j] *= at[i];", "S[(size_t)i * dv + j] *= at[i] * at[i];"),
    ("kread_with_query", "r[j] += S[(size_t)i * dv + j] * kt[i];", "r[j] += S[(size_t)i * dv + j] * qt[i];"),
    ("output_reads_with_key", "ot[j] += S[(size_t)i * dv + j] * qt[i];", "ot[j] += S[(size_t)i * dv + j] * kt[i];"),
    ("write_with_query", "S[(size_t)i * dv + j] += kt[i] * (wt[j] * vt[j]);",
     "S[(size_t)i * dv + j] += qt[i] * (wt[j] * vt[j]);"),
    ("gqa_interleaved", "const int G = J->Hv / J->Hqk, g = h / G;", "const int G = J->Hv / J->Hqk, g = h % J->Hqk; (void)G;"),
    ("erase_before_read_reset", "for (int j = 0; j < dv; ++j) r[j] = 0.0;", "for (int j = 0; j < dv; ++j) r[j] = 0.5;"),
]


@pytest.mark.parametrize("mut", MUTANTS, ids=lambda m: m[0])
def test_pins_catch_mutant(mut, tmp_path_factory):
    name, old, new = mut
    d = str(tmp_path_factory.mktemp("mutants"))
    lib = oracle.bind(build_mutant(name, old, new, d))
    fwd = functools.partial(oracle.forward, lib=lib)
    caught = []
    for pin in PINS:
        try:
            pin(fwd)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"mutant {name} passed every pin"
