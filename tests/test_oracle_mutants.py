"""Planted mistakes in the oracle must each fail at least one independent pin.

Each mutant is the oracle's C source built with ORACLE_MUTANT=n, a one-line
change (dropped scale, h % Hkv, diagonal off by one, top-left alignment, ...).
Mutants of the backward (a dropped softmax-Jacobian term, a missing scale,
...) must each fail at least one of the backward pins.
The brute-force cross-check is left out here on purpose: the pins that are not
a second implementation of the same formula must catch every mutant alone.
"""
import pytest

import pins
from oracle import attn_oracle, build


@pytest.fixture(scope="module")
def mutant_dir(tmp_path_factory):
    return str(tmp_path_factory.mktemp("oracle_mutants"))


@pytest.mark.parametrize("n", sorted(build.MUTANTS), ids=lambda n: f"m{n}")
def test_mutant_is_caught(mutant_dir, n):
    orc = attn_oracle.load(build.build_mutant(n, mutant_dir))
    failed = []
    for pin in (pins.BWD_PINS if n in build.BWD_MUTANTS else pins.INDEPENDENT_PINS):
        try:
            pin(orc)
        except (AssertionError, attn_oracle.OracleError) as e:
            failed.append(f"{pin.__name__}: {str(e)[:80]}")
    assert failed, f"mutant {n} ({build.MUTANTS[n]}) passed every pin"
