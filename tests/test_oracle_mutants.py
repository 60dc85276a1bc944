"""Each planted mistake in the oracle (compiled with ORACLE_MUTANT=n) must be
caught by at least one pin: evidence that the pins are discriminating.
CPU only."""
import os

import pytest

import oracle
import oracle_pins


@pytest.mark.parametrize("mutant", sorted(oracle.MUTANTS), ids=lambda m: f"m{m}")
def test_mutant_is_caught(tmp_path, mutant):
    path = oracle.build(os.path.join(str(tmp_path), f"mut{mutant}.so"), mutant=mutant)
    o = oracle.Oracle(path)
    assert o.mutant == mutant
    caught = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(o)
        except (AssertionError, ValueError):
            caught.append(pin.__name__)
            break
    assert caught, f"planted mistake {mutant} ({oracle.MUTANTS[mutant]}) passed every pin"
