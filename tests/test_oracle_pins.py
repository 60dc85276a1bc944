"""The oracle against its pins (hand-worked values, closed forms, library
routines, brute force, invariants).  CPU only."""
import pytest

import oracle
import oracle_pins


@pytest.fixture(scope="module")
def o():
    return oracle.load()


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda p: p.__name__)
def test_pin(o, pin):
    pin(o)
