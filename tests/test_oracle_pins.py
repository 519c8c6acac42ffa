"""The CPU oracle against its pins (library routines, finite differences,
closed forms, the contract page's worked example, invariants)."""
import pytest

import oracle
import oracle_pins


@pytest.fixture(scope="module")
def o():
    return oracle.get()


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(o, pin):
    pin(o)
