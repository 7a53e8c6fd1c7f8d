"""The CPU oracle against its pins (pages' worked values, closed forms,
invariants, brute force).  CPU only."""
import pytest

import oracle as O
from oracle_pins import ALL_PINS


@pytest.fixture(scope="module")
def lib():
    return O.load()


@pytest.mark.parametrize("pin", ALL_PINS, ids=[p.__name__ for p in ALL_PINS])
def test_pin(pin, lib):
    pin(lib)
