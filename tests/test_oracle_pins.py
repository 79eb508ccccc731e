"""The float64 oracle against the pins (pages' worked example, closed forms,
invariants, brute force in floating point and exact rationals)."""

import pytest

from oracle import default
from pins import ALL_PINS


@pytest.fixture(scope="module")
def orc():
    return default()


@pytest.mark.parametrize("pin", ALL_PINS, ids=[p.__name__ for p in ALL_PINS])
def test_pin(orc, pin):
    pin(orc)
