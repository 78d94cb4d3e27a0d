"""The fp64 oracle checked against the page's definitions and against mathematics.

See ``oracle_pins.py`` for what each pin compares against and why it is
independent of the oracle itself.
"""
import pytest

import oracle
from oracle_pins import ALL_PINS


@pytest.fixture(scope="module")
def orc():
    return oracle.default()


@pytest.mark.parametrize("pin", ALL_PINS, ids=[p.__name__ for p in ALL_PINS])
def test_oracle_pin(orc, pin):
    pin(orc)
