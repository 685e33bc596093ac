"""The oracle against its pins (CPU only)."""

import pytest

import oracle.reference as orc
from tests import oracle_pins

PINS = oracle_pins.ALL_PINS


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    pin(orc)
