"""The fp64 oracle against closed forms, invariants, finite differences, brute force and library routines."""

import pytest

import oracle
from tests import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda p: p.__name__)
def test_oracle_pin(pin):
    pin(oracle)
