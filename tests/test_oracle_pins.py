"""The fp64 oracle against its pins (CPU only)."""
import pytest

import oracle
import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(oracle.recurrence)


@pytest.mark.parametrize("pin", oracle_pins.BWD_PINS, ids=lambda f: f.__name__)
def test_backward_pin(pin):
    pin(oracle)
