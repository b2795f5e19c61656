"""The fp64 oracle against what the M2RNN slides and mathematics fix (CPU)."""
import pytest

import oracle
import oracle_pins


@pytest.fixture(scope="module")
def ref():
    return oracle.get()


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda p: p.__name__)
def test_pin(ref, pin):
    pin(ref)
