"""The fp64 oracle against values, closed forms and independent formulas from the paper."""
import pytest

from oracle import qalg_oracle as O
from oracle_pins import ALL_PINS


@pytest.mark.parametrize("pin", ALL_PINS, ids=[p.__name__ for p in ALL_PINS])
def test_oracle_pin(pin):
    pin(O)
