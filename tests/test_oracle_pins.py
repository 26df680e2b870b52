"""The oracle against its pins (CPU only): closed forms, library routines on
dense tiny inputs, exact integer cases and identities of the definitions."""
import pytest

from oracle_pins import ALL_PINS


@pytest.mark.parametrize("pin", ALL_PINS, ids=[p.__name__ for p in ALL_PINS])
def test_oracle_pin(pin):
    pin()
