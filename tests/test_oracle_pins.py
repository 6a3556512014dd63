"""The fp64 oracle against its pins (CPU only); the pins themselves live in oracle_pins.py."""
import pytest

import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin_holds(pin, oracle_lib):
    pin(oracle_lib)


def test_closed_form_with_nonzero_state(oracle_lib):
    oracle_pins.pin_closed_form(oracle_lib, B=2, H=3, D=8, T=6, zero_state=False, seed=3)
