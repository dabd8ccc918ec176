"""The CPU oracle against facts that do not come from it (see oracle_pins)."""
import pytest

import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_oracle_pin(pin, oracle_default):
    pin(oracle_default)
