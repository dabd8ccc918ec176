"""The CPU oracle against facts that do not come from it (see oracle_pins and
oracle_pins_fmt)."""
import pytest

import oracle_pins
import oracle_pins_fmt


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS + oracle_pins_fmt.ALL_PINS, ids=lambda f: f.__name__)
def test_oracle_pin(pin, oracle_default):
    pin(oracle_default)
