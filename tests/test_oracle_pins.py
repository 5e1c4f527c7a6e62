"""The float64 oracle against what the pages and the mathematics fix (CPU only)."""
import pytest

import oracle.moe_oracle as orc
import pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    pin(orc)
