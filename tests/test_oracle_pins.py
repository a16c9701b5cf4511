"""The fp64 oracle against its pins (CPU only)."""
import pytest

import oracle.eta_oracle as E
import pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(E)
