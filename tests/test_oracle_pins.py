"""The oracle against its pins (format tables, a hand-worked closed form,
library special cases, independent brute force, exact invariants)."""
import pytest

import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda p: p.__name__)
def test_pin(pin, orc):
    pin(orc)
