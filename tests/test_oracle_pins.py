"""The oracle against its pins (CPU only)."""
import os
import sys

import pytest

sys.path.insert(0, os.path.dirname(__file__))

from oracle_pins import ALL_PINS  # noqa: E402


@pytest.mark.parametrize("pin", ALL_PINS, ids=[p.__name__ for p in ALL_PINS])
def test_pin(pin):
    pin()
