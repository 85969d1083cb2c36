"""The fp64 oracle against closed forms, library routines, brute force and invariants."""
import pytest

from oracle import ref
from tests import pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(ref)
