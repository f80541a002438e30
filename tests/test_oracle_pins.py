"""The oracle against what the definition and mathematics fix (CPU only)."""
import pytest

import oracle
from tests.oracle_pins import PINS


@pytest.mark.parametrize("name", sorted(PINS))
def test_pin(name):
    PINS[name](oracle.load())
