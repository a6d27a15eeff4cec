"""The oracle against its pins (see tests/oracle_pins.py for each source)."""
import pytest

from tests import oracle_pins


@pytest.mark.parametrize("check", oracle_pins.ALL_CHECKS, ids=lambda f: f.__name__)
def test_oracle_pin(orc, check):
    check(orc)
