"""The CPU oracle against its pins (brute force, closed forms, invariants and
library routines); see tests/oracle_pins.py for what each check pins."""
import pytest

from tests import oracle_pins as P


@pytest.mark.parametrize("check", P.ALL_CHECKS, ids=lambda f: f.__name__)
def test_oracle_pin(check):
    check()
