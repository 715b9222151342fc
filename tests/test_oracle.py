"""The CPU oracle checked against its pins (hand examples, library routines,
brute force, invariants).  CPU only."""
import pytest

from oracle_pins import ALL_PINS


@pytest.mark.parametrize("pin", sorted(ALL_PINS))
def test_oracle_pin(orc, pin):
    ALL_PINS[pin](orc)
