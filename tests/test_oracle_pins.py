"""The CPU oracle against its pins (closed forms, library routines, brute force,
invariants, the hand-worked golden example). No GPU needed."""
import pytest

from pins import ALL_PINS


@pytest.mark.parametrize("pin", ALL_PINS, ids=[p.__name__ for p in ALL_PINS])
def test_pin(orc, pin):
    pin(orc)
