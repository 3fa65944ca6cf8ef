"""The CPU oracle against its pins (pages' worked examples, closed forms,
invariants, library special cases, brute force).  CPU only."""
import pytest

import pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin()
