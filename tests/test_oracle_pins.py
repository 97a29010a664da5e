"""The CPU oracle against its pins (library routines, closed forms,
invariants, exact brute force).  CPU only."""
import pytest

import oracle
import pins


@pytest.fixture(scope="module")
def orc():
    return oracle.default()


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(orc, pin):
    pin(orc)
