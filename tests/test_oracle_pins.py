"""The float64 oracle against facts that do not come from the oracle itself
(worked examples printed on the pages, closed forms, brute force, library
routines, invariants). CPU only."""
import pytest

import pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    pin()
