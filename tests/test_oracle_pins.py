"""Every oracle pin, run on the oracle itself (CPU only)."""
import pytest

import oracle
import oracle.check
import oracle.gemm
import oracle.rne
import oracle.ternary
import oracle.errors
import oracle.w4
import oracle.w4asym
from oracle_pins import ALL_PINS


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(oracle)
