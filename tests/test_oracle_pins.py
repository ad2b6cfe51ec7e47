"""The CPU oracle against what the LoSA pages and the mathematics fix (no GPU)."""
import pytest

import oracle
import oracle_pins as P


@pytest.fixture(scope="module")
def lib():
    return oracle.load()


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(lib, pin):
    pin(lib)
