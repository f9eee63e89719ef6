"""The CPU oracle against its pins (no GPU)."""
import pytest

import oracle
import oracle_pins


@pytest.fixture(scope="module")
def lib():
    oracle.build(force=False)
    return oracle.load()


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin, lib):
    pin(lib)
