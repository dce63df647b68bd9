"""The fp64 oracle against its pins (CPU only)."""
import pytest

import oracle
from tests import oracle_pins


@pytest.fixture(scope="module")
def lib():
    oracle.load()  # builds liboracle.so when missing or stale
    return oracle.oracle._LIB


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin, lib):
    pin(lib)


def test_threads_reported(lib):
    assert oracle.num_threads() >= 1
