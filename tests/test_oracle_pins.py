"""The CPU oracle against its pins (no GPU)."""
import os

import pytest

import oracle
import oracle_pins as pins


@pytest.fixture(scope="module")
def orc():
    oracle.build()
    return oracle.Oracle(oracle.LIBRARY)


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(orc, pin):
    pin(orc)


@pytest.mark.skipif(not os.environ.get("DT_SLOW_PINS"), reason="five-minute exhaustive sweep; set DT_SLOW_PINS=1")
def test_bf16_exhaustive(orc):
    pins.pin_bf16_exhaustive(orc)
