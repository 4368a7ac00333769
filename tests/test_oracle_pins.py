"""The fp64 reference against its pins (CPU only)."""
import pytest

import oracle
import pins


@pytest.fixture(scope="module")
def orc():
    oracle.build(force=False)
    return oracle.Oracle()


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(orc, pin):
    pin(orc)
