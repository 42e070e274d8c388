"""The fp64 oracle against facts other than itself (CPU only)."""
import pytest

import oracle
from tests import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    pin(oracle.rat_oracle)


@pytest.mark.parametrize("pin", oracle_pins.TOPK_PINS, ids=lambda p: p.__name__)
def test_topk_pin(pin):
    pin(oracle.topk_oracle)


@pytest.mark.parametrize("pin", oracle_pins.LOCAL_PINS, ids=lambda p: p.__name__)
def test_local_pin(pin):
    pin(oracle.local_oracle)
