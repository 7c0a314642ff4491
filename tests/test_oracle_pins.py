"""The CPU oracle against what the PISA pages and mathematics fix (no GPU)."""
import pytest

import oracle
import oracle.metrics
import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    pin(oracle)


@pytest.mark.parametrize("pin", oracle_pins.METRIC_PINS, ids=lambda p: p.__name__)
def test_metric_pin(pin):
    pin(oracle.metrics)
