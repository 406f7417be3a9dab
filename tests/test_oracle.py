"""The fp64 oracle against its pins (CPU only)."""

import pytest

import oracle
from tests import oracle_pins, oracle_pins_dropout


@pytest.mark.parametrize("check", oracle_pins.ALL_CHECKS,
                         ids=lambda c: c.__name__)
def test_oracle_pin(check):
    check(oracle.attention)


@pytest.mark.parametrize("check", oracle_pins_dropout.ALL_CHECKS,
                         ids=lambda c: c.__name__)
def test_dropout_oracle_pin(check):
    check(oracle.dropout)
