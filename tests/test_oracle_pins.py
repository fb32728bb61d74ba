"""The CPU oracle against what the EvoX virtual_noise page and the mathematics fix."""

import pytest

import pins


@pytest.mark.parametrize("check", pins.ALL_CHECKS, ids=lambda c: c.__name__)
def test_oracle_pin(check):
    check()
