"""The CPU oracle against its pins (runs without a GPU)."""
import pytest

import oracle
import _pins


@pytest.mark.parametrize("check", _pins.ALL_CHECKS, ids=lambda f: f.__name__)
def test_oracle_pin(check):
    check(oracle.get())
