"""The CPU oracle against what the pages and plain arithmetic fix (see pins.py)."""
import pytest

import oracle
from pins import ALL_CHECKS


@pytest.mark.parametrize("name,check", ALL_CHECKS, ids=[n for n, _ in ALL_CHECKS])
def test_oracle_pin(name, check):
    check(oracle.default())
