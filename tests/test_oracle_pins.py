"""The float64 oracle against facts other than itself (see oracle_checks.py)."""

import pytest

import oracle
from tests.oracle_checks import ALL_CHECKS


@pytest.mark.parametrize("check", ALL_CHECKS, ids=lambda f: f.__name__)
def test_oracle_pin(check):
    check(oracle.default())
