"""The float64 oracle against what the pages fix (CPU only)."""
import pytest

import oracle
from oracle_pin_checks import ALL_CHECKS


@pytest.fixture(scope="module")
def orc():
    oracle.build(force=False)
    return oracle.load()


@pytest.mark.parametrize("check", ALL_CHECKS, ids=lambda f: f.__name__[len("check_"):])
def test_oracle_pin(orc, check):
    check(orc)
