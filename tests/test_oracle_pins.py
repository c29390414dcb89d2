"""The oracle against its pins (CPU only)."""
import pytest

import oracle
from tests import oracle_pins as P


@pytest.fixture(scope="module")
def lib():
    return oracle.load()


@pytest.mark.parametrize("check", P.ALL_CHECKS, ids=lambda c: c.__name__)
def test_pin(lib, check):
    check(lib)
