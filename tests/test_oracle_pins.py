"""The oracle against its pins (CPU only)."""
import pytest

from tests import oracle_pins as P


@pytest.mark.parametrize("check", P.ALL_CHECKS, ids=[c.__name__ for c in P.ALL_CHECKS])
def test_pin(check):
    check()
