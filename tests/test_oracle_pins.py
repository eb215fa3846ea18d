"""The oracle against closed forms, library routines and brute force (CPU)."""
import pytest

from oracle_pins import ALL_CHECKS


@pytest.mark.parametrize("check", ALL_CHECKS, ids=lambda f: f.__name__)
def test_pin(check):
    check()
