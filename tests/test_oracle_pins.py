"""The CPU oracle against brute force, torch float64 SDPA, closed forms,
invariants and hand-derived golden cases (see _pins.py)."""
import pytest

import _pins


@pytest.mark.parametrize("check", _pins.ALL_CHECKS, ids=lambda f: f.__name__)
def test_oracle_pin(check):
    check()
