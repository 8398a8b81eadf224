"""The fp64 oracle against its pins (closed forms, invariants, finite
differences, torch fp64 routines, hand-derived worked examples)."""

import pytest

import oracle
from oracle_pins import CHECKS


@pytest.mark.parametrize("check", CHECKS, ids=[c.__name__ for c in CHECKS])
def test_oracle_pin(check):
    check(oracle)
