"""The fp64 oracle against closed forms, hand-derived values, brute force,
split/merge and paging invariants (CPU only)."""

import pytest

import oracle
from tests.oracle_pins import ALL_CHECKS


@pytest.mark.parametrize("check", ALL_CHECKS, ids=lambda c: c.__name__)
def test_oracle_pin(check):
    check(oracle)
