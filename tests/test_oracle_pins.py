"""The oracle against values the pages print, closed forms and invariants."""
import pytest

import oracle
import pins


@pytest.mark.parametrize("check", pins.ALL_CHECKS, ids=lambda c: c.__name__)
def test_oracle_pin(check):
    check(oracle.default())
