"""The CPU oracle against exact arithmetic, brute force, closed forms and
library attention (no GPU)."""
import pytest

import oracle_checks as oc


@pytest.mark.parametrize("check", oc.ALL_CHECKS, ids=lambda c: c.__name__)
def test_oracle_pin(check):
    check()
