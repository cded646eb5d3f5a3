"""The CPU oracle against its pins (no GPU needed)."""
import pytest

import oracle_checks


@pytest.mark.parametrize("check", oracle_checks.ALL_CHECKS, ids=lambda f: f.__name__)
def test_oracle_pin(check):
    check()
