"""The fp64 oracle against its pins (CPU only).  The checks live in oracle_checks.py."""
import pytest

import oracle
import oracle_checks as oc


@pytest.mark.parametrize("check", oc.ALL_CHECKS, ids=lambda f: f.__name__)
def test_oracle_pin(check):
    check(oracle)
